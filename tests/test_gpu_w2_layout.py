"""W2 in the pages' [R, V] layout: the one-launch transpose into the [V, R] layout the
verify problem takes is a bit-exact copy, and a verify call on its output equals one on
the host-transposed factor."""
import numpy as np
import pytest
import torch

import workloads
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mod():
    import draft_block_verification_row_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("R,V", [(256, 129280), (32, 333), (64, 1), (1, 70), (200, 65)])
def test_transpose_is_a_copy(mod, R, V):
    g = torch.Generator().manual_seed(R * 1000 + V)
    W2 = torch.randint(-32768, 32767, (R, V), dtype=torch.int16, generator=g).cuda()
    W2t = mod.w2_transpose(W2)
    torch.cuda.synchronize()
    assert torch.equal(W2t.cpu(), W2.cpu().t().contiguous())


def test_transpose_refuses_in_place(mod):
    W2 = torch.zeros(64, 64, dtype=torch.int16, device="cuda")
    with pytest.raises(RuntimeError):
        mod.w2_transpose(W2, out=W2.view(64, 64))


def test_verify_on_transposed_factor(mod):
    wl = workloads.make("h", V=4099, B=4)
    dev = H.to_dev(wl)
    W2 = torch.from_numpy(np.ascontiguousarray(wl.W2t.T).view(np.int16)).cuda()   # [R, V]
    dev2 = dict(dev, W2t=mod.w2_transpose(W2))
    for method in ("tokenwise", "block"):
        a = H.run_gpu(mod, dev, method, wl.seed, 3)
        b = H.run_gpu(mod, dev2, method, wl.seed, 3)
        assert np.array_equal(a["accepted_len"], b["accepted_len"])
        assert np.array_equal(a["out_tokens"], b["out_tokens"])
        assert np.array_equal(a["diag"], b["diag"], equal_nan=True)
