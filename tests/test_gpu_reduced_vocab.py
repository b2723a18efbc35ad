"""Reduced draft vocabulary on the HIP path vs the oracle, through the C ABI.

The drafter scores K of the V ids; its logits are scattered into the target's
columns with -inf elsewhere (q = 0 there).  The verifiers must keep the target's
mass on those columns in the residual; the walk must never propose them.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import harness as H
from tests.test_gpu_parity import _run, mod  # noqa: F401  (module fixture)
from tests.test_gpu_walk import _check as _check_walk

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V,dtype,K", [(1000, "bf16", 300), (3001, "f32", 500)])
@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_verify_reduced_vocab_small(mod, method, V, dtype, K):
    wl = workloads.make_zipf(f"rv{V}", seed=V + K, B=6, k=5, V=V, dtype=dtype, sigma=1.5, rho=(0.6, 0.99),
                             draft_vocab=K)
    _run(mod, wl, method, range(10), f"reduced-V{V}-K{K}")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_verify_reduced_vocab_full(mod, method):
    wl = workloads.make_zipf("rv-full", seed=12, B=8, k=5, dtype="bf16", draft_vocab=32768)
    _run(mod, wl, method, range(2), "reduced-full")


def test_walk_reduced_vocab(mod):
    wl = workloads.make_zipf("rv-walk", seed=13, B=6, k=5, V=2000, dtype="bf16", sigma=1.5, draft_vocab=400)
    _check_walk(mod, wl, range(6), "walk-reduced")
    dev = H.to_dev(wl)
    toks, _ = mod.draft_sample(dev["draft"], temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"],
                               anchor=dev["anchor"], seed=1, step=0)
    assert np.all(np.isin(toks.cpu().numpy(), wl.meta["draft_vocab"]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scatter_matches_the_definition(mod, dtype):
    rng = np.random.default_rng(3)
    rows, K, V = 10, 257, 1900
    ids = np.sort(rng.choice(V, size=K, replace=False)).astype(np.int32)
    red = rng.standard_normal((rows, K)).astype(np.float32)
    if dtype == "bf16":
        red_bits = workloads.f32_to_bf16_bits(red)
        t_red = torch.from_numpy(red_bits.view(np.int16)).cuda()
        want = np.full((rows, V), 0xFF80, dtype=np.uint16)
        want[:, ids] = red_bits
    else:
        t_red = torch.from_numpy(red).cuda()
        want = np.full((rows, V), -np.inf, dtype=np.float32)
        want[:, ids] = red
    out = mod.draft_scatter(t_red, torch.from_numpy(ids).cuda(), V)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if dtype == "bf16":
        got = got.view(np.uint16)
    assert np.array_equal(got, want)
