"""The allocation-free verify entry point (static per-device scratch) against the
workspace entry points, through the C ABI: identical outputs on two calls in a row,
the second with a smaller problem, for both verifiers; oversized problems and an
unknown method are refused before anything is enqueued."""
import ctypes

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


def _call_pair(mod, wl, method, step):
    dev = H.to_dev(wl)
    kw = dict(num_drafts=dev["num_drafts"], temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"],
              anchor=dev["anchor"], seed=wl.seed, step=step, diag=True)
    fn = mod.verify_block if method == "block" else mod.verify_tokenwise
    ref = fn(dev["target"], dev["draft"], dev["draft_tokens"], **kw)
    got = mod.verify_noalloc(method, dev["target"], dev["draft"], dev["draft_tokens"], **kw)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in ref], [t.cpu().numpy() for t in got]


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_noalloc_matches_workspace_entry_point(mod, method):
    big = workloads.make("c3", B=16)                    # B=16, k=5, V=129280, Markov on
    small = workloads.make_zipf("na-small", seed=21, B=3, k=4, V=1000, dtype="f32", R=64, sigma=1.5,
                                rho=(0.6, 0.99), greedy_every=3)
    small.num_drafts = np.array([4, 0, 2], dtype=np.int32)
    for wl, step in ((big, 3), (small, 4)):            # second call smaller than the first
        ref, got = _call_pair(mod, wl, method, step)
        print(f"[noalloc {method}] B={wl.B} k={wl.k} V={wl.V} accepted={got[0].tolist()}", flush=True)
        assert np.array_equal(ref[0], got[0])
        assert np.array_equal(ref[1], got[1])
        assert np.array_equal(np.nan_to_num(ref[2], nan=-7.0), np.nan_to_num(got[2], nan=-7.0))


def test_noalloc_refuses_oversized_and_unknown_method(mod):
    L = mod.lib()
    p = mod.VerifyProblem(B=4096, k=32, V=129280, dtype=1, target_logits=256, draft_logits=256, draft_tokens=256)
    o = mod.VerifyOutputs(accepted_len=256, out_tokens=256)
    assert L.dspark_workspace_bytes(ctypes.byref(p)) > mod.NOALLOC_SCRATCH_BYTES
    assert L.dspark_verify_noalloc(ctypes.byref(p), ctypes.byref(o), 1, None) == 6
    assert L.dspark_verify_noalloc(ctypes.byref(p), ctypes.byref(o), 2, None) == 1
