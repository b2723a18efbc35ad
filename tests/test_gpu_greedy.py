"""Greedy branch (temperature 0) on the HIP path vs the oracle, through the C ABI.

Mixed batches (greedy and sampled streams side by side), every logit dtype, the
full vocabulary, ragged draft counts, and rows with equal maxima inside one
256-id group and across groups.  Greedy decisions are exact comparisons, so
accepted lengths and tokens must match bit for bit.
"""
import numpy as np
import pytest

import workloads
from tests import harness as H
from tests.test_gpu_parity import _run, mod  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V,dtype", [(1000, "bf16"), (3001, "f32")])
@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_mixed_batch_small(mod, method, V, dtype):
    wl = workloads.make_zipf(f"greedy{V}", seed=V, B=8, k=5, V=V, dtype=dtype, sigma=1.5, rho=(0.6, 0.99),
                             greedy_every=2)
    t = _run(mod, wl, method, range(10), f"greedy-V{V}-{dtype}")
    assert t.streams == 80


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_mixed_batch_full_vocab(mod, method):
    wl = workloads.make_zipf("greedy-full", seed=77, B=8, k=5, dtype="bf16", greedy_every=2)
    _run(mod, wl, method, range(2), "greedy-full")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_mixed_batch_ragged(mod, method):
    wl = workloads.make_zipf("greedy-ragged", seed=5, B=8, k=5, V=2000, dtype="bf16", sigma=1.5,
                             rho=(0.6, 0.99), greedy_every=2)
    wl.num_drafts = np.array([0, 1, 5, 3, 2, 0, 4, 5], dtype=np.int32)
    _run(mod, wl, method, range(5), "greedy-ragged")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_equal_maxima(mod, method):
    """Each greedy target row gets copies of its maximum at a lower id in the same
    256-id group and in an earlier group; drafts name either the first copy (kept)
    or the original position (rejected: the first id wins)."""
    V = 1500
    wl = workloads.make_zipf("greedy-ties", seed=9, B=6, k=4, V=V, dtype="bf16", sigma=1.5, rho=(0.6, 0.99),
                             greedy_every=1)
    rng = np.random.default_rng(9)
    tgt = wl.target
    for b in range(wl.B):
        for j in range(wl.k + 1):
            row = workloads.bf16_bits_to_f32(tgt[b, j])
            top = int(np.argmax(row))
            if top < 300:                       # move the maximum up so lower copies fit
                tgt[b, j, top + 600] = tgt[b, j, top]
                top += 600
            same_group = (top // 256) * 256 + int(rng.integers(0, top % 256 + 1))
            earlier = int(rng.integers(0, (top // 256) * 256)) if top >= 256 else same_group
            for v in {same_group, earlier}:
                tgt[b, j, v] = tgt[b, j, top]
            first = min(same_group, earlier, top)
            if j < wl.k:
                wl.draft_tokens[b, j] = first if rng.random() < 0.7 else top
    _run(mod, wl, method, range(2), "greedy-ties")
