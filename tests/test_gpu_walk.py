"""The drafter's Markov walk on the HIP path vs the oracle, through the C ABI.

Tokens must match bit for bit, except on streams where the oracle's smallest
decision margin is below 1e-6 (counted, at most max(1, 1e-4 of the draws)).
log q_j(x_j) matches within 1e-5 where the tokens do.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dspark as odsp
from tests import harness as H
from tests.test_gpu_parity import mod  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


def _walk_both(mod, wl, step):
    dev = H.to_dev(wl)
    toks, lq = mod.draft_sample(dev["draft"], num_drafts=dev["num_drafts"], temperature=dev["temperature"],
                                W1=dev["W1"], W2t=dev["W2t"], anchor=dev["anchor"], seed=wl.seed, step=step,
                                logq=True)
    torch.cuda.synchronize()
    o = odsp.draft_walk(wl.draft, wl.dtype, wl.temperature, wl.anchor, wl.W1, wl.W2t, num_drafts=wl.num_drafts,
                        seed=wl.seed, step=step)
    return toks.cpu().numpy(), lq.cpu().numpy(), o


def _check(mod, wl, steps, label):
    draws = near = 0
    worst = 0.0
    for step in steps:
        g_t, g_lq, o = _walk_both(mod, wl, step)
        gam = np.full(wl.B, wl.k) if wl.num_drafts is None else np.asarray(wl.num_drafts)
        for b in range(wl.B):
            draws += int(gam[b])
            if o["margin"][b] < H.NEAR:
                near += 1
                continue
            assert np.array_equal(g_t[b], o["tokens"][b]), (label, step, b, g_t[b], o["tokens"][b])
            for j in range(int(gam[b])):
                if np.isnan(o["logq"][b, j]):
                    assert np.isnan(g_lq[b, j])
                else:
                    err = abs(g_lq[b, j] - o["logq"][b, j])
                    worst = max(worst, err)
                    assert err <= H.TOL_LOGPROB, (label, step, b, j, g_lq[b, j], o["logq"][b, j])
    print(f"[{label}] draws={draws} near_streams={near} max|dlogq|={worst:.2e}", flush=True)
    assert near <= max(1, int(1e-4 * draws))


SHAPES = [
    # (V, dtype, R, markov)
    (1000, "bf16", 256, True),
    (333, "bf16", 64, True),
    (4099, "f32", 128, True),
    (777, "f32", 256, False),
    (200000, "bf16", 32, True),   # more than 512 groups
]


@pytest.mark.parametrize("V,dtype,R,markov", SHAPES)
def test_walk_small_shapes(mod, V, dtype, R, markov):
    wl = workloads.make_zipf(f"walk{V}", seed=V + 3, B=6, k=5, V=V, dtype=dtype, R=R, markov=markov, sigma=1.5)
    _check(mod, wl, range(10), f"walk-V{V}-{dtype}-R{R}")


def test_walk_mixed_greedy_and_ragged(mod):
    wl = workloads.make_zipf("walk-mixed", seed=21, B=8, k=5, V=1500, dtype="bf16", sigma=1.5, greedy_every=3)
    wl.num_drafts = np.array([5, 0, 3, 5, 1, 4, 2, 5], dtype=np.int32)
    _check(mod, wl, range(6), "walk-mixed")


def test_walk_full_vocab(mod):
    wl = workloads.make_zipf("walk-full", seed=64, B=16, k=5, dtype="bf16")
    _check(mod, wl, range(2), "walk-full")


def test_walk_then_verify(mod):
    """Drafts drawn on the GPU go straight into the verify call; the same pipeline on
    the oracle gives the same drafts, accepted lengths and tokens."""
    wl = workloads.make_zipf("walk-verify", seed=31, B=8, k=5, V=3000, dtype="bf16", sigma=1.5,
                             rho=(0.8, 0.99))
    dev = H.to_dev(wl)
    toks, _ = mod.draft_sample(dev["draft"], temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"],
                               anchor=dev["anchor"], seed=wl.seed, step=3)
    o = odsp.draft_walk(wl.draft, wl.dtype, wl.temperature, wl.anchor, wl.W1, wl.W2t, seed=wl.seed, step=3)
    ok = o["margin"] >= H.NEAR
    assert np.array_equal(toks.cpu().numpy()[ok], o["tokens"][ok])
    wl.draft_tokens = o["tokens"]
    dev["draft_tokens"] = toks
    t = H.Tally()
    for method in ("tokenwise", "block"):
        g = H.run_gpu(mod, dev, method, wl.seed, 3)
        r = H.run_oracle(wl, method, 3)
        H.compare({k: v[ok] if v is not None else None for k, v in g.items()},
                  {k: (v[ok] if isinstance(v, np.ndarray) else v) for k, v in r.items()},
                  _subset(wl, ok), method, t, label=f"walk-verify/{method}")
    H.assert_clean(t)


def _subset(wl, ok):
    import dataclasses
    return dataclasses.replace(wl, B=int(ok.sum()), temperature=wl.temperature[ok],
                               num_drafts=None if wl.num_drafts is None else wl.num_drafts[ok])


PLAN_CASES = [
    # (B, k, V, dtype, R (0: no Markov head), greedy_every, ragged counts)
    (64, 5, 129280, "bf16", 256, 0, False),   # the headline shape
    (100, 4, 50000, "bf16", 128, 7, True),    # two blocks of streams, mixed greedy, ragged counts
    (6, 5, 1000, "bf16", 256, 0, False),      # fewer groups than streams
    (9, 3, 4099, "f32", 64, 4, True),         # rows not 16-byte aligned
    (16, 5, 3000, "f32", 0, 0, False),        # no Markov head
]


def _plan_inputs(B, k, V, dtype, R, greedy_every, ragged, seed):
    g = torch.Generator().manual_seed(seed)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kw = dict(draft=(torch.randn(B, k, V, generator=g) * 3.0).to(tdt).to(dev))
    T = torch.rand(B, generator=g) * 0.4 + 0.6
    if greedy_every:
        T[::greedy_every] = 0.0
    kw["temperature"] = T.to(dev)
    kw["anchor"] = torch.randint(0, V, (B,), generator=g, dtype=torch.int32).to(dev)
    if R:
        kw["W1"] = (torch.randn(V, R, generator=g) * 0.02).to(torch.bfloat16).to(dev)
        kw["W2t"] = (torch.randn(V, R, generator=g) * 0.02).to(torch.bfloat16).to(dev)
    if ragged:
        kw["num_drafts"] = torch.randint(0, k + 1, (B,), generator=g, dtype=torch.int32).to(dev)
    return kw


@pytest.mark.parametrize("B,k,V,dtype,R,greedy_every,ragged", PLAN_CASES)
def test_walk_launch_plans_agree(mod, monkeypatch, B, k, V, dtype, R, greedy_every, ragged):
    """The resident walk (one launch for every slot) and the two launches per slot give
    the same tokens and log q, bit for bit, on two steps."""
    kw = _plan_inputs(B, k, V, dtype, R, greedy_every, ragged, seed=B * 1000 + V)
    plan_kw = {n: kw[n] for n in ("num_drafts", "temperature", "W1", "W2t", "anchor") if n in kw}
    for step in (0, 7):
        got = {}
        for plan in ("resident", "separate"):
            if plan == "separate":
                monkeypatch.setenv("DSPARK_WALK_LAUNCH", "separate")
            else:
                monkeypatch.delenv("DSPARK_WALK_LAUNCH", raising=False)
            n = mod.draft_launches(kw["draft"], **plan_kw)
            toks, lq = mod.draft_sample(seed=11, step=step, logq=True, **kw)
            torch.cuda.synchronize()
            got[plan] = (n, toks.cpu(), lq.cpu())
        # without log q the partials skip their sums: the draws must not change (either plan)
        for plan in ("separate", "resident"):
            if plan == "resident":
                monkeypatch.delenv("DSPARK_WALK_LAUNCH", raising=False)
            toks_nolq, none = mod.draft_sample(seed=11, step=step, logq=False, **kw)
            torch.cuda.synchronize()
            assert none is None and torch.equal(toks_nolq.cpu(), got[plan][1]), (plan, step)
        assert got["resident"][0] == 2, got["resident"][0]
        assert got["separate"][0] == 2 * k
        assert torch.equal(got["resident"][1], got["separate"][1]), (step, got["resident"][1], got["separate"][1])
        torch.testing.assert_close(got["resident"][2], got["separate"][2], rtol=0, atol=0, equal_nan=True)
        gam = kw["num_drafts"].cpu() if "num_drafts" in kw else torch.full((B,), k)
        drawn = got["resident"][1]
        for b in range(B):
            assert bool((drawn[b, :int(gam[b])] >= 0).all()) and bool((drawn[b, int(gam[b]):] == -1).all())
        print(f"[walk-plans B={B} k={k} V={V} {dtype} R={R}] step {step}: identical", flush=True)
