"""Parity at the full sizes the benchmark and the configurations name, through the C
ABI: the headline shape (B=64, k=5, V=129280, bf16, Markov rank 256) over 30 steps per
verifier (more than 10^4 decisions, so the near-decision budget of 10^-4 is enforced
without a floor), the headline shape without the Markov head, the over-long drafts
(B=64, k=9) over 5 steps, and the adaptive ragged configuration at its full B=256:
confidence head -> per-stream counts -> ragged block verification, and confidence
head -> batch scheduler -> ragged block verification; and the drafter's walk at the
headline shape (the resident launch) over 4 steps."""
import numpy as np
import pytest
import torch

import workloads
from oracle import dspark as odsp
from oracle import schedule as osch
from tests import harness as H
from tests.oracle_pool import oracle_steps, walk_steps

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mod():
    import draft_block_verification_row_amd as m
    m.lib()
    return m


def _run_steps(mod, name, method, steps, label):
    """Every step on the device first, then the oracle's steps in worker processes."""
    wl = workloads.make(name)
    dev = H.to_dev(wl)
    steps = list(steps)
    print(f"[{label} {method}] B={wl.B} k={wl.k} V={wl.V} steps={len(steps)}", flush=True)
    gs = [H.run_gpu(mod, dev, method, wl.seed, s) for s in steps]
    del dev
    os_ = oracle_steps(name, method, steps)
    t = H.Tally()
    for s, g, o in zip(steps, gs, os_):
        H.compare(g, o, wl, method, t, label=f"{label}/step{s}")
    print(f"[{label} {method}] {t.summary()}", flush=True)
    H.assert_clean(t)
    return t


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_headline_thirty_steps(mod, method):
    t = _run_steps(mod, "h", method, range(30), "h30")
    assert t.decisions > 10000


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_headline_without_markov(mod, method):
    _run_steps(mod, "h_nomarkov", method, range(8), "h-nomarkov")


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_overlong_drafts_five_steps(mod, method):
    _run_steps(mod, "c4", method, range(5), "c4")


def _c5_devices(wl):
    hid = torch.from_numpy(wl.hidden.view(np.int16)).cuda()
    w = torch.from_numpy(wl.conf_w.view(np.int16)).cuda()
    return hid, w


def test_adaptive_ragged_full_batch(mod):
    """B=256: confidence head and per-stream adaptive counts on the device, then ragged
    block verification over those counts with no host round trip."""
    wl = workloads.make("c5")
    assert wl.B == 256
    dev = H.to_dev(wl)
    hid, w = _c5_devices(wl)
    n, c, a = mod.adaptive_k(hid, w, wl.conf_b, wl.verify_ms)
    dev["num_drafts"] = n
    g = H.run_gpu(mod, dev, "block", wl.seed, 0)
    ref = odsp.adaptive_k(wl.hidden, wl.conf_w, wl.conf_b, wl.verify_ms)
    assert np.allclose(c.cpu().numpy(), ref["c"], rtol=1e-5, atol=0)
    assert np.allclose(a.cpu().numpy(), ref["a"], rtol=1e-5, atol=0)
    n_g = n.cpu().numpy()
    near = ref["margin"] < H.NEAR
    assert np.array_equal(n_g[~near], ref["n"][~near])
    wl.num_drafts = n_g
    o = H.run_oracle(wl, "block", 0)
    t = H.Tally()
    H.compare(g, o, wl, "block", t, label="c5-adaptive")
    print(f"[c5 adaptive B=256] n histogram {np.bincount(n_g, minlength=6).tolist()} "
          f"near choices {int(near.sum())} {t.summary()}", flush=True)
    H.assert_clean(t)


def test_scheduled_ragged_full_batch(mod):
    """B=256: confidence head -> batch-level scheduler over the table 10 + 2.4 t ->
    ragged block verification."""
    wl = workloads.make("c5")
    dev = H.to_dev(wl)
    hid, w = _c5_devices(wl)
    _, c, _ = mod.adaptive_k(hid, w, wl.conf_b, wl.verify_ms)
    ms = (100.0 + 0.1 * np.arange(wl.B * (wl.k + 1) + 1)).astype(np.float32)   # most drafts pay
    n, total, _ = mod.schedule_batch(c, torch.from_numpy(ms).cuda())
    dev["num_drafts"] = n
    g = H.run_gpu(mod, dev, "block", wl.seed, 1)
    ref = osch.batch_schedule(c.cpu().numpy(), ms)
    n_g = n.cpu().numpy()
    exact = ref["margin"] >= 1e-12 and not 0.0 < ref["cut_gap"] <= 2.0 ** -40
    if exact:
        assert np.array_equal(n_g, ref["n"])
    wl.num_drafts = n_g
    o = H.run_oracle(wl, "block", 1)
    t = H.Tally()
    H.compare(g, o, wl, "block", t, label="c5-scheduled")
    print(f"[c5 scheduled B=256] m={ref['m']} total={int(total.item())} "
          f"n histogram {np.bincount(n_g, minlength=6).tolist()} {t.summary()}", flush=True)
    H.assert_clean(t)


def test_walk_headline_shape(mod):
    """The drafter's Markov walk at B=64, k=5, V=129280, bf16, rank 256 (one resident
    launch for the five slots): tokens bit-exact except on streams whose smallest race
    margin in the oracle is below the near-decision threshold; log q within tolerance."""
    wl = workloads.make("h")
    dev = H.to_dev(wl)
    assert mod.draft_launches(dev["draft"], temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"],
                              anchor=dev["anchor"]) == 2
    steps = range(4)
    got = []
    for s in steps:
        toks, lq = mod.draft_sample(dev["draft"], temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"],
                                    anchor=dev["anchor"], seed=wl.seed, step=s, logq=True)
        torch.cuda.synchronize()
        got.append((toks.cpu().numpy(), lq.cpu().numpy()))
    del dev
    draws = near = 0
    worst = 0.0
    for s, (g_t, g_lq), o in zip(steps, got, walk_steps("h", steps)):
        for b in range(wl.B):
            draws += wl.k
            if o["margin"][b] < H.NEAR:
                near += 1
                continue
            assert np.array_equal(g_t[b], o["tokens"][b]), (s, b, g_t[b], o["tokens"][b])
            err = float(np.max(np.abs(g_lq[b] - o["logq"][b])))
            worst = max(worst, err)
            assert err <= H.TOL_LOGPROB, (s, b, g_lq[b], o["logq"][b])
    print(f"[walk-h] draws={draws} near_streams={near} max|dlogq|={worst:.2e}", flush=True)
    assert near <= max(1, int(1e-4 * draws))
