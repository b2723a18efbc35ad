"""Batch-level scheduler and online cost table on the HIP path vs the oracle.

The oracle computes the scheduler's definition in fp64 (survivals multiplied left
to right, E(m) summed in rank order); the kernel ranks survivals rounded to
multiples of 2^-40 and sums them exactly as integers.  Comparison rule: the
draft counts n and the total B + m are bit-exact, except where the oracle's
ratio margin (best - runner-up) / best is below 1e-12 (then nothing is compared)
or where the survivals on either side of the cut differ by less than 2^-40 (then
only the total is compared: which stream takes the last draft is below the
kernel's resolution); those cases are counted and printed.  E(m) is within 1e-12
relative.  The cost table is fed by HIP event pairs around real verify calls;
its served table must equal the oracle's table rebuilt from the same filed
observations.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import dspark as odsp
from oracle import schedule as osch
from tests import harness as H
from tests.test_gpu_parity import mod  # noqa: F401  (module fixture)

pytestmark = pytest.mark.gpu


def _table(kind, B, k, rng):
    t = np.arange(B * (k + 1) + 1, dtype=np.float64)
    if kind == "linear":            # 10 + 2.4 t
        ms = 10.0 + 2.4 * t
    elif kind == "shallow":         # a fixed cost dominates: most drafts pay
        ms = 100.0 + 0.1 * t
    elif kind == "knee":            # flat up to 2B tokens, then steep
        ms = 20.0 + 0.5 * np.maximum(0.0, t - 2 * B)
    else:                           # arbitrary positive table
        ms = rng.uniform(1.0, 50.0, size=t.shape)
    return ms.astype(np.float32)


RATIO_NEAR = 1e-12          # the oracle's ratio margin below which no count is compared
KERNEL_RESOLUTION = 2.0 ** -40   # the kernel ranks survivals in these units


def _check(mod, c, ms, label):
    n, total, expected = mod.schedule_batch(torch.from_numpy(c).cuda(), torch.from_numpy(ms).cuda())
    torch.cuda.synchronize()
    ref = osch.batch_schedule(c, ms)
    n_g = n.cpu().numpy()
    B = c.shape[0]
    near_ratio = ref["margin"] < RATIO_NEAR
    near_cut = 0.0 < ref["cut_gap"] <= KERNEL_RESOLUTION
    print(f"[{label}] B={B} k={c.shape[1]} m={ref['m']} gpu_total={int(total.item())} "
          f"ratio_margin={ref['margin']:.3g} cut_gap={ref['cut_gap']:.3g} "
          f"near_ratio={near_ratio} near_cut={near_cut}", flush=True)
    if near_ratio:
        return ref
    assert int(total.item()) == B + ref["m"], label
    assert abs(float(expected.item()) - ref["expected"]) <= 1e-12 * ref["expected"], label
    if near_cut:
        assert int(n_g.sum()) == ref["m"], label
    else:
        assert np.array_equal(n_g, ref["n"]), label
    return ref


SHAPES = [(1, 1), (1, 4), (3, 3), (16, 5), (64, 5), (256, 5), (100, 7), (512, 8), (4096, 1), (1, 32)]


@pytest.mark.parametrize("B,k", SHAPES)
@pytest.mark.parametrize("kind", ["linear", "shallow", "knee", "random"])
def test_schedule_matches_oracle(mod, B, k, kind):
    rng = np.random.Generator(np.random.PCG64(1000 * B + k))
    c = rng.uniform(0.3, 0.99, size=(B, k)).astype(np.float32)
    _check(mod, c, _table(kind, B, k, rng), f"sched-{kind}")


@pytest.mark.parametrize("B,k", [(64, 5), (33, 4)])
def test_schedule_ties_and_extremes(mod, B, k):
    """Whole streams at c = 1 (equal survivals along a stream and across streams),
    zeros that end a stream's survival, and duplicated rows."""
    rng = np.random.Generator(np.random.PCG64(7 + B))
    c = rng.uniform(0.3, 0.99, size=(B, k)).astype(np.float32)
    c[::4, :] = 1.0
    c[1::5, 1] = 0.0
    c[5] = c[4]
    for kind in ("linear", "shallow", "knee"):
        _check(mod, c, _table(kind, B, k, rng), f"sched-ties-{kind}")
    flat = np.full(B * (k + 1) + 1, 5.0, dtype=np.float32)
    ref = _check(mod, c, flat, "sched-flat")
    assert np.array_equal(ref["n"], (ref["a"] > 0).sum(axis=1))   # a flat cost takes every positive survival


def test_confidence_schedule_then_ragged_verify(mod):
    """Confidence head -> batch scheduler -> ragged block verification, all on the
    device with no host round trip between the launches."""
    wl = workloads.make("c5", B=64)
    dev = H.to_dev(wl)
    hid = torch.from_numpy(wl.hidden.view(np.int16)).cuda()
    w = torch.from_numpy(wl.conf_w.view(np.int16)).cuda()
    _, c, _ = mod.adaptive_k(hid, w, wl.conf_b, wl.verify_ms)
    ms = _table("shallow", wl.B, wl.k, None)
    n, total, _ = mod.schedule_batch(c, torch.from_numpy(ms).cuda())
    dev["num_drafts"] = n
    g = H.run_gpu(mod, dev, "block", wl.seed, 0)
    c_h = c.cpu().numpy()
    ref = osch.batch_schedule(c_h, ms)
    n_g = n.cpu().numpy()
    if ref["margin"] >= RATIO_NEAR and not 0.0 < ref["cut_gap"] <= KERNEL_RESOLUTION:
        assert np.array_equal(n_g, ref["n"])
    wl.num_drafts = n_g
    o = H.run_oracle(wl, "block", 0)
    t = H.Tally()
    H.compare(g, o, wl, "block", t, label="c5-batch-scheduled")
    print(f"[c5 batch schedule] m={ref['m']} n histogram {np.bincount(n_g, minlength=6).tolist()} "
          f"{t.summary()}", flush=True)
    H.assert_clean(t)
    # the confidences the scheduler read are the confidence head's (fp32 of the fp64 sigmoid)
    refc = odsp.adaptive_k(wl.hidden, wl.conf_w, wl.conf_b, wl.verify_ms)
    assert np.allclose(c_h, refc["c"], rtol=1e-5, atol=0)


def test_cost_table_times_real_verify_steps(mod):
    """Event pairs around 45 verify calls at three token counts, read back without a
    host wait inside the loop; then one synchronisation and a final poll."""
    wl = workloads.make_zipf("costtable", seed=21, B=4, k=5, V=5000, dtype="bf16", sigma=2.0)
    dev = H.to_dev(wl)
    n_tab = 64
    boot = (10.0 + 2.4 * np.arange(n_tab)).astype(np.float32)
    table = mod.CostTable(boot, window=32, min_samples=3, rebuild_every=8)
    counts = [wl.B * (g + 1) for g in (1, 3, 5)]           # B streams x (gamma + 1) tokens
    filed_in_loop = 0
    for i in range(45):
        gamma = (1, 3, 5)[i % 3]
        nd = torch.full((wl.B,), gamma, dtype=torch.int32, device="cuda")
        table.begin(counts[i % 3])
        mod.verify_block(dev["target"], dev["draft"], dev["draft_tokens"], num_drafts=nd,
                         temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"], anchor=dev["anchor"],
                         seed=wl.seed, step=i)
        table.end()
        filed_in_loop += table.poll()
    torch.cuda.synchronize()
    filed_after = table.poll()
    st = table.stats()
    print(f"[cost table] filed in loop {filed_in_loop}, after sync {filed_after}, stats {st}", flush=True)
    assert st["filed"] == 45 and st["in_flight"] == 0 and st["dropped"] == 0
    toks, ms = table.log()
    assert sorted(set(toks.tolist())) == sorted(counts)
    assert toks.tolist() == [counts[i % 3] for i in range(45)]       # filed in launch order
    assert np.all(ms > 0) and np.all(ms < 1000)
    ref, _ = osch.online_table(boot, list(zip(toks.tolist(), ms.tolist())), 32, 3, 8)
    assert np.array_equal(table.table(), ref)
    live = table.table()
    assert all(live[t] != boot[t] for t in counts)                   # 15 samples each: live medians served
    # the served table drives the scheduler directly
    c = np.random.Generator(np.random.PCG64(3)).uniform(0.5, 0.95, size=(4, 5)).astype(np.float32)
    ms_tab = np.concatenate([live, np.full(max(0, 4 * 6 + 1 - n_tab), live[-1], np.float32)])
    _check(mod, c, ms_tab, "sched-live-table")
