"""Pins of the batch-level scheduler and the online cost table in the oracle.

Scheduler: brute force over every per-stream draft count vector on small
batches (any positive cost table, unrounded fp64 survivals, 1e-12 relative), the single-stream case against the
per-stream adaptive choice and the pages' worked example, and closed-form
special cases (flat cost, zero confidence, a linear cost whose marginal price
exceeds every survival).  Online table: hand-computed medians, windows and
rebuild points.
"""
import itertools

import numpy as np
import pytest

from oracle import dspark, schedule


def _rng(seed):
    return np.random.default_rng(seed)


def _brute_force(a, ms):
    """max over all n in [0, k]^B of (B + sum_b sum_{j<n_b} a[b, j]) / ms[B + sum n],
    with the survivals a as the oracle computes them (fp64, unrounded)."""
    B, k = a.shape
    best = -1.0
    for n in itertools.product(range(k + 1), repeat=B):
        E = B + sum(float(np.sum(a[b, :n[b]])) for b in range(B))
        best = max(best, E / float(ms[B + sum(n)]))
    return best


@pytest.mark.parametrize("B,k,seed", [(2, 4, 0), (3, 3, 1), (4, 2, 2), (3, 3, 3)])
def test_batch_schedule_matches_brute_force(B, k, seed):
    g = _rng(seed)
    for trial in range(6):
        c = g.uniform(0.0, 1.0, size=(B, k)).astype(np.float32)
        if trial % 3 == 1:
            c[0, :] = 1.0                       # ties along a stream
        kind = trial % 3
        t = np.arange(B * (k + 1) + 1, dtype=np.float64)
        if kind == 0:
            ms = 10.0 + 2.4 * t
        elif kind == 1:
            ms = 5.0 + 0.3 * np.maximum(0.0, t - B - 2) ** 2      # flat, then convex
        else:
            ms = g.uniform(1.0, 20.0, size=t.shape)                 # arbitrary positive table
        ms = ms.astype(np.float32)
        r = schedule.batch_schedule(c, ms)
        a = r["a"]
        # survivals: running products of the confidences (independent of the oracle's loop)
        assert np.allclose(a, np.cumprod(c.astype(np.float64), axis=1), rtol=1e-15, atol=0)
        bf = _brute_force(a, ms)
        assert abs(r["ratio"][r["m"]] - bf) <= 1e-12 * bf
        # the returned counts realise that optimum
        E = B + sum(float(np.sum(a[b, :r["n"][b]])) for b in range(B))
        assert abs(E / float(ms[B + int(r["n"].sum())]) - bf) <= 1e-12 * bf
        assert int(r["n"].sum()) == r["m"]


def test_greedy_order_takes_prefixes_of_each_stream():
    g = _rng(7)
    c = g.uniform(0.0, 1.0, size=(6, 5)).astype(np.float32)
    c[1, 2:] = 1.0
    c[2, 1] = 0.0
    order = schedule.greedy_order(schedule.prefix_survival_rows(c))
    for m in range(len(order) + 1):
        taken = {}
        for (b, j) in order[:m]:
            taken.setdefault(b, []).append(j)
        for b, js in taken.items():
            assert sorted(js) == list(range(len(js)))


def test_single_stream_is_the_per_stream_choice():
    """B = 1: B + m tokens = 1 + n, the per-stream rule's verify_ms[n + 1]."""
    g = _rng(11)
    for _ in range(50):
        k = int(g.integers(1, 9))
        c = g.uniform(0.2, 1.0, size=(1, k)).astype(np.float32)
        ms = (g.uniform(5, 10) + g.uniform(0.5, 4.0) * np.arange(k + 2)).astype(np.float32)
        r = schedule.batch_schedule(c, ms)
        n_ps, _ = dspark.adaptive_choice(dspark.prefix_survival(c[0].astype(np.float64)), ms)
        assert r["n"][0] == n_ps


def test_worked_example_single_stream():
    """c = (.95, .90, .85, .40), verify_ms[t] = 10 + 2.4 t: n* = 3 (E/ms .1802 at 4 tokens)."""
    c = np.array([[0.95, 0.90, 0.85, 0.40]], dtype=np.float32)
    ms = (10.0 + 2.4 * np.arange(64)).astype(np.float32)
    r = schedule.batch_schedule(c, ms)
    assert r["n"].tolist() == [3] and r["m"] == 3
    assert abs(r["ratio"][3] - 0.1802) < 5e-5


def test_flat_cost_takes_every_positive_draft():
    g = _rng(5)
    c = g.uniform(0.05, 1.0, size=(8, 4)).astype(np.float32)
    ms = np.full(8 * 5 + 1, 7.0, dtype=np.float32)
    r = schedule.batch_schedule(c, ms)
    assert r["n"].tolist() == [4] * 8


def test_zero_confidence_takes_nothing():
    c = np.zeros((5, 3), dtype=np.float32)
    ms = np.full(5 * 4 + 1, 7.0, dtype=np.float32)      # flat: every m ties, the smallest wins
    assert schedule.batch_schedule(c, ms)["n"].tolist() == [0] * 5


def test_linear_cost_above_every_survival_takes_nothing():
    """verify_ms[t] = 10 + 2.4 t at B = 256: one more token costs 2.4 ms while the
    batch already earns 256 / 624.4 tokens per ms, so a draft pays only if its
    survival exceeds 2.4 * 256 / 624.4 = 0.98398; with c <= 0.9 none does."""
    g = _rng(9)
    c = g.uniform(0.5, 0.9, size=(256, 5)).astype(np.float32)
    ms = (10.0 + 2.4 * np.arange(256 * 6 + 1)).astype(np.float32)
    r = schedule.batch_schedule(c, ms)
    assert r["m"] == 0 and r["n"].sum() == 0


def test_marginal_price_threshold():
    """Adding a candidate of survival a to a batch earning E tokens in ms milliseconds
    raises the ratio iff a > (ms' - ms) E / ms.  At the chosen m the last candidate
    taken passed that test and the next one fails it (linear costs alpha + beta t)."""
    g = _rng(13)
    for _ in range(20):
        B, k = int(g.integers(1, 7)), int(g.integers(1, 6))
        c = g.uniform(0.3, 1.0, size=(B, k)).astype(np.float32)
        alpha, beta = float(g.uniform(5, 40)), float(g.uniform(0.1, 1.5))
        ms = (alpha + beta * np.arange(B * (k + 1) + 1)).astype(np.float32).astype(np.float64)
        r = schedule.batch_schedule(c, ms)
        a = r["a"]
        order = schedule.greedy_order(a)
        m = r["m"]
        if m > 0:
            b, j = order[m - 1]
            assert a[b, j] > (ms[B + m] - ms[B + m - 1]) * r["ratio"][m - 1] * (1 - 1e-12)
        if m < len(order):
            b, j = order[m]
            assert a[b, j] <= (ms[B + m + 1] - ms[B + m]) * r["ratio"][m] * (1 + 1e-12)


def test_cut_gap_is_the_ranking_resolution_needed():
    """Two streams whose first survivals differ by one fp32 step, a table that pays for
    exactly one draft: the draft goes to the larger survival, and cut_gap is the gap."""
    hi = np.float32(0.9)
    lo = np.nextafter(hi, np.float32(0))
    c = np.array([[lo, 0.5], [hi, 0.5]], dtype=np.float32)
    ms = np.array([1.0, 1.0, 1.0, 1.2, 10.0, 100.0, 100.0], dtype=np.float32)   # B = 2: t = 2..6
    r = schedule.batch_schedule(c, ms)
    assert r["m"] == 1 and r["n"].tolist() == [0, 1]
    assert r["cut_gap"] == float(hi) - float(lo)


def test_schedule_rejects_short_table():
    with pytest.raises(ValueError):
        schedule.batch_schedule(np.full((4, 3), 0.5, np.float32), np.ones(16, np.float32))


# ---------------------------------------------------------------------------
# online cost table
# ---------------------------------------------------------------------------
BOOT = (10.0 + 2.4 * np.arange(64)).astype(np.float32)


def test_table_holds_boot_until_the_first_rebuild():
    obs = [(5, 100.0)] * 31
    table, hist = schedule.online_table(BOOT, obs)
    assert np.array_equal(table, BOOT)
    assert all(np.array_equal(h, BOOT) for h in hist)


def test_first_rebuild_takes_the_median():
    obs = [(5, float(v)) for v in range(1, 33)]         # 1..32 at t = 5
    table, hist = schedule.online_table(BOOT, obs)
    assert table[5] == np.float32(16.5)                   # (16 + 17) / 2
    assert np.array_equal(np.delete(table, 5), np.delete(BOOT, 5))
    assert np.array_equal(hist[30], BOOT)


def test_window_keeps_the_last_32():
    obs = [(5, float(v)) for v in range(1, 65)]         # rebuilds after 32 and 64
    table, hist = schedule.online_table(BOOT, obs)
    assert hist[39][5] == np.float32(16.5)                # 40 observations: still the first rebuild
    assert table[5] == np.float32(48.5)                   # last 32 = 33..64


def test_min_samples_and_odd_medians():
    obs = [(9, 1.0), (9, 10.0), (9, 2.0), (7, 50.0), (7, 60.0)]
    obs += [(5, 3.0)] * 27                                # 32 observations
    table, _ = schedule.online_table(BOOT, obs)
    assert table[9] == np.float32(2.0)                    # median of (1, 10, 2)
    assert table[7] == BOOT[7]                            # only 2 samples: boot kept
    assert table[5] == np.float32(3.0)


def test_out_of_table_observations_are_dropped():
    obs = [(64, 1.0), (-1, 1.0)] + [(3, 4.0)] * 32
    table, hist = schedule.online_table(BOOT, obs)
    assert np.array_equal(hist[32], BOOT)                 # 31 filed so far
    assert table[3] == np.float32(4.0)


def test_cadence_parameters():
    obs = [(2, float(v)) for v in (5, 1, 4, 2)]
    table, hist = schedule.online_table(BOOT, obs, window=3, min_samples=2, rebuild_every=2)
    assert hist[1][2] == np.float32(3.0)                  # (5, 1) -> 3
    assert table[2] == np.float32(2.0)                    # last 3 = (1, 4, 2) -> 2
