"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties one oracle step to something other than itself: exact
enumeration of the emitted-sequence distribution (losslessness), closed forms,
special cases, and the worked numbers the pages print (tests/golden/).  The
"planted mistake" tests put a plausible bug into the oracle on the CPU and
check that a pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import dspark, enumerate as en, philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")


def _rows_c1(b):
    wl = workloads.make("c1")
    p = np.exp(dspark.log_softmax(dspark.widen(wl.target[b], "f32")))
    q = np.exp(dspark.log_softmax(dspark.widen(wl.draft[b], "f32")))
    return p, q


def _position_only(p, q):
    return (lambda pre: p[len(pre)]), (lambda pre: q[len(pre)])


# ---------------------------------------------------------------- losslessness
@pytest.mark.parametrize("method", ["tokenwise", "block"])
@pytest.mark.parametrize("b", range(4))
def test_lossless_c1(method, b):
    """Emitted sequences are distributed as target-only sampling (exact, C1 shape)."""
    p, q = _rows_c1(b)
    pf, qf = _position_only(p, q)
    E = en.emitted_distribution(pf, qf, 3, 16, method)
    assert en.lossless_error(E, en.target_joint(pf, 3, 16)) < 1e-12


def _markov_model(seed, V=8, k=3, R=4, scale=0.9):
    """Markov drafter and Markov target with a tiny vocabulary (bias big enough to matter)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W1 = workloads.f32_to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * scale)
    W2t = workloads.f32_to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32) * scale)
    d = rng.standard_normal((k, V)) * 1.5
    t = rng.standard_normal((k + 1, V)) * 1.5
    A = rng.standard_normal((V, V)) * 1.2
    anchor = 3
    T = 0.8

    def qf(pre):
        j = len(pre)
        prev = anchor if j == 0 else pre[-1]
        return np.exp(dspark.log_softmax((d[j] + dspark.markov_bias(W1, W2t, [prev])[0]) / T))

    def pf(pre):
        j = len(pre)
        prev = anchor if j == 0 else pre[-1]
        return np.exp(dspark.log_softmax((t[j] + A[prev]) / T))

    return pf, qf, V, k


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_lossless_markov_draft_and_target(method):
    """Drafter conditioned on the previous draft token through W1 W2, target conditioned on the prefix."""
    pf, qf, V, k = _markov_model(7)
    E = en.emitted_distribution(pf, qf, k, V, method)
    assert en.lossless_error(E, en.target_joint(pf, k, V)) < 1e-12


@pytest.mark.parametrize("gamma", [1, 2, 4])
def test_lossless_other_block_lengths(gamma):
    rng = np.random.Generator(np.random.PCG64(gamma))
    V = 6
    p = np.exp(dspark.log_softmax(rng.standard_normal((gamma + 1, V)) * 2))
    q = np.exp(dspark.log_softmax(rng.standard_normal((gamma, V)) * 2))
    pf, qf = _position_only(p, q)
    J = en.target_joint(pf, gamma, V)
    for method in ("tokenwise", "block"):
        assert en.lossless_error(en.emitted_distribution(pf, qf, gamma, V, method), J) < 1e-12


def test_planted_unclipped_prefix_is_caught(monkeypatch):
    """The page's prefix ratio read without clipping breaks losslessness by a wide margin."""
    def unclipped(logr):
        return np.concatenate([[0.0], np.cumsum(logr)])
    p, q = _rows_c1(0)
    pf, qf = _position_only(p, q)
    monkeypatch.setattr(dspark, "block_prefix", unclipped)
    with np.errstate(all="ignore"):
        E = en.emitted_distribution(pf, qf, 3, 16, "block")
        err = en.lossless_error(E, en.target_joint(pf, 3, 16))
    assert not err <= 1e-6  # large, or NaN where P > 1 makes h meaningless


def test_planted_misaligned_threshold_is_caught(monkeypatch):
    """Using slot i-1's distributions for R_i (an off-by-one) breaks losslessness."""
    orig = dspark.block_thresholds

    def shifted(logP, p_rows, q_rows):
        return orig(logP, np.roll(p_rows, 1, axis=0), np.roll(q_rows, 1, axis=0))
    p, q = _rows_c1(1)
    pf, qf = _position_only(p, q)
    monkeypatch.setattr(dspark, "block_thresholds", shifted)
    E = en.emitted_distribution(pf, qf, 3, 16, "block")
    assert en.lossless_error(E, en.target_joint(pf, 3, 16)) > 1e-6  # vs < 1e-12 when correct


def test_planted_wrong_residual_sign_is_caught(monkeypatch):
    monkeypatch.setattr(dspark, "residual_weights",
                        lambda logP, p, q: np.maximum(0.0, q - math.exp(logP) * p))
    p, q = _rows_c1(2)
    pf, qf = _position_only(p, q)
    E = en.emitted_distribution(pf, qf, 3, 16, "tokenwise")
    assert en.lossless_error(E, en.target_joint(pf, 3, 16)) > 1e-6  # vs < 1e-12 when correct


# ---------------------------------------------------------------- dominance
@pytest.mark.parametrize("b", range(4))
def test_block_dominates_tokenwise(b):
    """P(tau >= m) >= P(t >= m) for all m, equal at m = 1 (P1 §5 Figure 4: position 1 unchanged)."""
    p, q = _rows_c1(b)
    pf, qf = _position_only(p, q)
    tw = en.accepted_length_tail(en.emitted_distribution(pf, qf, 3, 16, "tokenwise"))
    bl = en.accepted_length_tail(en.emitted_distribution(pf, qf, 3, 16, "block"))
    assert np.all(bl >= tw - 1e-13)
    assert abs(bl[1] - tw[1]) < 1e-13
    assert np.sum(bl[1:]) >= np.sum(tw[1:])


def test_pathwise_block_can_stop_before_tokenwise():
    """Counterexample: r_0 = 0.5 and p_1 = q_1 give h_1 = 0, h_2 = 0.5; u = (0.1, 0.7) -> t = 2, tau = 0.

    So "block length >= token-wise length on the same uniforms" is not a
    pathwise property; only the distributional dominance above holds.
    """
    V = 4
    p0 = np.array([0.1, 0.2, 0.3, 0.4])
    q0 = np.array([0.2, 0.2, 0.3, 0.3])
    p1 = q1 = np.array([0.25, 0.25, 0.25, 0.25])
    p2 = np.array([0.4, 0.3, 0.2, 0.1])
    x = np.array([0, 1])
    logp = np.log(np.stack([p0, p1, p2]))
    logq = np.log(np.stack([q0, q1]))
    logr = dspark.log_ratios(logp, logq, x)
    assert abs(math.exp(logr[0]) - 0.5) < 1e-15 and abs(logr[1]) < 1e-15
    logP = dspark.block_prefix(logr)
    R, h = dspark.block_thresholds(logP, np.exp(logp), np.exp(logq))
    assert abs(h[1]) < 1e-15 and abs(h[2] - 0.5) < 1e-15
    u = np.array([0.1, 0.7])
    assert dspark.tokenwise_stop(logr, u)[0] == 2
    assert dspark.block_stop(h, u)[0] == 0
    del V


# ---------------------------------------------------------------- closed forms
def test_log_softmax_closed_forms():
    a, b = 1.7, -0.4
    ls = dspark.log_softmax(np.array([a, b]))
    assert abs(ls[0] - (-math.log1p(math.exp(b - a)))) < 1e-15
    assert np.allclose(dspark.log_softmax(np.zeros(129280)), -math.log(129280), atol=1e-12, rtol=0)
    x = np.random.Generator(np.random.PCG64(0)).standard_normal(1000) * 3
    assert np.allclose(dspark.log_softmax(x), dspark.log_softmax(x + 123.25), atol=1e-12)


def test_markov_bias_closed_forms():
    """One-hot W1 rows pick a column of W2 (a row of W2t); prev = -1 gives zero."""
    rng = np.random.Generator(np.random.PCG64(1))
    V, R = 40, 8
    W2t = workloads.f32_to_bf16_bits(rng.standard_normal((V, R)).astype(np.float32))
    W1f = np.zeros((V, R), dtype=np.float32)
    W1f[5, 3] = 1.0
    W1f[6, 2] = 2.0
    W1f[6, 7] = -0.5
    W1 = workloads.f32_to_bf16_bits(W1f)
    w2 = workloads.bf16_bits_to_f32(W2t).astype(np.float64)
    bias = dspark.markov_bias(W1, W2t, [5, 6, -1])
    assert np.array_equal(bias[0], w2[:, 3])
    assert np.array_equal(bias[1], 2.0 * w2[:, 2] - 0.5 * w2[:, 7])
    assert np.array_equal(bias[2], np.zeros(V))


def test_tokenwise_acceptance_is_one_minus_tv():
    """Averaged over x ~ q, min(1, p(x)/q(x)) has mean sum_v min(p, q) = 1 - TV(p, q) (P2 §7's TV link)."""
    for b in range(4):
        p, q = _rows_c1(b)
        P_stop, _ = (None, None)
        acc = 0.0
        for x in range(16):
            logr = dspark.log_ratios(np.log(p[:2]), np.log(q[:1]), np.array([x]))
            P_stop, _ = en.stop_distribution("tokenwise", logr, p[:2], q[:1])
            acc += q[0, x] * P_stop[1]
        assert abs(acc - (1.0 - 0.5 * np.sum(np.abs(p[0] - q[0])))) < 1e-14


def test_k1_block_equals_tokenwise():
    """With one draft h_1 = P_1 = min(1, r_0) and both residuals are max(0, p_0 - q_0)."""
    for seed in range(30):
        wl = workloads.make_tiny(seed=100 + seed, k=1)
        kw = dict(target=wl.target, draft=wl.draft, dtype="f32", draft_tokens=wl.draft_tokens,
                  seed=seed, step=seed)
        a = dspark.verify(method="tokenwise", **kw)
        b = dspark.verify(method="block", **kw)
        assert np.array_equal(a["accepted_len"], b["accepted_len"])
        assert np.array_equal(a["out_tokens"], b["out_tokens"])


def test_q_equals_p_accepts_everything():
    wl = workloads.make_tiny(seed=3)
    draft = wl.target[:, :3].copy()
    for step in range(20):
        for method in ("tokenwise", "block"):
            r = dspark.verify(wl.target, draft, "f32", wl.draft_tokens, seed=1, step=step, method=method)
            assert np.all(r["accepted_len"] == 3)


def test_one_hot_target_is_deterministic():
    """A target with one overwhelming logit per row emits that token with certainty."""
    wl = workloads.make_tiny(seed=4)
    tgt = np.zeros_like(wl.target)
    tgt[:, :, 7] = 80.0
    for step in range(10):
        r = dspark.verify(tgt, wl.draft, "f32", wl.draft_tokens, seed=2, step=step, method="block")
        for b in range(4):
            s = r["accepted_len"][b]
            assert np.all(r["out_tokens"][b, :s] == 7) and r["out_tokens"][b, s] == 7


def test_zero_drafts_sample_the_first_position():
    wl = workloads.make_tiny(seed=5)
    r = dspark.verify(wl.target, wl.draft, "f32", wl.draft_tokens, num_drafts=np.zeros(4, np.int32),
                      seed=1, step=0, method="block")
    assert np.all(r["accepted_len"] == 0)
    assert np.all(r["out_tokens"][:, 1:] == -1)


def test_race_two_point_closed_form():
    """Exponential race over two weights: P(first) = w1 / (w1 + w2)."""
    w = np.array([0.3, 0.0, 0.0, 0.7])
    wins = 0
    n = 4000
    for step in range(n):
        Y, _ = dspark.race_sample(w, seed=9, b=0, step=step)
        assert Y in (0, 3)
        wins += Y == 0
    # binomial sd = sqrt(n * .21) ~ 29
    assert abs(wins - 0.3 * n) < 4.5 * math.sqrt(n * 0.21)


# ---------------------------------------------------------------- pages' numbers
def _golden():
    return json.load(open(GOLDEN))


def test_prefix_survival_worked_example():
    g = _golden()["prefix_survival"]
    a = dspark.prefix_survival(g["c"])
    assert np.allclose(np.round(a, g["printed_decimals"]), g["a_printed"], atol=1e-12)
    assert abs(a[2] - 0.72675) < 1e-12 and abs(a[3] - 0.2907) < 1e-12


@pytest.mark.parametrize("key", ["tokens_per_step_k5", "tokens_per_step_k9"])
def test_tokens_per_step_worked_examples(key):
    g = _golden()[key]
    assert round(dspark.tokens_per_step(g["a_p"]), g["printed_decimals"]) == g["tokens_per_step_printed"]
    if "positions_6_to_9_printed" in g:
        assert round(float(np.sum(g["a_p"][5:])), 3) == g["positions_6_to_9_printed"]


def test_figure4_sums():
    g = _golden()["figure4_per_position"]
    assert round(dspark.tokens_per_step(g["tokenwise"]), 3) == g["tokens_per_step_printed"]["tokenwise"]
    assert abs(dspark.tokens_per_step(g["block"]) - g["tokens_per_step_printed"]["block"]) <= 0.0025
    assert abs(np.sum(np.array(g["block"]) - np.array(g["tokenwise"])) - g["gap_sum_printed"]) <= 0.0025
    m = dspark.marginal_acceptance(g["tokenwise"])
    assert abs(m[0] - 0.793) < 1e-12 and abs(m[1] - 0.604 / 0.793) < 1e-12


def test_adaptive_worked_example():
    """c = (.95, .90, .85, .40) with verify_ms[t] = 10 + 2.4 t.

    E/ms by hand: n=0 1/12.4 = .0806, n=1 1.95/14.8 = .1318, n=2 2.805/17.2 = .1631,
    n=3 3.53175/19.6 = .1802, n=4 3.82245/22.0 = .1737 -> n* = 3.
    """
    a = dspark.prefix_survival([0.95, 0.90, 0.85, 0.40])
    ms = (10.0 + 2.4 * np.arange(64)).astype(np.float32)
    n, margin = dspark.adaptive_choice(a, ms)
    assert n == 3
    assert abs(margin - (3.53175 / float(np.float32(19.6)) - 3.82245 / float(np.float32(22.0)))
               / (3.53175 / float(np.float32(19.6)))) < 1e-12


def test_adaptive_ties_pick_smallest_n():
    a = np.array([0.0, 0.0])
    ms = np.full(8, 5.0, dtype=np.float32)
    assert dspark.adaptive_choice(a, ms)[0] == 0


def test_confidence_closed_form():
    """sigmoid(w . h + b) with one-hot hidden states picks single weights."""
    H = 16
    w = workloads.f32_to_bf16_bits(np.linspace(-2, 2, H).astype(np.float32))
    hid = np.zeros((1, 3, H), dtype=np.float32)
    hid[0, 0, 0] = 1.0
    hid[0, 1, H - 1] = 1.0
    c = dspark.confidence(workloads.f32_to_bf16_bits(hid), w, 0.5)
    assert abs(c[0, 0] - 1 / (1 + math.exp(-(-2.0 + 0.5)))) < 1e-15
    assert abs(c[0, 1] - 1 / (1 + math.exp(-(2.0 + 0.5)))) < 1e-15
    assert abs(c[0, 2] - 1 / (1 + math.exp(-0.5))) < 1e-15


def test_accept_uniform_threshold_ends():
    """u in (0, 1]: a threshold of 1 always accepts, 0 never."""
    u = philox.accept_uniforms(3, 0, 5000, 0)
    assert np.all(u <= 1.0) and np.all(u > 0.0)
    assert dspark.tokenwise_stop(np.zeros(3), u[:3])[0] == 3
    assert dspark.tokenwise_stop(np.full(3, -np.inf), u[:3])[0] == 0


# ----------------------------------------------------------------------------
# greedy branch, temperature 0 [P1 §4 "Greedy is a different code path"]
# ----------------------------------------------------------------------------
def _separated_rows(rng, rows, V, gap=4.0):
    """Gaussian logits whose largest entry leads the second by at least `gap`."""
    x = rng.standard_normal((rows, V))
    top = np.argmax(x, axis=-1)
    x[np.arange(rows), top] = np.max(np.delete(x, 0, axis=-1), axis=-1).clip(min=x.max()) + gap
    return x.astype(np.float32)


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_greedy_is_the_low_temperature_limit(seed):
    """As T -> 0, p_j and q_j become one-hot at their argmax; with greedy drafts
    (x_j = argmax q_j) both sampled verifiers then keep exactly the drafts that equal
    the target argmax and emit the target argmax at the stop.  The T = 0 branch must
    give the same lengths and tokens as both verifiers at T = 1e-3."""
    rng = np.random.default_rng(100 + seed)
    B, k, V = 6, 4, 40
    target = np.stack([_separated_rows(rng, k + 1, V) for _ in range(B)])
    draft = np.stack([_separated_rows(rng, k, V) for _ in range(B)])
    # let some drafts agree with the target so that blocks are partly kept
    for b in range(B):
        for j in range(k):
            if rng.random() < 0.6:
                draft[b, j] = target[b, j]
    x = np.argmax(draft, axis=-1).astype(np.int32)
    g = dspark.verify(target, draft, "f32", x, temperature=np.zeros(B, np.float32), seed=seed, method="block")
    for method in ("tokenwise", "block"):
        r = dspark.verify(target, draft, "f32", x, temperature=np.full(B, 1e-3, np.float32), seed=seed,
                          method=method)
        assert np.array_equal(g["accepted_len"], r["accepted_len"]), method
        assert np.array_equal(g["out_tokens"], r["out_tokens"]), method
    assert 0 < int(np.sum(g["accepted_len"])) < B * k   # both kept and rejected drafts occur


def test_greedy_ties_go_to_the_lowest_id():
    V, k = 12, 2
    target = np.zeros((1, k + 1, V), np.float32)
    target[0, 0, [5, 9]] = 3.0        # two equal maxima: id 5 is the argmax
    target[0, 1, 2] = 1.0
    target[0, 2, [7, 8]] = 2.0
    draft = np.zeros((1, k, V), np.float32)
    zero = np.zeros(1, np.float32)
    r = dspark.verify(target, draft, "f32", np.array([[9, 2]], np.int32), temperature=zero, method="tokenwise")
    assert r["accepted_len"][0] == 0 and r["out_tokens"][0].tolist() == [5, -1, -1]
    r = dspark.verify(target, draft, "f32", np.array([[5, 2]], np.int32), temperature=zero, method="block")
    assert r["accepted_len"][0] == 2 and r["out_tokens"][0].tolist() == [5, 2, 7]


def test_greedy_ignores_seed_step_and_method():
    wl = workloads.make_zipf("g", 11, 6, 4, V=300, dtype="bf16", greedy_every=1)
    outs = [dspark.verify(wl.target, wl.draft, wl.dtype, wl.draft_tokens, wl.temperature, wl.anchor, wl.W1,
                          wl.W2t, seed=sd, step=st, method=m)
            for sd, st, m in ((1, 0, "block"), (2, 5, "tokenwise"), (3, 9, "block"))]
    for o in outs[1:]:
        assert np.array_equal(o["accepted_len"], outs[0]["accepted_len"])
        assert np.array_equal(o["out_tokens"], outs[0]["out_tokens"])
    assert np.all(np.isnan(outs[0]["diag"]))


# ----------------------------------------------------------------------------
# reduced draft vocabulary [P1 §3: the drafter scores a reduced vocabulary and
# scatters its logits into target columns; q = 0 on every other id]
# ----------------------------------------------------------------------------
def _reduced(q_rows, keep):
    """q restricted to the ids in `keep` (renormalised), zero elsewhere."""
    r = np.where(keep[None, :], q_rows, 0.0)
    return r / r.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_lossless_with_reduced_draft_vocab(method):
    """Target mass on ids the drafter cannot propose must still reach the output: the
    residual max(0, P p - q) keeps P p where q = 0, and the law stays target-only."""
    rng = np.random.Generator(np.random.PCG64(5))
    V, gamma = 7, 3
    keep = np.zeros(V, dtype=bool)
    keep[[0, 2, 3, 6]] = True
    p = np.exp(dspark.log_softmax(rng.standard_normal((gamma + 1, V)) * 1.5))
    q = _reduced(np.exp(dspark.log_softmax(rng.standard_normal((gamma, V)) * 1.5)), keep)
    pf, qf = _position_only(p, q)
    with np.errstate(divide="ignore"):
        E = en.emitted_distribution(pf, qf, gamma, V, method)
    assert en.lossless_error(E, en.target_joint(pf, gamma, V)) < 1e-12


def test_planted_residual_over_draft_vocab_only_is_caught(monkeypatch):
    """A residual that skips the ids outside the draft vocabulary loses their target mass."""
    rng = np.random.Generator(np.random.PCG64(6))
    V, gamma = 7, 2
    keep = np.zeros(V, dtype=bool)
    keep[[1, 4, 5]] = True
    p = np.exp(dspark.log_softmax(rng.standard_normal((gamma + 1, V)) * 1.5))
    q = _reduced(np.exp(dspark.log_softmax(rng.standard_normal((gamma, V)) * 1.5)), keep)
    pf, qf = _position_only(p, q)
    real = dspark.residual_weights

    def draft_vocab_only(logP, p_row, q_row):
        return np.where(q_row > 0, real(logP, p_row, q_row), 0.0)
    monkeypatch.setattr(dspark, "residual_weights", draft_vocab_only)
    with np.errstate(all="ignore"):
        E = en.emitted_distribution(pf, qf, gamma, V, "tokenwise")
        err = en.lossless_error(E, en.target_joint(pf, gamma, V))
    assert not err <= 1e-6
