"""Monte Carlo of the oracle's full sampler (Philox uniforms, race sampler) against exact enumeration.

This pins the parts the enumeration integrates out analytically: the
u-based stop rules, the uniform conversion and the exponential race.
"""
import numpy as np
import pytest

import workloads
from oracle import dspark, enumerate as en


def _chi2(counts, expected, min_expected=5.0):
    """Pearson chi^2 after pooling cells with small expectation; returns (chi2, dof)."""
    counts = np.asarray(counts, dtype=np.float64).ravel()
    expected = np.asarray(expected, dtype=np.float64).ravel()
    big = expected >= min_expected
    c = np.append(counts[big], counts[~big].sum())
    e = np.append(expected[big], expected[~big].sum())
    keep = e > 0
    c, e = c[keep], e[keep]
    return float(np.sum((c - e) ** 2 / e)), int(len(e) - 1)


CHI2_999 = {d: d + 3.09 * np.sqrt(2 * d) + 2 for d in range(1, 200)}  # generous 0.999 bound


def test_race_sample_distribution():
    rng = np.random.Generator(np.random.PCG64(11))
    w = rng.random(16) ** 3
    w[[2, 9]] = 0.0
    n = 20000
    counts = np.zeros(16)
    for step in range(n):
        Y, _ = dspark.race_sample(w, seed=3, b=1, step=step)
        counts[Y] += 1
    assert counts[2] == 0 and counts[9] == 0
    chi2, dof = _chi2(counts, n * w / w.sum())
    assert chi2 < CHI2_999[dof], (chi2, dof)


def test_race_ids_sharing_a_generator_block_are_independent():
    """Ids 4i .. 4i+3 read the four words of one Philox block: a race over such a quad
    with equal weights must still pick each of them a quarter of the time, and the
    pairs (winner at step s over ids 0..3, winner over ids 4..7) must be uniform on
    the 16 cells (independent blocks)."""
    n = 16000
    pair = np.zeros((4, 4))
    w = np.ones(4)
    for step in range(n):
        a, _ = dspark.race_sample(np.concatenate([w, np.zeros(4)]), seed=8, b=0, step=step)
        c, _ = dspark.race_sample(np.concatenate([np.zeros(4), w]), seed=8, b=0, step=step)
        pair[a, c - 4] += 1
    chi2, dof = _chi2(pair, np.full((4, 4), n / 16))
    assert chi2 < CHI2_999[dof], (chi2, dof)


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_verify_matches_enumeration(method):
    """(accepted length, emitted token) frequencies of oracle.verify at C1 vs the exact law."""
    wl = workloads.make("c1")
    streams = [0, 2]
    n = 3000
    rng = np.random.Generator(np.random.PCG64(2024))
    p = {b: np.exp(dspark.log_softmax(dspark.widen(wl.target[b], "f32"))) for b in streams}
    q = {b: np.exp(dspark.log_softmax(dspark.widen(wl.draft[b], "f32"))) for b in streams}
    counts = {b: np.zeros((4, 16)) for b in streams}
    for step in range(n):
        toks = np.zeros((4, 3), dtype=np.int32)
        for b in streams:
            for j in range(3):
                toks[b, j] = rng.choice(16, p=q[b][j])
        r = dspark.verify(wl.target, wl.draft, "f32", toks, seed=1, step=step, method=method)
        for b in streams:
            s = r["accepted_len"][b]
            counts[b][s, r["out_tokens"][b, s]] += 1
    for b in streams:
        pf = lambda pre, b=b: p[b][len(pre)]
        qf = lambda pre, b=b: q[b][len(pre)]
        E = en.emitted_distribution(pf, qf, 3, 16, method)
        law = np.stack([E[m].reshape(-1, 16).sum(axis=0) for m in range(4)])
        assert abs(law.sum() - 1.0) < 1e-12
        chi2, dof = _chi2(counts[b], n * law)
        assert chi2 < CHI2_999[dof], (b, chi2, dof)


# ----------------------------------------------------------------------------
# the Markov path of oracle.verify [P2 §6 "Why the Markov Head Helps"; P1 §3 "The
# Markov fix-up", Figure 2]: drafts drawn slot by slot from the drafter with its
# Markov head, x_j ~ softmax((d_j + W1[x_{j-1}] W2) / T), x_{-1} = the anchor, then
# verified by the oracle with W1, W2t, the anchor and T.  The emitted prefix,
# continued by sampling the target, must be distributed as the target alone [P1 §1
# "One token per step"]: Pr(z) = prod_j softmax(t_j / T)(z_j).  This law involves
# neither the drafter nor anything the oracle computes.
# ----------------------------------------------------------------------------
def _markov_case():
    import workloads as wls
    rng = np.random.Generator(np.random.PCG64(77))
    V, k, R, B = 4, 3, 4, 32
    W1 = wls.f32_to_bf16_bits((rng.standard_normal((V, R)) * 0.9).astype(np.float32))
    W2t = wls.f32_to_bf16_bits((rng.standard_normal((V, R)) * 0.9).astype(np.float32))
    d = (rng.standard_normal((k, V)) * 1.2).astype(np.float32)
    t = (rng.standard_normal((k + 1, V)) * 1.2).astype(np.float32)
    return dict(V=V, k=k, B=B, W1=W1, W2t=W2t, d=d, t=t, anchor=2, T=np.float32(0.5))


def _markov_full_sequences(case, method, n_calls, seed):
    V, k, B, T = case["V"], case["k"], case["B"], float(case["T"])
    w1 = workloads.bf16_bits_to_f32(case["W1"]).astype(np.float64)
    w2t = workloads.bf16_bits_to_f32(case["W2t"]).astype(np.float64)
    d = case["d"].astype(np.float64)
    t = case["t"].astype(np.float64)

    def softmax(z):
        e = np.exp(z - z.max())
        return e / e.sum()

    p_rows = np.stack([softmax(t[j] / T) for j in range(k + 1)])
    target = np.broadcast_to(case["t"], (B, k + 1, V)).copy()
    draft = np.broadcast_to(case["d"], (B, k, V)).copy()
    temps = np.full(B, case["T"], np.float32)
    anchors = np.full(B, case["anchor"], np.int64)
    rng = np.random.Generator(np.random.PCG64(seed))
    counts = np.zeros((V,) * (k + 1))
    for step in range(n_calls):
        toks = np.zeros((B, k), np.int32)
        for b in range(B):
            prev = case["anchor"]
            for j in range(k):
                toks[b, j] = rng.choice(V, p=softmax((d[j] + w2t @ w1[prev]) / T))
                prev = toks[b, j]
        r = dspark.verify(target, draft, "f32", toks, temps, anchors, case["W1"], case["W2t"], seed=seed,
                          step=step, method=method)
        for b in range(B):
            s = int(r["accepted_len"][b])
            z = list(r["out_tokens"][b, : s + 1])
            for j in range(s + 1, k + 1):
                z.append(rng.choice(V, p=p_rows[j]))
            counts[tuple(z)] += 1
    law = p_rows[0]
    for j in range(1, k + 1):
        law = np.multiply.outer(law, p_rows[j])
    return counts, law


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_markov_verify_is_target_only_sampling(method):
    case = _markov_case()
    counts, law = _markov_full_sequences(case, method, 500, 5)
    chi2, dof = _chi2(counts, counts.sum() * law)
    assert chi2 < CHI2_999[dof], (chi2, dof)


def _planted_prev_is_current(anchor, x, gamma):
    return np.asarray(x[:gamma], dtype=np.int64)


def _planted_anchor_ignored(anchor, x, gamma):
    return np.concatenate([[-1], np.asarray(x[: max(gamma - 1, 0)], dtype=np.int64)])[:gamma]


def _planted_temperature_first(d, W1, W2t, prev, T):
    return d / T + (dspark.markov_bias(W1, W2t, prev) if W1 is not None else 0.0)


@pytest.mark.parametrize("plant", ["prev_is_current", "anchor_ignored", "temperature_first"])
def test_markov_planted_mistakes_are_caught(monkeypatch, plant):
    if plant == "prev_is_current":
        monkeypatch.setattr(dspark, "draft_prev_tokens", _planted_prev_is_current)
    elif plant == "anchor_ignored":
        monkeypatch.setattr(dspark, "draft_prev_tokens", _planted_anchor_ignored)
    else:
        monkeypatch.setattr(dspark, "draft_scaled_logits", _planted_temperature_first)
    case = _markov_case()
    counts, law = _markov_full_sequences(case, "block", 250, 6)
    chi2, dof = _chi2(counts, counts.sum() * law)
    assert chi2 > 3 * CHI2_999[dof], (plant, chi2, dof)
