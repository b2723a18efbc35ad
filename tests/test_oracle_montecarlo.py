"""Monte Carlo of the oracle's full sampler (Philox uniforms, race sampler) against exact enumeration.

This pins the parts the enumeration integrates out analytically: the
u-based stop rules, the uniform conversion and the two-level race.
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


def test_race_sample_distribution_two_levels():
    rng = np.random.Generator(np.random.PCG64(11))
    w = rng.random(16) ** 3
    w[[2, 9]] = 0.0
    n = 20000
    counts = np.zeros(16)
    for step in range(n):
        Y, _ = dspark.race_sample(w, seed=3, b=1, step=step, group=4)
        counts[Y] += 1
    assert counts[2] == 0 and counts[9] == 0
    chi2, dof = _chi2(counts, n * w / w.sum())
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
