"""Pins of the oracle's drafter walk (Markov head, [P2 §6; P1 §3 "The Markov fix-up"]).

The walk draws x_j from q_j(. | x_{j-1}) = softmax((d_j + W1[x_{j-1}] W2) / T).  Its
joint law is the chain-rule product of those conditionals; the test builds it from
the separately pinned pieces (``markov_bias``, ``log_softmax``) over every sequence
of a tiny vocabulary and checks the walk's draws against it with a chi-square test.
Plausible slips (conditioning on the wrong token, no bias at slot 0, one set of
clocks for every slot) each change the law by far more than the test's tolerance;
``test_walk_same_clocks_every_slot_is_caught`` plants the last one.
"""
import itertools

import numpy as np
import pytest

from oracle import dspark


def _bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # round to nearest even, as bf16 storage does
    r = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + r) >> 16).astype(np.uint16)


def _tiny(seed, V=5, k=3, R=32, scale=0.35):
    rng = np.random.default_rng(seed)
    draft = (rng.standard_normal((1, k, V)) * 1.2).astype(np.float32)
    W1 = _bf16(rng.standard_normal((V, R)) * scale)
    W2t = _bf16(rng.standard_normal((V, R)) * scale)
    return draft, W1, W2t


def _exact_law(draft, W1, W2t, anchor, T):
    _, k, V = draft.shape
    d = draft[0].astype(np.float64)
    law = {}
    for seq in itertools.product(range(V), repeat=k):
        p, prev = 1.0, anchor
        for j, x in enumerate(seq):
            logits = d[j] + dspark.markov_bias(W1, W2t, prev)[0]
            p *= np.exp(dspark.log_softmax(logits / T)[x])
            prev = x
        law[seq] = p
    return law


@pytest.mark.parametrize("anchor", [-1, 2])
def test_walk_follows_the_chain_rule(anchor):
    draft, W1, W2t = _tiny(7)
    T = 0.8
    law = _exact_law(draft, W1, W2t, anchor, T)
    assert abs(sum(law.values()) - 1.0) < 1e-12
    n = 6000
    counts = dict.fromkeys(law, 0)
    for step in range(n):
        r = dspark.draft_walk(draft, "f32", np.array([T], np.float32), np.array([anchor]), W1, W2t,
                              seed=11, step=step)
        counts[tuple(int(t) for t in r["tokens"][0])] += 1
    keys = sorted(law)
    exp = np.array([law[s] * n for s in keys])
    obs = np.array([counts[s] for s in keys])
    big = exp >= 5
    chi2 = float(np.sum((obs[big] - exp[big]) ** 2 / exp[big]))
    dof = int(big.sum()) - 1
    # 5-sigma band of a chi-square with dof degrees of freedom
    assert chi2 < dof + 5 * np.sqrt(2 * dof), (chi2, dof)
    # the tail outside the tested cells is small and must stay small
    assert obs[~big].sum() <= max(20, 3 * exp[~big].sum())


def test_walk_conditioning_matters():
    """The same draft logits with a different previous token give a different law at
    slot 1: a walk that ignored the Markov head would fail the chain-rule test above."""
    draft, W1, W2t = _tiny(8)
    l0 = dspark.log_softmax(draft[0, 1].astype(np.float64) + dspark.markov_bias(W1, W2t, 0)[0])
    l1 = dspark.log_softmax(draft[0, 1].astype(np.float64) + dspark.markov_bias(W1, W2t, 1)[0])
    assert np.max(np.abs(np.exp(l0) - np.exp(l1))) > 0.05


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_greedy_walk_is_the_low_temperature_limit(seed):
    rng = np.random.default_rng(50 + seed)
    B, k, V = 5, 4, 50
    draft = (rng.standard_normal((B, k, V)) * 3.0).astype(np.float32)
    top = np.argmax(draft, axis=-1)
    for b in range(B):
        for j in range(k):
            draft[b, j, top[b, j]] += 6.0      # a clear leader so the bias cannot reorder it
    W1 = _bf16(rng.standard_normal((V, 32)) * 0.02)
    W2t = _bf16(rng.standard_normal((V, 32)) * 0.02)
    anchor = rng.integers(0, V, size=B)
    g = dspark.draft_walk(draft, "f32", np.zeros(B, np.float32), anchor, W1, W2t, seed=seed)
    s = dspark.draft_walk(draft, "f32", np.full(B, 1e-3, np.float32), anchor, W1, W2t, seed=seed)
    assert np.array_equal(g["tokens"], s["tokens"])
    assert np.array_equal(g["tokens"], top.astype(np.int32))


def test_walk_ragged_and_seed_dependence():
    draft, W1, W2t = _tiny(9, V=40, k=4)
    draft = np.repeat(draft, 3, axis=0)
    r1 = dspark.draft_walk(draft, "f32", np.ones(3, np.float32), np.array([1, 2, 3]), W1, W2t,
                           num_drafts=np.array([0, 2, 4]), seed=1, step=0)
    assert r1["tokens"][0].tolist() == [-1] * 4 and r1["tokens"][1, 2:].tolist() == [-1, -1]
    assert np.all(r1["tokens"][2] >= 0)
    draws = {tuple(dspark.draft_walk(draft[:1], "f32", np.ones(1, np.float32), np.array([1]), W1, W2t,
                                     seed=s, step=0)["tokens"][0]) for s in range(40)}
    assert len(draws) > 10   # different seeds give different walks


def test_walk_same_clocks_every_slot_is_caught(monkeypatch):
    """Reusing slot 0's clocks at every slot correlates the slots' draws: the chain-rule
    test's statistic blows far past its band."""
    from oracle import philox
    draft, W1, W2t = _tiny(7)
    T, anchor = 0.8, 2
    law = _exact_law(draft, W1, W2t, anchor, T)
    monkeypatch.setattr(philox, "walk_purpose", lambda j: philox.WALK_PURPOSE_BASE)
    n = 3000
    counts = dict.fromkeys(law, 0)
    for step in range(n):
        r = dspark.draft_walk(draft, "f32", np.array([T], np.float32), np.array([anchor]), W1, W2t,
                              seed=11, step=step)
        counts[tuple(int(t) for t in r["tokens"][0])] += 1
    keys = sorted(law)
    exp = np.array([law[s] * n for s in keys])
    obs = np.array([counts[s] for s in keys])
    big = exp >= 5
    chi2 = float(np.sum((obs[big] - exp[big]) ** 2 / exp[big]))
    dof = int(big.sum()) - 1
    assert chi2 > dof + 10 * np.sqrt(2 * dof), (chi2, dof)
