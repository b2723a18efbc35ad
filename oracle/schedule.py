"""Batch-level draft scheduler and the online verify-cost table (fp64, plain Python).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources (page titles; sections as headed on each page):
  [P2] "MTP Heads and Confidence Heads" (naphjohn.github.io LLM-blog, ep7),
       §9 "Why It Is Called Prefix Survival Probability": the scheduler takes
       draft positions in descending prefix survival and cuts the tail once the
       expected accepted tokens stop paying for themselves.
  [P3] "Teaching the Speculator What a Draft Costs" (al-engr.com), "The
       controller, and the table it reads from" (a cost table indexed by the
       verify batch's token count) and "What we changed" (a live table: timed
       real verify steps filed by token count, rebuilt at a fixed cadence from
       the boot curve with live medians laid over it; window 32, at least 3
       samples, rebuilt every 32 observations).

READING (batch scheduler).  Candidates are the (stream b, slot j) pairs with
prefix survival a[b, j] = c[b, 0] * ... * c[b, j] (fp64, multiplied left to
right).  They are taken in descending survival, ties by slot j then stream b;
since a never grows along a stream (c <= 1), every leading part of that order
holds, for each stream, a prefix of its slots.  Taking the first m candidates
puts B + m tokens in the verify batch (each stream's n_b drafts plus its own
target position) and expects E(m) = B + the sum of those m survivals accepted
tokens, added one at a time in rank order in fp64.  The scheduler keeps the m
with the largest E(m) / verify_ms[B + m] (fp64), the smallest m on ties.  With
B = 1 this is the per-stream adaptive choice.

READING (online table).  Observations (token count t, milliseconds) are filed
in arrival order.  The table in force is the boot table until the first
rebuild; a rebuild happens right after every ``rebuild_every``-th observation
and sets, for each t, the median of the last ``window`` observations filed
under t when there are at least ``min_samples`` of them, else the boot value.
The median of an even count is the mean of the two middle values.  Table
entries are float32 (as the boot table is); medians are taken in fp64 and
rounded once.
"""
from __future__ import annotations

import numpy as np


def prefix_survival_rows(c: np.ndarray) -> np.ndarray:
    """a[b, j] = prod_{i<=j} c[b, i], multiplied left to right in fp64 [P2 §9]."""
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    a = np.empty_like(c)
    for b in range(c.shape[0]):
        run = 1.0
        for j in range(c.shape[1]):
            run = run * c[b, j]
            a[b, j] = run
    return a


def greedy_order(a: np.ndarray):
    """All (b, j) pairs by descending survival, ties by slot j then stream b."""
    B, k = a.shape
    pairs = [(b, j) for b in range(B) for j in range(k)]
    return sorted(pairs, key=lambda bj: (-float(a[bj[0], bj[1]]), bj[1], bj[0]))


def batch_schedule(c: np.ndarray, verify_ms) -> dict:
    """Per-stream draft counts n[B] chosen jointly for one verify batch.

    verify_ms[t] is the cost of a verify batch of t tokens; it must cover
    t = B .. B (k + 1).  Returns n, the chosen m = sum n, E(m), every ratio, the
    survivals, the margin (best - runner-up) / best of the ratio, and cut_gap, the
    survival of the last candidate taken minus that of the first one left out
    (inf when m is 0 or B k): how finely the ranking must resolve survivals for the
    same streams to receive the m drafts.
    """
    c = np.asarray(c, dtype=np.float32)
    B, k = c.shape
    ms = np.asarray(verify_ms, dtype=np.float32).astype(np.float64)
    if len(ms) < B * (k + 1) + 1:
        raise ValueError("verify_ms must cover B (k + 1) tokens")
    a = prefix_survival_rows(c)
    order = greedy_order(a)
    E = [float(B)]
    for (b, j) in order:
        E.append(E[-1] + float(a[b, j]))
    ratio = [E[m] / ms[B + m] for m in range(len(E))]
    m_best = 0
    for m in range(1, len(ratio)):
        if ratio[m] > ratio[m_best]:
            m_best = m
    n = np.zeros(B, dtype=np.int32)
    for (b, j) in order[:m_best]:
        n[b] += 1
    others = [r for m, r in enumerate(ratio) if m != m_best]
    margin = (ratio[m_best] - max(others)) / ratio[m_best] if others else 1.0
    cut_gap = (float(a[order[m_best - 1]]) - float(a[order[m_best]])) if 0 < m_best < len(order) else np.inf
    return dict(n=n, m=m_best, expected=E[m_best], ratio=np.array(ratio), a=a, margin=float(margin),
                cut_gap=cut_gap)


def _median(values) -> float:
    s = sorted(float(v) for v in values)
    h = len(s) // 2
    return s[h] if len(s) % 2 else (s[h - 1] + s[h]) / 2.0


def online_table(boot_ms, observations, window: int = 32, min_samples: int = 3, rebuild_every: int = 32):
    """The table in force after each observation [P3 "What we changed"].

    observations: sequence of (tokens, ms).  An observation whose token count
    lies outside the table is dropped: it is neither filed nor counted.
    Returns (final table as float32, list of tables in force after each
    observation).
    """
    boot = np.asarray(boot_ms, dtype=np.float32).copy()
    live = {}
    table = boot.copy()
    history = []
    count = 0
    for (t, ms) in observations:
        t = int(t)
        if 0 <= t < len(boot):
            count += 1
            live.setdefault(t, []).append(np.float32(ms))
            live[t] = live[t][-window:]
            if count % rebuild_every == 0:
                table = boot.copy()
                for tt, vals in live.items():
                    if len(vals) >= min_samples:
                        table[tt] = np.float32(_median(vals))
        history.append(table.copy())
    return table, history
