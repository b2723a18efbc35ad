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
prefix survival a[b, j] = c[b, 0] * ... * c[b, j] (fp64, left to right).  The
pages leave the arithmetic of the expected-token sums open; here each survival
is clipped to [0, 1] and rounded to the nearest multiple of 2^-40 (ties to
even), and E is accumulated in those units as an exact integer, so neither the
ranking nor any sum depends on the order of additions (the resolution, 2^-40
tokens, is far below anything the ratio can resolve).  Candidates are taken in
descending rounded survival, ties by slot j then stream b; since a never grows
along a stream, every prefix of that order holds, for each stream, a prefix of
its slots.  Taking the first m candidates puts B + m tokens in the verify batch
(each stream's n_b drafts plus its own target position) and expects
E(m) = B + (sum of those m survivals) accepted tokens.  The scheduler keeps the
m with the largest E(m) / verify_ms[B + m] (fp64 division, E exact in fp64),
the smallest m on ties.  With B = 1 this is the per-stream adaptive choice.

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


FIXED_BITS = 40   # survivals are counted in units of 2^-40 tokens


def fixed_survival(a: np.ndarray) -> np.ndarray:
    """round(clip(a, 0, 1) * 2^40) as exact integers (NaN counts as 0)."""
    a = np.where(np.isnan(a), 0.0, np.clip(a, 0.0, 1.0))
    return np.rint(a * float(1 << FIXED_BITS)).astype(np.int64)


def greedy_order(a_fixed: np.ndarray):
    """All (b, j) pairs by descending rounded survival, ties by j then b."""
    B, k = a_fixed.shape
    pairs = [(b, j) for b in range(B) for j in range(k)]
    return sorted(pairs, key=lambda bj: (-int(a_fixed[bj[0], bj[1]]), bj[1], bj[0]))


def batch_schedule(c: np.ndarray, verify_ms) -> dict:
    """Per-stream draft counts n[B] chosen jointly for one verify batch.

    verify_ms[t] is the cost of a verify batch of t tokens; it must cover
    t = B .. B (k + 1).  Returns n, the chosen m = sum n, E(m), every ratio,
    the survivals (fp64 and rounded) and the margin (best - runner-up) / best.
    """
    c = np.asarray(c, dtype=np.float32)
    B, k = c.shape
    ms = np.asarray(verify_ms, dtype=np.float32).astype(np.float64)
    if len(ms) < B * (k + 1) + 1:
        raise ValueError("verify_ms must cover B (k + 1) tokens")
    a = prefix_survival_rows(c)
    aq = fixed_survival(a)
    order = greedy_order(aq)
    units = [B << FIXED_BITS]                    # exact integers
    for (b, j) in order:
        units.append(units[-1] + int(aq[b, j]))
    E = [u / float(1 << FIXED_BITS) for u in units]   # exact: below 2^53 units
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
    return dict(n=n, m=m_best, expected=E[m_best], ratio=np.array(ratio), a=a, a_fixed=aq,
                margin=float(margin))


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
