"""Plain fp64 CPU reference of the DSpark verify sampler.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): slow, obviously correct
numpy in float64, one stream at a time, following the pages' statement of each
step.  Nothing here is blocked, fused or reordered beyond what the definitions
say; library routines (``np.exp``, ``np.sum``, ``@``) serve as single steps.

Sources (page titles; sections as headed on each page):
  [P1] "MTP, DSpark and Block Verification, Explained" (al-engr.com)
  [P2] "MTP Heads and Confidence Heads" (naphjohn.github.io LLM-blog, ep7)
  [P3] "Teaching the Speculator What a Draft Costs" (al-engr.com)

Notation (0-based).  A stream carries gamma drafts x_0..x_{gamma-1}.  q_j is
the drafter's distribution for slot j (after the Markov bias), p_j the
target's distribution at slot j conditioned on x_{<j}; p_gamma is the bonus
position.  Readings of points the pages leave open are marked READING.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import philox

NEAR_MARGIN = 1e-6      # decisions closer than this to their threshold are "near"


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits -> float64, exactly.  bf16 arrives as uint16 bit patterns."""
    if dtype == "bf16":
        bits = np.asarray(arr, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def log_softmax(x: np.ndarray) -> np.ndarray:
    """log softmax over the last axis, fp64: x - max - log(sum(exp(x - max)))."""
    m = np.max(x, axis=-1, keepdims=True)
    return x - m - np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True))


# ----------------------------------------------------------------------------
# DSpark Markov head  [P2 §6 "Why the Markov Head Helps"; P1 §3 "The Markov
# fix-up" and Figure 2]
# ----------------------------------------------------------------------------
def markov_bias(W1: np.ndarray, W2t: np.ndarray, prev) -> np.ndarray:
    """Low-rank logit bias B = W1 @ W2 read at the previous token: bias[v] = W1[prev] . W2[:, v].

    W1 [V, R] and W2t [V, R] (W2t[v, r] = W2[r, v]) are bf16 bit patterns
    (uint16) or already-widened float64 copies of them.
    prev < 0 gives a zero row (READING: slot 0 with no prior token, Figure 2 of P1).
    """
    prev = np.atleast_1d(np.asarray(prev, dtype=np.int64))
    w1 = W1 if W1.dtype == np.float64 else widen(W1, "bf16")
    w2 = W2t if W2t.dtype == np.float64 else widen(W2t, "bf16")
    out = np.zeros((prev.size, w2.shape[0]), dtype=np.float64)
    for i, t in enumerate(prev):
        if t >= 0:
            out[i] = w2 @ w1[t]
    return out


def draft_prev_tokens(anchor: int, x: np.ndarray, gamma: int) -> np.ndarray:
    """prev_0 = anchor (the last accepted token), prev_j = x_{j-1}: the Markov walk's conditioning."""
    return np.concatenate([[int(anchor)], np.asarray(x[: max(gamma - 1, 0)], dtype=np.int64)])[:gamma]


def draft_scaled_logits(d: np.ndarray, W1, W2t, prev, T: float) -> np.ndarray:
    """(d + W1[prev] . W2) / T: the drafter's logits with the Markov bias of their previous
    tokens, then divided by the temperature (READING: the bias belongs to the drafter's
    logits, the temperature to the sampler).  d [rows, V], prev [rows]; W1 None: no bias."""
    if W1 is not None:
        d = d + markov_bias(W1, W2t, prev)
    return d / T


# ----------------------------------------------------------------------------
# accept tests  [P1 §4 "Token by token", "Block verification"]
# ----------------------------------------------------------------------------
def log_ratios(logp_rows: np.ndarray, logq_rows: np.ndarray, x: np.ndarray) -> np.ndarray:
    """log r_j = log p_j(x_j) - log q_j(x_j), j < gamma."""
    g = len(x)
    return np.array([logp_rows[j, x[j]] - logq_rows[j, x[j]] for j in range(g)], dtype=np.float64)


def tokenwise_stop(logr: np.ndarray, u: np.ndarray):
    """Token-wise rule (Leviathan et al.): draft j is kept iff u_j <= min(1, r_j).

    Returns t = first rejected slot (or gamma) and the decision margin
    min_{j <= t, j < gamma} |u_j - min(1, r_j)|.
    """
    gamma = len(logr)
    margin = math.inf
    for j in range(gamma):
        thr = 1.0 if logr[j] >= 0 else math.exp(logr[j])
        margin = min(margin, abs(u[j] - thr))
        if not u[j] <= thr:
            return j, margin
    return gamma, margin


def block_prefix(logr: np.ndarray) -> np.ndarray:
    """Clipped joint prefix ratio, log P_i for i = 0..gamma.

    READING: the page's prefix_joint is the running product of p/q clipped at 1
    after every slot, P_0 = 1, P_i = min(1, P_{i-1} r_{i-1}) (Sun et al.); the
    unclipped product does not keep the output distribution.
    """
    gamma = len(logr)
    logP = np.zeros(gamma + 1, dtype=np.float64)
    for i in range(1, gamma + 1):
        logP[i] = min(0.0, logP[i - 1] + logr[i - 1])
    return logP


def residual_weights(logP: float, p_row: np.ndarray, q_row: np.ndarray) -> np.ndarray:
    """Unnormalised residual max(0, P p - q) over the vocabulary."""
    return np.maximum(0.0, math.exp(logP) * p_row - q_row)


def block_thresholds(logP: np.ndarray, p_rows: np.ndarray, q_rows: np.ndarray):
    """Residual masses R_i and thresholds h_i of block verification.

    For i = 1..gamma-1: R_i = sum_v max(0, P_i p_i(v) - q_i(v)),
    h_i = R_i / (R_i + 1 - P_i), and h_i = 1 when P_i = 1 (READING: the 0/0 case);
    the last slot uses h_gamma = P_gamma.  Index alignment (READING): R_i and
    h_i use the distributions of slot i, i.e. after i drafts were accepted.
    Arrays have length gamma + 1 with NaN where undefined.
    """
    gamma = len(logP) - 1
    R = np.full(gamma + 1, np.nan)
    h = np.full(gamma + 1, np.nan)
    for i in range(1, gamma):
        R[i] = float(np.sum(residual_weights(logP[i], p_rows[i], q_rows[i])))
        if logP[i] == 0.0:
            h[i] = 1.0
        else:
            one_minus_P = -math.expm1(logP[i])
            h[i] = R[i] / (R[i] + one_minus_P)
    if gamma >= 1:
        h[gamma] = math.exp(logP[gamma])
    return R, h


def block_stop(h: np.ndarray, u: np.ndarray):
    """tau = the last i in 1..gamma with u_{i-1} <= h_i, else 0.

    Margin: min |u_{i-1} - h_i| over the tests that decide tau (i = gamma down to max(tau, 1)).
    """
    gamma = len(h) - 1
    margin = math.inf
    for i in range(gamma, 0, -1):
        margin = min(margin, abs(u[i - 1] - h[i]))
        if u[i - 1] <= h[i]:
            return i, margin
    return 0, margin


# ----------------------------------------------------------------------------
# sampler: exponential race over the vocabulary
# ----------------------------------------------------------------------------
def race_sample(w: np.ndarray, seed: int, b: int, step: int, purpose: int = philox.PURPOSE_SAMPLE):
    """Draw Y with P(Y = v) = w_v / sum(w) by an exponential race.

    READING (the pages only say "sample from the normalized residual"): every id v
    with w_v > 0 gets an Exp(1) clock E_v (``philox.race_clocks``, one per id, keyed by
    stream b, ``purpose`` and ``step``) and Y is the id with the largest w_v / E_v,
    the lowest id on ties.  The first of independent exponential clocks of rates w_v
    to ring is v with probability w_v / sum(w), which is the normalised law.
    Returns (Y, margin) with margin = 1 - second best / best score (1 if only one
    id has weight), or (-1, 0) if no id has weight.
    """
    w = np.asarray(w, dtype=np.float64)
    cand = w > 0
    if not np.any(cand):
        return -1, 0.0
    E = philox.race_clocks(seed, b, np.arange(w.shape[0]), purpose, step)
    score = np.where(cand, w / E, -np.inf)
    best = int(np.argmax(score))           # np.argmax: the first (lowest) id of equal maxima
    if np.count_nonzero(cand) == 1:
        return best, 1.0
    second = float(np.max(np.delete(score, best)))
    return best, float(1.0 - second / score[best])


# ----------------------------------------------------------------------------
# one stream, one call
# ----------------------------------------------------------------------------
def verify_stream(tl: np.ndarray, dl: np.ndarray, x: np.ndarray, gamma: int, T: float,
                  anchor: int, W1, W2t, seed: int, b: int, step: int, method: str) -> dict:
    """Verify one stream's block.

    tl [gamma+1, V] and dl [gamma, V] are raw fp64 logits (target rows 0..gamma,
    draft rows 0..gamma-1).  READING (temperature): the Markov bias is added to
    the raw draft logits, then both target and biased draft logits are divided
    by T before the softmax.  Steps [P1 §4]: softmax both sides, accept tests,
    then sample the emitted token from the residual of the stop slot, or from
    the bonus position when every draft survives [P1 §1; Glossary "Verify step"].
    """
    logp = log_softmax(tl[: gamma + 1] / T)
    if gamma > 0:
        logq = log_softmax(draft_scaled_logits(dl[:gamma], W1, W2t, draft_prev_tokens(anchor, x, gamma), T))
    else:
        logq = np.zeros((0, tl.shape[1]))
    p = np.exp(logp)
    q = np.exp(logq)
    logr = log_ratios(logp, logq, x[:gamma])
    u = philox.accept_uniforms(seed, b, gamma, step)
    logP = block_prefix(logr)
    diag = np.full((gamma + 1, 5), np.nan)
    for j in range(gamma):
        diag[j, 0] = logp[j, x[j]]
        diag[j, 1] = logq[j, x[j]]
    diag[:, 2] = np.exp(logP)

    if method == "tokenwise":
        s, m_acc = tokenwise_stop(logr, u)
        logP_s = 0.0
    elif method == "block":
        R, h = block_thresholds(logP, p, q)
        diag[:, 3] = R
        diag[:, 4] = h
        s, m_acc = block_stop(h, u)
        logP_s = logP[s]
    else:
        raise ValueError(method)

    degenerate = False
    if s == gamma:
        w = p[gamma]
    else:
        w = residual_weights(logP_s, p[s], q[s])
        if not np.sum(w) > 0:
            # READING: an all-zero residual cannot occur in exact arithmetic on
            # the path that reaches it; should rounding produce one, draw from p_s.
            w = p[s]
            degenerate = True
    Y, m_smp = race_sample(w, seed, b, step)
    return dict(s=s, Y=Y, diag=diag, margin_accept=m_acc, margin_sample=m_smp,
                degenerate=degenerate, logr=logr, u=u)


def greedy_stream(tl: np.ndarray, x: np.ndarray, gamma: int) -> dict:
    """Temperature 0 [P1 §4 "Greedy is a different code path"]: a draft is kept iff it
    equals the target's argmax at its slot; the first mismatch stops the block and the
    emitted token is the target's argmax there (the bonus position's argmax when every
    draft is kept).  READING: ties go to the lowest vocabulary id.  The decisions are
    exact comparisons, so no margin applies; log-probabilities and the block quantities
    are undefined at T = 0 (NaN in diag).
    """
    am = [int(np.argmax(tl[j])) for j in range(gamma + 1)]   # np.argmax: first of equal maxima
    s = gamma
    for j in range(gamma):
        if am[j] != int(x[j]):
            s = j
            break
    return dict(s=s, Y=am[s], diag=np.full((gamma + 1, 5), np.nan), margin_accept=np.inf,
                margin_sample=np.inf, degenerate=False)


def verify(target, draft, dtype: str, draft_tokens, temperature=None, anchor=None,
           W1=None, W2t=None, num_drafts=None, seed: int = 0, step: int = 0,
           method: str = "block") -> dict:
    """Both verifiers over B streams.

    target [B, k+1, V], draft [B, k, V] (fp32 or bf16 bits), draft_tokens [B, k],
    temperature [B] (None = 1; a stream with T = 0 takes the greedy branch whatever
    the method, as the pages' sampler does), anchor [B] (None = -1), num_drafts [B]
    (None = k; READING: ragged gamma_b reads rows 0..gamma_b only).
    Returns accepted_len [B], out_tokens [B, k+1] (x_0..x_{s-1}, Y, then -1),
    diag [B, k+1, 5] = (log p(x_j), log q(x_j), P_j, R_j, h_j), and margins.
    """
    target = np.asarray(target)
    B, k1, V = target.shape
    k = k1 - 1
    x_all = np.asarray(draft_tokens, dtype=np.int64).reshape(B, k)
    T_all = np.ones(B) if temperature is None else np.asarray(temperature, dtype=np.float32).astype(np.float64)
    a_all = np.full(B, -1) if anchor is None else np.asarray(anchor, dtype=np.int64)
    g_all = np.full(B, k) if num_drafts is None else np.asarray(num_drafts, dtype=np.int64)
    if W1 is not None:
        W1 = widen(W1, "bf16")
        W2t = widen(W2t, "bf16")
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, k + 1), -1, dtype=np.int32)
    diag = np.full((B, k + 1, 5), np.nan)
    m_acc = np.full(B, np.inf)
    m_smp = np.full(B, np.inf)
    degen = np.zeros(B, dtype=bool)
    for b in range(B):
        gamma = int(g_all[b])
        tl = widen(target[b, : gamma + 1], dtype)
        dl = widen(np.asarray(draft)[b, :gamma], dtype) if gamma > 0 else np.zeros((0, V))
        if T_all[b] == 0.0:
            r = greedy_stream(tl, x_all[b], gamma)
        else:
            r = verify_stream(tl, dl, x_all[b], gamma, float(T_all[b]), int(a_all[b]), W1, W2t,
                              seed, b, step, method)
        s = r["s"]
        acc[b] = s
        out[b, :s] = x_all[b, :s]
        out[b, s] = r["Y"]
        diag[b, : gamma + 1] = r["diag"]
        m_acc[b] = r["margin_accept"]
        m_smp[b] = r["margin_sample"]
        degen[b] = r["degenerate"]
    return dict(accepted_len=acc, out_tokens=out, diag=diag, margin_accept=m_acc,
                margin_sample=m_smp, degenerate=degen)


# ----------------------------------------------------------------------------
# the drafter's Markov walk  [P2 §6 "Why the Markov Head Helps"; P1 §3 "The Markov
# fix-up" and Figure 2]
# ----------------------------------------------------------------------------
def draft_walk(draft, dtype: str, temperature=None, anchor=None, W1=None, W2t=None, num_drafts=None,
               seed: int = 0, step: int = 0) -> dict:
    """Draw the drafts slot by slot from the drafter with its Markov head:
    x_j ~ softmax((d_j + W1[x_{j-1}] . W2) / T), x_{-1} = the anchor token.

    The drafter's logits d_j [B, k, V] come from its parallel pass; the Markov head
    is what makes slot j depend on the token drawn at slot j-1.  T = 0 takes the
    largest biased logit (first id on ties).  Draws use the exponential race with the
    slot's own clocks (READING: Philox purpose ``philox.walk_purpose(j)`` = 16 + j, apart
    from the verifiers' words).  Returns tokens [B, k] (-1 past
    gamma_b), log q_j(x_j) [B, k] and the smallest decision margin per stream:
    the race margin, or for T = 0 (x_1 - x_2) / (|x_1| + 1) over the two largest
    biased logits.
    """
    draft = np.asarray(draft)
    B, k, V = draft.shape
    T_all = np.ones(B) if temperature is None else np.asarray(temperature, dtype=np.float32).astype(np.float64)
    a_all = np.full(B, -1) if anchor is None else np.asarray(anchor, dtype=np.int64)
    g_all = np.full(B, k) if num_drafts is None else np.asarray(num_drafts, dtype=np.int64)
    if W1 is not None:
        W1 = widen(W1, "bf16")
        W2t = widen(W2t, "bf16")
    toks = np.full((B, k), -1, dtype=np.int32)
    logq = np.full((B, k), np.nan)
    margin = np.full(B, np.inf)
    for b in range(B):
        prev = int(a_all[b])
        for j in range(int(g_all[b])):
            d = widen(draft[b, j], dtype)
            if W1 is not None:
                d = d + markov_bias(W1, W2t, [prev])[0]
            T = float(T_all[b])
            if T == 0.0:
                order = np.argsort(-d, kind="stable")
                x = int(np.argmax(d))
                m = (d[order[0]] - d[order[1]]) / (abs(d[order[0]]) + 1.0) if V > 1 else np.inf
            else:
                ls = log_softmax(d / T)
                x, m = race_sample(np.exp(ls), seed, b, step, philox.walk_purpose(j))
                logq[b, j] = ls[x]
            toks[b, j] = x
            margin[b] = min(margin[b], m)
            prev = x
    return dict(tokens=toks, logq=logq, margin=margin)


# ----------------------------------------------------------------------------
# confidence head and adaptive verification  [P2 §7-9; P3 "The controller,
# and the table it reads from"; P1 §6 "The arithmetic you need before tuning k"]
# ----------------------------------------------------------------------------
def confidence(hidden_bits: np.ndarray, w_bits: np.ndarray, bias: float) -> np.ndarray:
    """c = sigmoid(w . h + b): hidden -> Linear -> sigmoid, per draft slot [P2 §7]."""
    h = widen(hidden_bits, "bf16")
    w = widen(w_bits, "bf16")
    z = h @ w + float(np.float32(bias))
    return 1.0 / (1.0 + np.exp(-z))


def prefix_survival(c: np.ndarray) -> np.ndarray:
    """a_j = prod_{i<=j} c_i, the chance the first j+1 drafts all survive [P2 §9]."""
    return np.cumprod(np.asarray(c, dtype=np.float64), axis=-1)


def tokens_per_step(a) -> float:
    """1 + sum_p a_p: the +1 is the token the target always samples [P1 §6]."""
    return 1.0 + float(np.sum(a))


def marginal_acceptance(a) -> np.ndarray:
    """a_p / a_{p-1} with a_0 := 1 [P1 §6]."""
    a = np.asarray(a, dtype=np.float64)
    return a / np.concatenate([[1.0], a[:-1]])


def adaptive_choice(a_row: np.ndarray, verify_ms: np.ndarray):
    """n* = argmax_{n in 0..k} (1 + sum_{j<n} a_j) / verify_ms[n + 1], smallest n on ties.

    READING: verify_ms is indexed by the token count of one stream's verify,
    n drafts plus the target's own position [P3: verify_ms[num_tokens]].
    Returns (n*, margin = (best - runner-up) / best).
    """
    k = len(a_row)
    ms = np.asarray(verify_ms, dtype=np.float32).astype(np.float64)
    ratio = np.array([(1.0 + float(np.sum(a_row[:n]))) / ms[n + 1] for n in range(k + 1)])
    n = int(np.argmax(ratio))
    if k == 0:
        return n, 1.0
    second = np.max(np.delete(ratio, n))
    return n, float((ratio[n] - second) / ratio[n])


def adaptive_k(hidden_bits, w_bits, bias: float, verify_ms) -> dict:
    """Per stream: c -> a -> n (the count of drafts to verify)."""
    c = confidence(hidden_bits, w_bits, bias)
    a = prefix_survival(c)
    B = c.shape[0]
    n = np.zeros(B, dtype=np.int32)
    margin = np.zeros(B)
    for b in range(B):
        n[b], margin[b] = adaptive_choice(a[b], verify_ms)
    return dict(n=n, c=c, a=a, margin=margin)
