"""Exact enumeration of what one verify step emits, on tiny vocabularies.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Both verifiers claim to leave the output distribution unchanged [P1 §1 "One
token per step": the emitted text is distributed as if the target sampled it
alone; P1 §4 "Block verification": the joint test keeps the output
distribution].  With a vocabulary of a few ids this can be checked exactly:
enumerate every draft block, integrate the accept uniforms out analytically
(they are independent U(0,1)), and add up the probability of each emitted
sequence.  No random numbers are drawn here.

The decision quantities (ratios, clipped prefix P_i, residual masses R_i,
thresholds h_i, residual weights) come from ``oracle.dspark``, so a wrong
formula there breaks the equality checked by :func:`lossless_error`.
"""
from __future__ import annotations

import itertools
from typing import Callable, List

import numpy as np

from . import dspark

Row = Callable[[tuple], np.ndarray]


def stop_distribution(method: str, logr: np.ndarray, p_rows: np.ndarray, q_rows: np.ndarray):
    """P(stop slot = s) for s = 0..gamma with u_j ~ U(0,1) independent.

    token-wise: P(t = j) = prod_{i<j} min(1, r_i) * (1 - min(1, r_j)), P(t = gamma) = prod min(1, r_i).
    block:      P(tau = i) = h_i prod_{j>i} (1 - h_j) for i >= 1, P(tau = 0) = prod_{j>=1} (1 - h_j).
    Also returns log P (all zeros for token-wise, where the residual is max(0, p - q)).
    """
    gamma = len(logr)
    P_stop = np.zeros(gamma + 1)
    if method == "tokenwise":
        acc = np.minimum(1.0, np.exp(np.minimum(logr, 0.0)))
        run = 1.0
        for j in range(gamma):
            P_stop[j] = run * (1.0 - acc[j])
            run *= acc[j]
        P_stop[gamma] = run
        return P_stop, np.zeros(gamma + 1)
    logP = dspark.block_prefix(logr)
    _, h = dspark.block_thresholds(logP, p_rows, q_rows)
    tail = 1.0
    for i in range(gamma, 0, -1):
        P_stop[i] = h[i] * tail
        tail *= (1.0 - h[i])
    P_stop[0] = tail
    return P_stop, logP


def emitted_distribution(p_fn: Row, q_fn: Row, gamma: int, V: int, method: str) -> List[np.ndarray]:
    """E[m][z_0..z_m] = P(the step emits exactly z_0..z_m), m = 0..gamma.

    p_fn(prefix) is the target's distribution after ``prefix``; q_fn(prefix)
    the drafter's.  Draft blocks are enumerated with probability prod q_j(x_j).
    """
    E = [np.zeros((V,) * (m + 1)) for m in range(gamma + 1)]
    for x in itertools.product(range(V), repeat=gamma):
        prob = 1.0
        q_rows = np.zeros((gamma, V))
        for j in range(gamma):
            q_rows[j] = q_fn(x[:j])
            prob *= q_rows[j, x[j]]
        if prob == 0.0:
            continue
        p_rows = np.array([p_fn(x[:j]) for j in range(gamma + 1)])
        logr = dspark.log_ratios(np.log(p_rows), np.log(q_rows), np.asarray(x, dtype=np.int64))
        P_stop, logP = stop_distribution(method, logr, p_rows, q_rows)
        for s in range(gamma + 1):
            if P_stop[s] <= 0.0:
                continue
            if s == gamma:
                w = p_rows[gamma]
            else:
                w = dspark.residual_weights(logP[s], p_rows[s], q_rows[s])
                if not np.sum(w) > 0:
                    w = p_rows[s]
            E[s][tuple(x[:s])] += prob * P_stop[s] * (w / np.sum(w))
    return E


def target_joint(p_fn: Row, gamma: int, V: int) -> List[np.ndarray]:
    """J[m][z_0..z_m] = prod_{j<=m} p_j(z_j | z_<j): the target sampling alone."""
    J = [np.asarray(p_fn(()), dtype=np.float64).copy()]
    for m in range(1, gamma + 1):
        nxt = np.zeros((V,) * (m + 1))
        for pre in itertools.product(range(V), repeat=m):
            nxt[pre] = J[-1][pre] * p_fn(pre)
        J.append(nxt)
    return J


def lossless_error(E: List[np.ndarray], J: List[np.ndarray]) -> float:
    """max_z |sum_m E[m](z_<=m) prod_{j>m} p_j(z_j|z_<j) - prod_j p_j(z_j|z_<j)| over z in V^{gamma+1}.

    The continuation after the emitted prefix is the target's own sampling,
    prod_{j>m} p_j = J[gamma](z) / J[m](z_<=m).
    """
    gamma = len(E) - 1
    full = J[gamma]
    lhs = np.zeros_like(full)
    for m in range(gamma + 1):
        ratio = E[m] / J[m]
        lhs += ratio.reshape(ratio.shape + (1,) * (gamma - m)) * full
    return float(np.max(np.abs(lhs - full)))


def accepted_length_tail(E: List[np.ndarray]) -> np.ndarray:
    """P(accepted length >= m) for m = 0..gamma (emitting z_0..z_m means m drafts were kept)."""
    mass = np.array([np.sum(e) for e in E])
    return np.array([np.sum(mass[m:]) for m in range(len(E))])
