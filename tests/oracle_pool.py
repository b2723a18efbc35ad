"""Oracle steps of one named workload in parallel worker processes.

Each worker is a fresh interpreter (spawn) that rebuilds the workload from its name
and seed, so no large array crosses a pipe and no worker inherits GPU state; the
workers import numpy, the workload generators and the oracle only.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

_CACHE = {}


def _single_threaded():
    # one BLAS thread per worker: the workers already fill the cores
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"


def _workload(name, B):
    import workloads
    key = (name, B)
    if key not in _CACHE:
        _CACHE[key] = workloads.make(name, B=B)
    return _CACHE[key]


def _one(args):
    name, B, method, step, num_drafts = args
    from oracle import dspark as odsp
    wl = _workload(name, B)
    nd = wl.num_drafts if num_drafts is None else num_drafts
    r = odsp.verify(wl.target, wl.draft, wl.dtype, wl.draft_tokens, wl.temperature, wl.anchor, wl.W1, wl.W2t,
                    num_drafts=nd, seed=wl.seed, step=step, method=method)
    return {k: r[k] for k in ("accepted_len", "out_tokens", "diag", "margin_accept", "margin_sample")}


def workers() -> int:
    return max(1, min(8, (os.cpu_count() or 1) - 1))


def oracle_steps(name, method, steps, B=None, num_drafts=None):
    """oracle.verify of workload ``name`` (optionally with B streams) at every step."""
    steps = list(steps)
    jobs = [(name, B, method, s, num_drafts) for s in steps]
    n = min(workers(), len(jobs))
    if n <= 1:
        return [_one(j) for j in jobs]
    with ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"), initializer=_single_threaded) as ex:
        return list(ex.map(_one, jobs))



def _walk(args):
    name, step = args
    from oracle import dspark as odsp
    wl = _workload(name, None)
    o = odsp.draft_walk(wl.draft, wl.dtype, wl.temperature, wl.anchor, wl.W1, wl.W2t, num_drafts=wl.num_drafts,
                        seed=wl.seed, step=step)
    return {k: o[k] for k in ("tokens", "logq", "margin")}


def walk_steps(name, steps):
    """oracle.draft_walk of workload ``name`` at every step, one worker per step."""
    steps = list(steps)
    jobs = [(name, s) for s in steps]
    n = min(workers(), len(jobs))
    if n <= 1:
        return [_walk(j) for j in jobs]
    with ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"), initializer=_single_threaded) as ex:
        return list(ex.map(_walk, jobs))
