"""Shared test helpers: upload a workload, run the HIP path, run the oracle, compare.

Comparison rule.  Probabilities (diag) match within the stated tolerances.
Accepted lengths and emitted tokens are bit-exact, except for streams where the
oracle's margin to a deciding threshold is below NEAR (1e-6); those are counted
and reported, not compared.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import dspark as odsp

NEAR = 1e-6
TOL_LOGPROB = 1e-5     # |d log p(x)|, |d log q(x)|  (~1e-5 relative on the probability)
TOL_P_REL = 1e-5       # |dP| <= 1e-5 P
TOL_R_REL, TOL_R_ABS = 1e-5, 1e-6
TOL_H = 1e-5


def to_dev(wl, device="cuda:0"):
    def t(x, dt=None):
        if x is None:
            return None
        arr = np.ascontiguousarray(x)
        if arr.dtype == np.uint16:
            arr = arr.view(np.int16)
        return torch.from_numpy(arr).to(device)
    d = dict(target=t(wl.target), draft=t(wl.draft), draft_tokens=t(wl.draft_tokens.astype(np.int32)),
             temperature=t(wl.temperature.astype(np.float32)), anchor=t(wl.anchor.astype(np.int32)),
             W1=t(wl.W1), W2t=t(wl.W2t),
             num_drafts=None if wl.num_drafts is None else t(wl.num_drafts.astype(np.int32)))
    return d


def run_gpu(mod, dev, method, seed, step, diag=True, workspace=None):
    fn = mod.verify_block if method == "block" else mod.verify_tokenwise
    acc, toks, dg = fn(dev["target"], dev["draft"], dev["draft_tokens"], num_drafts=dev["num_drafts"],
                       temperature=dev["temperature"], W1=dev["W1"], W2t=dev["W2t"], anchor=dev["anchor"],
                       seed=seed, step=step, diag=diag, workspace=workspace)
    torch.cuda.synchronize()
    return dict(accepted_len=acc.cpu().numpy(), out_tokens=toks.cpu().numpy(),
                diag=None if dg is None else dg.cpu().numpy())


def run_oracle(wl, method, step, num_drafts=None):
    nd = wl.num_drafts if num_drafts is None else num_drafts
    return odsp.verify(wl.target, wl.draft, wl.dtype, wl.draft_tokens, wl.temperature, wl.anchor, wl.W1, wl.W2t,
                       num_drafts=nd, seed=wl.seed, step=step, method=method)


class Tally:
    def __init__(self):
        self.streams = 0
        self.decisions = 0
        self.near = 0
        self.len_mismatch = 0
        self.tok_mismatch = 0
        self.unexplained = []
        self.max_err = dict(lpx=0.0, lqx=0.0, P=0.0, R=0.0, h=0.0)

    def summary(self):
        return (f"streams={self.streams} decisions={self.decisions} near={self.near} "
                f"len_mismatch={self.len_mismatch} tok_mismatch={self.tok_mismatch} "
                f"unexplained={len(self.unexplained)} max_err={self.max_err}")


def compare(g, o, wl, method, tally: Tally, label=""):
    B = len(o["accepted_len"])
    k = wl.k
    gam = np.full(B, k) if wl.num_drafts is None else np.asarray(wl.num_drafts)
    for b in range(B):
        tally.streams += 1
        gamma = int(gam[b])
        tally.decisions += (gamma if method == "tokenwise" else max(gamma, 1)) + 1
        near_acc = o["margin_accept"][b] < NEAR
        near_smp = o["margin_sample"][b] < NEAR
        tally.near += int(near_acc) + int(near_smp)
        la, lo = int(g["accepted_len"][b]), int(o["accepted_len"][b])
        if la != lo:
            tally.len_mismatch += 1
            if not near_acc:
                tally.unexplained.append((label, b, "len", la, lo, o["margin_accept"][b]))
            continue
        if not np.array_equal(g["out_tokens"][b], o["out_tokens"][b]):
            tally.tok_mismatch += 1
            if not (near_smp or near_acc):
                tally.unexplained.append((label, b, "tok", g["out_tokens"][b].tolist(),
                                          o["out_tokens"][b].tolist(), o["margin_sample"][b]))
        if g.get("diag") is None:
            continue
        dg, do = g["diag"][b], o["diag"][b]
        if float(wl.temperature[b]) == 0.0:   # greedy branch: no probabilities on either side
            if not (np.all(np.isnan(dg[: gamma + 1])) and np.all(np.isnan(do[: gamma + 1]))):
                tally.unexplained.append((label, b, "greedy diag not NaN"))
            continue
        for j in range(gamma):
            e1 = abs(dg[j, 0] - do[j, 0])
            e2 = abs(dg[j, 1] - do[j, 1])
            tally.max_err["lpx"] = max(tally.max_err["lpx"], e1)
            tally.max_err["lqx"] = max(tally.max_err["lqx"], e2)
            if not (e1 <= TOL_LOGPROB and e2 <= TOL_LOGPROB):
                tally.unexplained.append((label, b, "logprob", j, dg[j, :2].tolist(), do[j, :2].tolist()))
        for j in range(gamma + 1):
            eP = abs(dg[j, 2] - do[j, 2])
            tally.max_err["P"] = max(tally.max_err["P"], eP / max(do[j, 2], 1e-300))
            if not eP <= TOL_P_REL * do[j, 2] + 1e-300:
                tally.unexplained.append((label, b, "P", j, dg[j, 2], do[j, 2]))
        if method == "block" and not near_acc:
            for j in range(1, gamma + 1):
                if not np.isnan(dg[j, 3]):
                    eR = abs(dg[j, 3] - do[j, 3])
                    tally.max_err["R"] = max(tally.max_err["R"], eR / max(do[j, 3], 1e-12))
                    if not eR <= TOL_R_REL * do[j, 3] + TOL_R_ABS:
                        tally.unexplained.append((label, b, "R", j, dg[j, 3], do[j, 3]))
                if not np.isnan(dg[j, 4]):
                    eh = abs(dg[j, 4] - do[j, 4])
                    tally.max_err["h"] = max(tally.max_err["h"], eh)
                    if not eh <= TOL_H:
                        tally.unexplained.append((label, b, "h", j, dg[j, 4], do[j, 4]))


def assert_clean(tally: Tally, max_near_frac: float = 1e-4):
    """No unexplained difference; near decisions at most max_near_frac of all decisions
    (at least one is let through only while there are fewer than 10^4 decisions)."""
    assert not tally.unexplained, tally.summary() + "\n" + "\n".join(map(str, tally.unexplained[:20]))
    limit = max_near_frac * tally.decisions
    if tally.decisions <= 10000:
        limit = max(1.0, limit)
    assert tally.near <= limit, tally.summary()
