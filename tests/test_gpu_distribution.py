"""The GPU's emitted law against the exact law, with no reference to the oracle's
sampling convention: at the tiny configuration (V=16, k=3, four draft blocks each
replicated over 16 streams, so every stream draws its own Philox numbers), 10^5
verify calls per verifier with the step varied.  For fixed drafts x the exact law of
(accepted length s, emitted token y) integrates the accept uniforms out analytically
and draws y from the normalised residual (the bonus distribution at s = gamma) [P1 §4
"Token by token", "Block verification"]; the histogram of the GPU's outputs must pass a
chi-square test against it for every draft block and both verifiers."""
import numpy as np
import pytest
import torch

import workloads
from oracle import dspark as odsp, enumerate as en

pytestmark = pytest.mark.gpu

CALLS = 100_000
REPLICAS = 16


@pytest.fixture(scope="module")
def mod():
    import draft_block_verification_row_amd as m
    m.lib()
    return m


def _exact_law(p_rows, q_rows, x, method):
    gamma = len(x)
    logr = odsp.log_ratios(np.log(p_rows), np.log(q_rows), np.asarray(x, dtype=np.int64))
    P_stop, logP = en.stop_distribution(method, logr, p_rows, q_rows)
    V = p_rows.shape[1]
    law = np.zeros((gamma + 1, V))
    for s in range(gamma + 1):
        w = p_rows[gamma] if s == gamma else odsp.residual_weights(logP[s], p_rows[s], q_rows[s])
        if not np.sum(w) > 0:
            w = p_rows[s]
        law[s] = P_stop[s] * w / np.sum(w)
    return law


def _chi2(counts, expected, min_expected=5.0):
    c, e = counts.ravel().astype(np.float64), expected.ravel()
    big = e >= min_expected
    c2 = np.append(c[big], c[~big].sum())
    e2 = np.append(e[big], e[~big].sum())
    keep = e2 > 0
    return float(np.sum((c2[keep] - e2[keep]) ** 2 / e2[keep])), int(keep.sum() - 1)


@pytest.mark.parametrize("method", ["tokenwise", "block"])
def test_emitted_law_matches_exact_law(mod, method):
    base = workloads.make("c1")
    B0, k, V = base.B, base.k, base.V
    B = B0 * REPLICAS
    dev = torch.device("cuda:0")
    target = torch.from_numpy(np.tile(base.target, (REPLICAS, 1, 1))).to(dev)
    draft = torch.from_numpy(np.tile(base.draft, (REPLICAS, 1, 1))).to(dev)
    toks = torch.from_numpy(np.tile(base.draft_tokens.astype(np.int32), (REPLICAS, 1))).to(dev)
    fn = mod.verify_block if method == "block" else mod.verify_tokenwise
    ws = torch.empty(mod.workspace_bytes(B, k, V, mod.DSPARK_F32), dtype=torch.uint8, device=dev)
    acc_all = torch.empty(CALLS, B, dtype=torch.int32, device=dev)
    out_all = torch.empty(CALLS, B, k + 1, dtype=torch.int32, device=dev)
    for i in range(CALLS):
        fn(target, draft, toks, seed=11, step=i, workspace=ws, out=(acc_all[i], out_all[i], None))
    torch.cuda.synchronize()
    acc = acc_all.cpu().numpy()
    out = out_all.cpu().numpy()
    for b0 in range(B0):
        p_rows = np.exp(odsp.log_softmax(odsp.widen(base.target[b0], "f32")))
        q_rows = np.exp(odsp.log_softmax(odsp.widen(base.draft[b0], "f32")))
        law = _exact_law(p_rows, q_rows, base.draft_tokens[b0], method)
        cols = np.arange(b0, B, B0)                      # the stream's replicas
        s = acc[:, cols].ravel()
        y = out[:, cols, :][np.arange(CALLS)[:, None], np.arange(len(cols))[None, :], acc[:, cols]].ravel()
        counts = np.zeros_like(law)
        np.add.at(counts, (s, y), 1)
        # the accepted drafts are the drafts themselves
        for r in range(len(cols)):
            for m in range(1, k + 1):
                sel = acc[:, cols[r]] >= m
                assert np.all(out[sel, cols[r], m - 1] == base.draft_tokens[b0, m - 1])
        chi2, dof = _chi2(counts, counts.sum() * law)
        bound = dof + 5.0 * np.sqrt(2.0 * dof)
        print(f"[T4 {method} block {b0}] samples={int(counts.sum())} chi2={chi2:.1f} dof={dof} "
              f"P(s)={np.round(counts.sum(axis=1) / counts.sum(), 4).tolist()} "
              f"exact={np.round(law.sum(axis=1), 4).tolist()}", flush=True)
        assert chi2 < bound, (b0, chi2, dof)
