"""Small hand-built problems for the oracle's pin tests.

A target distribution p is planted exactly (up to fp32 rounding of log p) by
taking d = V, W = I and h = log p, so the target logits are log p.
"""
import numpy as np


def identity_problem(p_rows, q_rows, drafts):
    """p_rows: [B, gamma+1, V] target probabilities; q_rows: [B, gamma, V];
    drafts: int [B, gamma].  Returns (W, h, draft, q_hat) for oracle.run."""
    p_rows = np.asarray(p_rows, dtype=np.float64)
    B, T1, V = p_rows.shape
    with np.errstate(divide="ignore"):
        logp = np.log(p_rows)
    logp = np.where(np.isfinite(logp), logp, -1000.0)
    W = np.eye(V, dtype=np.float32)
    h = logp.astype(np.float32)
    q = np.asarray(q_rows, dtype=np.float32).reshape(B, T1 - 1, V)
    d = np.asarray(drafts, dtype=np.int32).reshape(B, T1 - 1)
    return W, h, d, q


def chi2_pvalue(counts, probs):
    from scipy.stats import chisquare

    counts = np.asarray(counts, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    keep = probs > 0
    assert counts[~keep].sum() == 0, "a zero-probability token was emitted"
    exp = probs[keep] / probs[keep].sum() * counts.sum()
    return chisquare(counts[keep], exp).pvalue
