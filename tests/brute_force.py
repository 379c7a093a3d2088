"""Second, independent formulation of the oracle for tiny shapes (a pin, not the oracle).

Builds the full [Hq, N, N] fp64 logits tensor with a -inf causal mask, takes
scipy's softmax along keys, averages over heads, and ranks keys with one
stable argsort per row. Sparse outputs use an explicit [N, N] support mask.
Nothing here is imported from ``oracle/``.
"""
import numpy as np
from scipy.special import softmax


def full_mass(q, k, scale):
    """Returns (P [N,N] head-averaged mass, probs [Hq,N,N], logits [Hq,N,N])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    n, hq, d = q.shape
    hkv = k.shape[1]
    k_rep = np.repeat(k, hq // hkv, axis=1)           # [N, Hq, d]
    logits = scale * np.einsum("ihc,jhc->hij", q, k_rep)
    mask = np.tril(np.ones((n, n), dtype=bool))
    logits = np.where(mask[None], logits, -np.inf)
    probs = softmax(logits, axis=-1)
    return probs.mean(axis=0), probs, logits


def full_topk(p_row, i, k):
    """Top-k keys of row i by (mass desc, index asc) from one stable argsort."""
    cand = p_row[: i + 1]
    order = np.argsort(-cand, kind="stable")
    return np.sort(order[: min(k, i + 1)])


def full_sparse_out(logits, v, supports):
    """O[i,h,:] with attention restricted to supports[i] (renormalised)."""
    hq, n, _ = logits.shape
    v = np.asarray(v, np.float64)
    v_rep = np.repeat(v, hq // v.shape[1], axis=1)    # [N, Hq, d]
    mask = np.zeros((n, n), dtype=bool)
    for i, s in enumerate(supports):
        mask[i, s] = True
    lg = np.where(mask[None], logits, -np.inf)
    w = softmax(lg, axis=-1)
    return np.einsum("hij,jhc->ihc", w, v_rep)


def full_block_topk(P, rows, k):
    """Shared top-k of a block of query rows from the full mass matrix: the
    column mean over the rows (entries past a row's diagonal are 0 in P),
    ranked by one stable argsort over the keys the last row sees."""
    last = rows[-1]
    score = P[list(rows), : last + 1].mean(axis=0)
    order = np.argsort(-score, kind="stable")
    return score, np.sort(order[: min(k, last + 1)])
