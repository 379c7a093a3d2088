"""Plain fp64 CPU oracle of the attention-mass top-k prefill path.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product. Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it. The HIP library never calls it, and the two share no code: the
oracle takes its inputs from the seeded generator and nothing else.

Sources. Everything here restates the paper "How Much Dense Attention is
Necessary? Oracle-Guided Sparse Prefill for Full/GQA Layers in Hybrid
Long-Context Models" (arXiv 2606.07703). It is cited in two places:
  [Abstract]  the authors' abstract (searcharxiv.org page, "Abstract");
  [TB 2.1]    the gist.science page, "Technischer Bericht", section 2.1 (the
              attention-mass top-k oracle); [TB 2.2] is its section 2.2 (the
              head-collapsed indexer and its KL distillation), [TB 2.3] its
              section 2.3 (the oracle,
              indexer and realization gaps) and [TB 3.1] its section 3.1
              (oracle feasibility, with the sparsity range of the 4K-100K
              sweep).
Readings of points those pages leave open are marked READING; each one is
listed in the design notes of the repository.

Notation: N tokens, Hq query heads, Hkv KV heads, G = Hq/Hkv, head h reads
KV head g(h) = h // G (READING: contiguous groups), d = head dim, scale
tau = 1/sqrt(d) unless given. Row i sees keys j <= i (causal prefill).

Every floating-point step runs in float64 on the exact input values (bf16 and
fp32 inputs convert to float64 without rounding). Matrix products use numpy's
BLAS matmul as a library primitive; nothing is blocked, fused or reordered.

Pins (tests marked "not gpu"): brute-force full-tensor enumeration, torch fp64
scaled_dot_product_attention for dense outputs, closed forms (equal keys,
single head, one-token support, hand-derived golden rows) and invariants
(mass rows sum to 1, k >= i+1 keeps everything, nesting over k, causality,
planted needles selected, the pages' sparsity range).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def default_scale(d: int) -> float:
    """Softmax temperature tau = 1/sqrt(d) (READING: one factor on the logits)."""
    return 1.0 / math.sqrt(d)


def kv_head(h: int, hq: int, hkv: int) -> int:
    """GQA routing: query head h uses KV head floor(h / G), G = Hq/Hkv (READING)."""
    return h // (hq // hkv)


def row_logits(q_i: np.ndarray, k_t: np.ndarray, i: int, scale: float) -> np.ndarray:
    """Logits s_h(j) = tau * <Q[i,h], K[j,g(h)]> for every head h and key j <= i.

    q_i: [Hq, d] float64 query row; k_t: [Hkv, N, d] float64 keys (KV-head major).
    Returns [Hq, i+1] float64. [TB 2.1]: the oracle scores the whole causal
    history of each query position with dense attention; [Abstract].
    """
    hq = q_i.shape[0]
    hkv = k_t.shape[0]
    g = hq // hkv
    out = np.empty((hq, i + 1), dtype=np.float64)
    for kv in range(hkv):
        heads = slice(kv * g, (kv + 1) * g)
        out[heads] = scale * (q_i[heads] @ k_t[kv, : i + 1].T)
    return out


def log_sum_exp(s: np.ndarray) -> np.ndarray:
    """Per-head row log-sum-exp: LSE_h = m_h + log sum_j exp(s_h(j) - m_h)."""
    m = np.max(s, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))[..., 0]


def head_mass(s: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """Head-averaged attention mass P(j) = (1/Hq) sum_h exp(s_h(j) - LSE_h).

    [TB 2.1]: the per-head softmax distributions of the query are aggregated
    over the query heads into one head-averaged token-importance distribution
    (P_{l,t}); [Abstract]: "head-averaged token support". READING: arithmetic
    mean of post-softmax probabilities over all Hq heads, so P sums to 1.
    """
    return np.mean(np.exp(s - lse[:, None]), axis=0)


def top_units(score: np.ndarray, k: int) -> np.ndarray:
    """The k best units by (score descending, index ascending), returned ascending.

    [TB 2.1]: top-k indices of the distribution under budget k. READING: when
    a row has at most k units it keeps all of them; equal scores go to the
    smaller index.
    """
    n = score.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -score))
    return np.sort(order[:k]).astype(np.int64)


def kth_score(score: np.ndarray, k: int) -> float:
    """The k-th largest score of the row (the selection boundary); -inf if n <= k."""
    n = score.shape[0]
    if n <= k:
        return -math.inf
    return float(np.sort(score)[::-1][k - 1])


def block_masses(p: np.ndarray, block: int) -> np.ndarray:
    """M(b) = sum of P(j) over the visible keys of key block b.

    READING: key blocks are aligned runs of ``block`` tokens; the diagonal
    block only holds keys j <= i (those are the only keys P covers).
    """
    nb = (p.shape[0] + block - 1) // block
    out = np.zeros(nb, dtype=np.float64)
    for b in range(nb):
        out[b] = np.sum(p[b * block:(b + 1) * block])
    return out


def tokens_of_blocks(blocks: np.ndarray, block: int, i: int) -> np.ndarray:
    """Token support covered by the chosen key blocks, clipped causally to j <= i."""
    if blocks.size == 0:
        return np.zeros(0, dtype=np.int64)
    toks = [np.arange(b * block, min((b + 1) * block, i + 1)) for b in blocks]
    return np.concatenate(toks).astype(np.int64)


def support_attention(s: np.ndarray, v_t: np.ndarray, support: np.ndarray):
    """Attention recomputed on the support only, with the original Q/K/V.

    O_h = sum_{j in S} exp(s_h(j) - LSE^S_h) V[j, g(h)], with LSE^S_h the
    log-sum-exp over S. [TB 2.1] and [Abstract]: after selection the
    attention output is recomputed restricted to the chosen support.
    READING: the softmax is renormalised over S (keys outside S are masked).

    s: [Hq, i+1] logits; v_t: [Hkv, N, d] float64; support: sorted key ids.
    Returns (O [Hq, d], LSE^S [Hq]).
    """
    hq = s.shape[0]
    hkv = v_t.shape[0]
    g = hq // hkv
    ss = s[:, support]
    lse_s = log_sum_exp(ss)
    w = np.exp(ss - lse_s[:, None])
    out = np.empty((hq, v_t.shape[2]), dtype=np.float64)
    for kv in range(hkv):
        heads = slice(kv * g, (kv + 1) * g)
        out[heads] = w[heads] @ v_t[kv, support]
    return out, lse_s


def dense_attention(s: np.ndarray, lse: np.ndarray, v_t: np.ndarray, i: int) -> np.ndarray:
    """Dense causal attention O_h = sum_{j<=i} exp(s_h(j) - LSE_h) V[j, g(h)]."""
    hq = s.shape[0]
    hkv = v_t.shape[0]
    g = hq // hkv
    w = np.exp(s - lse[:, None])
    out = np.empty((hq, v_t.shape[2]), dtype=np.float64)
    for kv in range(hkv):
        heads = slice(kv * g, (kv + 1) * g)
        out[heads] = w[heads] @ v_t[kv, : i + 1]
    return out


def causal_sparsity(n: int, k: int) -> float:
    """Fraction of causal query-key pairs a token budget k skips.

    sparsity = 1 - sum_i min(i+1, k) / sum_i (i+1), over rows i = 0..n-1.
    READING of [TB 3.1]'s sparsity figures: with this count the 4K/k=256 and
    100K/k=2048 ends of the sweep give 87.9 % and 96.0 %.
    """
    i = np.arange(n, dtype=np.float64)
    kept = np.minimum(i + 1, k).sum()
    return float(1.0 - kept / ((n * (n + 1)) / 2.0))


def captured_mass(p: np.ndarray, support: np.ndarray) -> float:
    """Head-averaged dense mass a support keeps: sum over j in S of P_i(j).

    [TB 2.3] splits a sparse layer's loss into the oracle gap (oracle support
    against dense attention), the indexer gap (an indexer's support in place
    of the oracle's) and the realization gap (runtime constraints such as
    selection-block sharing). READING: at the level of one layer their
    synthetic analogue is the share of the dense head-averaged mass P_i
    (which sums to 1) that a support keeps. p is row i's mass [i+1]; support
    holds token ids <= i.
    """
    sup = np.asarray(support, dtype=np.int64)
    return float(p[sup].sum()) if sup.size else 0.0


def support_overlap(a: Sequence[int], b: Sequence[int]) -> int:
    """Number of ids two supports share (negative ids never count).

    [TB 2.3]: the indexer gap compares an indexer's support with the
    oracle's; overlap / |a| is the recall of support a by support b.
    """
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    return int(np.intersect1d(a[a >= 0], b[b >= 0]).size)


def query_block_rows(t: int, b_sel: int, n: int) -> range:
    """Query rows of selection block t: b_sel consecutive rows, the last block
    holding what is left of [0, N)."""
    return range(t * b_sel, min((t + 1) * b_sel, n))


class OracleLayer:
    """The oracle for one GQA layer: per-row support selection and outputs.

    q: [N,Hq,d], k/v: [N,Hkv,d] arrays (float32 or float64 values).
    """

    def __init__(self, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                 scale: Optional[float] = None):
        self.q = np.asarray(q, dtype=np.float64)
        self.k_t = np.ascontiguousarray(np.asarray(k, dtype=np.float64).transpose(1, 0, 2))
        self.v_t = np.ascontiguousarray(np.asarray(v, dtype=np.float64).transpose(1, 0, 2))
        self.n, self.hq, self.d = self.q.shape
        self.hkv = self.k_t.shape[0]
        if self.hq % self.hkv:
            raise ValueError("Hq must be a multiple of Hkv")
        self.scale = default_scale(self.d) if scale is None else float(scale)

    def logits(self, i: int) -> np.ndarray:
        return row_logits(self.q[i], self.k_t, i, self.scale)

    def row(self, i: int, k: int, key_block: int = 1, dense: bool = False) -> dict:
        """Everything the oracle records for row i.

        Keys: lse [Hq]; p [i+1] (head-averaged mass); score [units] (P for
        tokens, M for key blocks); units (selected unit ids, ascending);
        unit_mass; kth (k-th largest score, -inf when all units are kept);
        support (token ids); captured (sum of P over the support); out [Hq,d]
        and lse_s [Hq] on the oracle's own support; dense_out when asked.
        """
        s = self.logits(i)
        lse = log_sum_exp(s)
        p = head_mass(s, lse)
        score = p if key_block == 1 else block_masses(p, key_block)
        units = top_units(score, k)
        support = units if key_block == 1 else tokens_of_blocks(units, key_block, i)
        out, lse_s = support_attention(s, self.v_t, support)
        res = {"lse": lse, "p": p, "score": score, "units": units,
               "unit_mass": score[units], "kth": kth_score(score, k),
               "support": support, "captured": float(p[support].sum()),
               "out": out, "lse_s": lse_s}
        if dense:
            res["dense_out"] = dense_attention(s, lse, self.v_t, i)
        return res

    def query_block(self, t: int, k: int, b_sel: int = 64) -> dict:
        """Support shared by selection block t (b_sel consecutive query rows).

        [TB 2.1]: with selection-block-shared granularity (b_sel = 64) one
        support set is chosen for a block of consecutive queries, to amortise
        system costs. READING: the block scores key j by the mean over its
        rows of their head-averaged masses P_i(j), a key after row i counting
        0 for that row; the top-k keys by (score descending, id ascending)
        among the keys the block's last row sees are shared by every row of
        the block; each row then attends over the shared keys j <= i.

        Keys: rows; score [last row + 1]; units (ascending); unit_mass; kth;
        out {i: [Hq,d]} and lse_s {i: [Hq]} per row (zeros and -inf for a
        row that sees none of the shared keys).
        """
        rows = query_block_rows(t, b_sel, self.n)
        last = rows[-1]
        score = np.zeros(last + 1, dtype=np.float64)
        logits = {}
        for i in rows:
            s = self.logits(i)
            score[: i + 1] += head_mass(s, log_sum_exp(s))
            logits[i] = s
        score /= len(rows)
        units = top_units(score, k)
        out, lse_s = {}, {}
        for i in rows:
            sup = units[units <= i]
            if sup.size:
                out[i], lse_s[i] = support_attention(logits[i], self.v_t, sup)
            else:
                out[i] = np.zeros((self.hq, self.d))
                lse_s[i] = np.full(self.hq, -math.inf)
        return {"rows": rows, "score": score, "units": units, "unit_mass": score[units],
                "kth": kth_score(score, k), "out": out, "lse_s": lse_s}

    def attention_on(self, i: int, support: Sequence[int]):
        """Sparse output of row i on a given support (used with the GPU's support)."""
        sup = np.asarray(sorted(int(j) for j in support), dtype=np.int64)
        return support_attention(self.logits(i), self.v_t, sup)

    def captured(self, i: int, support: Sequence[int]) -> float:
        """Head-averaged dense mass of row i on a given token support ([TB 2.3])."""
        s = self.logits(i)
        return captured_mass(head_mass(s, log_sum_exp(s)), np.asarray(support, dtype=np.int64))

    def dense(self, i: int) -> np.ndarray:
        s = self.logits(i)
        return dense_attention(s, log_sum_exp(s), self.v_t, i)


class IndexerOracle:
    """Head-collapsed indexer scoring + key-block top-k ([TB 2.2], [Abstract]).

    One shared score per key replaces the per-head scores: s(j) = tau_idx *
    <q_idx[i], k_idx[j]>; P_idx = causal softmax over j <= i; block mass =
    sum of P_idx over the block's visible keys; the top-k blocks form the
    support that the sparse layer then attends over with the main Q/K/V.
    READING: the block score is the summed softmax mass with temperature
    tau_idx = 1/sqrt(d_idx).
    """

    def __init__(self, q_idx: np.ndarray, k_idx: np.ndarray, scale: Optional[float] = None):
        self.q = np.asarray(q_idx, dtype=np.float64)
        self.k = np.asarray(k_idx, dtype=np.float64)
        self.scale = default_scale(self.q.shape[1]) if scale is None else float(scale)

    def query_block(self, t: int, k: int, key_block: int, b_sel: int = 64) -> dict:
        """The indexer's support shared by selection block t ([TB 2.1] b_sel,
        realised with the indexer as in [TB 2.2]; [TB 2.3] names the cost of
        such runtime sharing the realization gap).

        READING (as for the oracle's selection blocks): unit u (a key block,
        or a token when key_block = 1) scores the mean over the block's rows of
        the indexer mass the row puts on u's keys up to itself; the top-k units
        by (score descending, id ascending) among those the block's last row
        sees are shared by every row, each row attending over their tokens
        j <= i.

        Keys: rows; score [units the last row sees]; units (ascending); kth;
        support {i: token ids of the shared units clipped to j <= i}.
        """
        rows = query_block_rows(t, b_sel, self.q.shape[0])
        last = rows[-1]
        colmean = np.zeros(last + 1)
        for i in rows:
            s = self.scale * (self.k[: i + 1] @ self.q[i])
            m = np.max(s)
            colmean[: i + 1] += np.exp(s - (m + math.log(np.sum(np.exp(s - m)))))
        colmean /= len(rows)
        score = colmean if key_block == 1 else block_masses(colmean, key_block)
        units = top_units(score, k)
        support = {i: tokens_of_blocks(units, key_block, i) if key_block > 1 else units[units <= i]
                   for i in rows}
        return {"rows": rows, "score": score, "units": units, "kth": kth_score(score, k),
                "support": support}

    def row(self, i: int, k: int, key_block: int) -> dict:
        s = self.scale * (self.k[: i + 1] @ self.q[i])
        m = np.max(s)
        lse = m + math.log(np.sum(np.exp(s - m)))
        p = np.exp(s - lse)
        score = p if key_block == 1 else block_masses(p, key_block)
        units = top_units(score, k)
        support = units if key_block == 1 else tokens_of_blocks(units, key_block, i)
        return {"lse": lse, "p": p, "score": score, "units": units,
                "unit_mass": score[units], "kth": kth_score(score, k),
                "support": support}


class KLDistillOracle:
    """KL-distillation loss of the indexer against the oracle's mass ([TB 2.2]).

    The indexer is trained by KL divergence from the dense head-averaged
    attention-mass distribution, the backbone frozen. READING: teacher P_i =
    the oracle's head-averaged mass over keys j <= i (token level); student
    Q_i = causal softmax over j <= i of t_ij = tau_idx * <q_idx[i], k_idx[j]>
    (tau_idx = 1/sqrt(d_idx), as in the indexer's scoring); per-row loss
    KL_i = sum_j P_ij (log P_ij - log Q_ij) (terms with P_ij = 0 count 0);
    training loss L = (1/N) sum_i KL_i; gradients of L with respect to q_idx
    and k_idx only (the teacher is a constant):
      dL/dt_ij = (Q_ij - P_ij) / N,
      dL/dq_idx[i] = tau_idx sum_j dL/dt_ij k_idx[j],
      dL/dk_idx[j] = tau_idx sum_{i >= j} dL/dt_ij q_idx[i].
    """

    def __init__(self, layer: "OracleLayer", q_idx: np.ndarray, k_idx: np.ndarray,
                 scale: Optional[float] = None):
        self.layer = layer
        self.q = np.asarray(q_idx, dtype=np.float64)
        self.k = np.asarray(k_idx, dtype=np.float64)
        self.scale = default_scale(self.q.shape[1]) if scale is None else float(scale)
        self.n = self.q.shape[0]

    def row(self, i: int) -> dict:
        """Teacher P, student log Q, KL_i and dL/dt (length i+1) of row i."""
        s = self.layer.logits(i)
        p = head_mass(s, log_sum_exp(s))
        t = self.scale * (self.k[: i + 1] @ self.q[i])
        m = np.max(t)
        log_q = t - (m + math.log(np.sum(np.exp(t - m))))
        pos = p > 0
        kl = float(np.sum(p[pos] * (np.log(p[pos]) - log_q[pos])))
        dt = (np.exp(log_q) - p) / self.n
        return {"p": p, "log_q": log_q, "kl": kl, "dt": dt}

    def dq(self, i: int) -> np.ndarray:
        """dL/dq_idx[i] (needs row i only)."""
        return self.scale * (self.row(i)["dt"] @ self.k[: i + 1])

    def dk(self, keys: Sequence[int]) -> np.ndarray:
        """dL/dk_idx[j] for the given keys (needs every row i >= min(keys))."""
        keys = np.asarray(keys, dtype=np.int64)
        out = np.zeros((keys.size, self.q.shape[1]))
        for i in range(int(keys.min()), self.n):
            dt = self.row(i)["dt"]
            sel = keys <= i
            out[sel] += self.scale * np.outer(dt[keys[sel]], self.q[i])
        return out

    def full(self) -> dict:
        """Per-row KL, the loss and both gradients over all rows (small N)."""
        d = self.q.shape[1]
        kl = np.zeros(self.n)
        dq = np.zeros((self.n, d))
        dk = np.zeros((self.n, d))
        for i in range(self.n):
            r = self.row(i)
            kl[i] = r["kl"]
            dq[i] = self.scale * (r["dt"] @ self.k[: i + 1])
            dk[: i + 1] += self.scale * np.outer(r["dt"], self.q[i])
        return {"kl": kl, "loss": float(kl.mean()), "dq": dq, "dk": dk}
