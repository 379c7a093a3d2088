"""Seeded synthetic GQA prefill inputs (sink key + planted needle keys + indexer).

This module only builds inputs. It holds none of the method's arithmetic (no
logits, softmax, mass, top-k or attention), so both the CPU oracle and the HIP
path can take their inputs from it without sharing any computation.

Workloads follow the five layer shapes the oracle is exercised on: a tiny fp32
layer, and bf16 GQA layers of 4K, 32K and 100K tokens (32 query heads, 8 KV
heads, head_dim 128), plus a 32K layer with a single-head 64-wide indexer.
The needles stand in for the retrieval-heavy ("needle in a haystack") long
context evaluations the paper measures on; no item of any benchmark suite is
reproduced here.

Construction (all draws from ``numpy.random.default_rng(seed)`` in this order):
  1. Q[N,Hq,d], K[N,Hkv,d], V[N,Hkv,d] ~ N(0,1) in float32.
  2. For bf16 workloads Q, K, V are rounded to bf16 (round-to-nearest-even).
  3. Sink: K[0,:,:] *= 4 (every KV head; V unchanged).
  4. Needles: for query rows i = 2..N-1 in increasing order, ``min(n, i-1)``
     distinct positions are drawn uniformly from [1, i-1]; each drawn key row
     j is assigned K[j,g,:] = 3*sqrt(d)*m_g/|m_g| for every KV head g, where
     m_g is the mean of row i's G query heads of group g (after rounding).
     Later rows overwrite earlier ones; ``owner[j]`` records the row whose
     needle survives at j (-1 where none). The needle rows are computed in
     float64 from the rounded Q and then rounded to the workload dtype.
  5. Indexer (workload ``indexer_bf16_32k`` only): with colstd() a per-column
     zero-mean/unit-variance standardisation over tokens,
     q_idx = 0.8*colstd(mean_h Q[:,h,:64]) + 0.6*eps_q and
     k_idx = 0.8*colstd(mean_g K[:,g,:64]) + 0.6*eps_k (K after sink and
     needles), eps ~ N(0,1), then rounded to bf16.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    hq: int
    hkv: int
    d: int
    dtype: str            # "f32" or "bf16"
    k: int                # budget in key_block units (default of a sweep)
    key_block: int        # 1 = token support, 64 = 64-token key blocks
    needles: int
    seed: int
    row_seed: int
    sample_rows: Optional[int]   # None = every row
    k_sweep: tuple = ()
    indexer_d: int = 0    # 0 = no indexer; else width of q_idx/k_idx

    @property
    def group(self) -> int:
        return self.hq // self.hkv


WORKLOADS = {
    "tiny_fp32_512": Workload("tiny_fp32_512", 512, 8, 2, 64, "f32", 32, 1, 2,
                              1001, 2001, None),
    "mid_bf16_4k": Workload("mid_bf16_4k", 4096, 32, 8, 128, "bf16", 82, 1, 4,
                            1002, 2002, None),
    "long_bf16_32k": Workload("long_bf16_32k", 32768, 32, 8, 128, "bf16", 655, 1, 8,
                              1003, 2003, 256),
    "vlong_bf16_100k": Workload("vlong_bf16_100k", 100000, 32, 8, 128, "bf16", 2048, 1, 8,
                                1004, 2004, 128, k_sweep=(512, 1024, 2048)),
    "indexer_bf16_32k": Workload("indexer_bf16_32k", 32768, 32, 8, 128, "bf16", 16, 64, 8,
                                 1005, 2005, 256, indexer_d=64),
}
ORDER = ["tiny_fp32_512", "mid_bf16_4k", "long_bf16_32k", "vlong_bf16_100k",
         "indexer_bf16_32k"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    bits = x.view(np.uint32)          # finite inputs: bits + 0x8000 cannot wrap
    bias = bits >> 16
    bias &= 1
    bias += 0x7FFF
    bits += bias
    bits &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-exact float32 values (the bf16 storage pattern)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("values are not bf16-exact")
    return (bits >> 16).astype(np.uint16)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)


def needle_owners(n: int, needles: int, rng: np.random.Generator) -> np.ndarray:
    """owner[j] = the last row i (2 <= i < n) that planted a needle at key j, else -1.

    Row i draws ``min(needles, i-1)`` distinct positions uniformly from [1, i-1]
    (all of them when i-1 <= needles). Draws are made for every row at once;
    a row whose draws collide redraws the colliding slots, in row order.
    """
    owner = np.full(n, -1, dtype=np.int64)
    if needles <= 0 or n < 3:
        return owner
    rows = np.arange(2, n, dtype=np.int64)
    span = rows - 1                                   # size of [1, i-1]
    u = rng.random((rows.size, needles))
    pos = 1 + np.minimum((u * span[:, None]).astype(np.int64), span[:, None] - 1)
    full = span <= needles                            # these rows take all of [1, i-1]
    for r in np.nonzero(full)[0]:
        pos[r, :] = -1
        pos[r, :span[r]] = np.arange(1, span[r] + 1)
    srt = np.sort(pos, axis=1)
    dup = np.nonzero(np.any((srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] > 0), axis=1))[0]
    for r in dup:
        seen = set()
        for c in range(needles):
            while pos[r, c] in seen:
                pos[r, c] = 1 + int(rng.integers(0, span[r]))
            seen.add(pos[r, c])
    owner_rows = np.broadcast_to(rows[:, None], pos.shape)
    ok = pos > 0
    np.maximum.at(owner, pos[ok], owner_rows[ok])
    return owner


def plant(q: np.ndarray, k: np.ndarray, owner: np.ndarray, dtype: str) -> None:
    """Overwrite needle key rows in place from their owners' group-mean queries."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    js = np.nonzero(owner >= 0)[0]
    if js.size == 0:
        return
    rows = owner[js]
    m = q[rows].astype(np.float64).reshape(js.size, hkv, g, d).mean(axis=2)
    norm = np.linalg.norm(m, axis=2, keepdims=True)
    norm[norm == 0] = 1.0
    k[js] = _cast(3.0 * np.sqrt(d) * m / norm, dtype)


def _colstd(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    mu = x.mean(axis=0, keepdims=True)
    sd = x.std(axis=0, keepdims=True)
    sd[sd == 0] = 1.0
    return (x - mu) / sd


def generate(w: Workload, n: Optional[int] = None, needles: Optional[int] = None,
             seed: Optional[int] = None) -> dict:
    """Build the inputs of workload ``w`` (optionally at another length/seed).

    Returns a dict of float32 arrays (bf16-exact for bf16 workloads):
    ``q`` [N,Hq,d], ``k``/``v`` [N,Hkv,d], ``owner`` [N] int64, and for the
    indexer workload ``q_idx``/``k_idx`` [N,indexer_d].
    """
    n = w.n if n is None else int(n)
    needles = w.needles if needles is None else int(needles)
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _cast(rng.standard_normal((n, w.hq, w.d), dtype=np.float32), w.dtype)
    k = _cast(rng.standard_normal((n, w.hkv, w.d), dtype=np.float32), w.dtype)
    v = _cast(rng.standard_normal((n, w.hkv, w.d), dtype=np.float32), w.dtype)
    k[0] = _cast(k[0].astype(np.float64) * 4.0, w.dtype)
    owner = needle_owners(n, needles, rng)
    plant(q, k, owner, w.dtype)
    out = {"q": q, "k": k, "v": v, "owner": owner}
    if w.indexer_d:
        di = w.indexer_d
        zq = _colstd(q[:, :, :di].astype(np.float64).mean(axis=1))
        zk = _colstd(k[:, :, :di].astype(np.float64).mean(axis=1))
        eq = rng.standard_normal((n, di))
        ek = rng.standard_normal((n, di))
        out["q_idx"] = _cast(0.8 * zq + 0.6 * eq, "bf16")
        out["k_idx"] = _cast(0.8 * zk + 0.6 * ek, "bf16")
    return out


def sample_rows(w: Workload, n: Optional[int] = None, count: Optional[int] = None) -> np.ndarray:
    """Rows the oracle evaluates: every row, or a seeded uniform sample (sorted)."""
    n = w.n if n is None else int(n)
    count = w.sample_rows if count is None else count
    if count is None or count >= n:
        return np.arange(n, dtype=np.int64)
    rng = np.random.default_rng(w.row_seed)
    return np.sort(rng.choice(n, size=count, replace=False)).astype(np.int64)


def random_inputs(n: int, hq: int, hkv: int, d: int, dtype: str, seed: int,
                  sink: bool = False) -> dict:
    """Plain N(0,1) Q/K/V of any shape (for edge-case tests), optionally with a sink."""
    rng = np.random.default_rng(seed)
    q = _cast(rng.standard_normal((n, hq, d), dtype=np.float32), dtype)
    k = _cast(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    v = _cast(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    if sink and n > 0:
        k[0] = _cast(k[0].astype(np.float64) * 4.0, dtype)
    return {"q": q, "k": k, "v": v}
