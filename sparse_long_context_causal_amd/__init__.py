"""amtk: attention-mass top-k oracle for long-context GQA prefill on MI355X (gfx950).

Thin Python binding over libamtk.so. Every step of the path runs in the HIP
kernels behind the C ABI (include/amtk.h); this module only marshals
arguments: it checks tensor shapes, allocates outputs and the workspace with
torch (device memory plumbing), and passes raw pointers plus torch's current
HIP stream. There is no CPU fallback: without the built library every call
raises.

Functions (names follow the C ABI):
  topk_support(q, k, budget, key_block=1)      -> idx, count, mass, lse
  sparse_attn(q, k, v, idx, count, key_block)  -> out, lse_sparse
  sparse_attn_blocks(q, k, v, idx, count, query_block=64) -> out, lse_sparse
  captured_mass(lse_dense, lse_support)        -> captured [N]
  support_overlap(idx_a, count_a, idx_b, count_b) -> overlap [N]
  kl_distill(q, k, q_idx, k_idx)               -> kl_row, loss, dq_idx, dk_idx
  oracle_prefill(q, k, v, budget, key_block=1) -> out, idx, count, mass, lse
  indexer_topk(q_idx, k_idx, budget, key_block=64) -> idx, count, mass
  indexer_prefill(q, k, v, q_idx, k_idx, budget, key_block=64, query_block=1)
                                               -> out, idx, count, mass
q: [N, Hq, d], k/v: [N, Hkv, d], bf16 or fp32 CUDA (HIP) tensors, contiguous.
"""
import ctypes
from typing import Optional

from . import _abi
from ._abi import AttnDesc, SupportDesc

_LIB = None


class AmtkError(RuntimeError):
    """A non-zero return code from libamtk.so."""

    def __init__(self, fn, code):
        lib = load()
        msg = lib.amtk_strerror(code).decode()
        if code == _abi.AMTK_E_HIP:
            msg += f" (hipError {lib.amtk_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [code {code}]")
        self.code = code


def load():
    """Load libamtk.so once (raises RuntimeError when it was not built)."""
    global _LIB
    if _LIB is None:
        _LIB = _abi.open_library()
    return _LIB


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _abi.AMTK_BF16
    if t.dtype == torch.float32:
        return _abi.AMTK_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _check_dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(device):
    return ctypes.c_void_p(_torch().cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def attn_desc(q, k, scale: Optional[float] = None) -> AttnDesc:
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError(f"q must be [N,Hq,d] and k [N,Hkv,d]; got {tuple(q.shape)}, {tuple(k.shape)}")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share a dtype")
    return AttnDesc(q.shape[0], q.shape[1], k.shape[1], q.shape[2], _dtype_code(q), 1,
                    float(scale) if scale else 0.0)


def support_desc(budget: int, key_block: int = 1, candidate_cap: int = 0,
                 query_block: int = 1) -> SupportDesc:
    return SupportDesc(int(budget), int(key_block), int(query_block), int(candidate_cap))


def _call(name, *args):
    rc = getattr(load(), name)(*args)
    if rc != _abi.AMTK_OK:
        raise AmtkError(name, rc)


def topk_workspace_bytes(ad: AttnDesc, sd: SupportDesc) -> int:
    n = ctypes.c_size_t(0)
    _call("amtk_topk_workspace", ctypes.byref(ad), ctypes.byref(sd), ctypes.byref(n))
    return n.value


def indexer_workspace_bytes(n: int, d_idx: int, dtype_code: int, sd: SupportDesc) -> int:
    b = ctypes.c_size_t(0)
    _call("amtk_indexer_workspace", n, d_idx, dtype_code, ctypes.byref(sd), ctypes.byref(b))
    return b.value


def workspace(nbytes: int, device):
    """A device byte buffer for the workspace (torch allocations are 256-byte aligned)."""
    return _torch().empty(max(int(nbytes), 1), dtype=_torch().uint8, device=device)


def topk_support(q, k, budget: int, key_block: int = 1, scale: Optional[float] = None,
                 candidate_cap: int = 0, want_mass: bool = True, want_lse: bool = True,
                 ws=None, query_block: int = 1):
    """Oracle support selection. Returns (idx [N,k] int32, count [N] int32,
    mass [N,k] fp32 or None, lse [Hq,N] fp32 or None). query_block = 64 shares
    one support among each block of 64 consecutive queries."""
    torch = _torch()
    _check_dev(q, k)
    ad, sd = attn_desc(q, k, scale), support_desc(budget, key_block, candidate_cap, query_block)
    n, hq = q.shape[0], q.shape[1]
    if ws is None:
        ws = workspace(topk_workspace_bytes(ad, sd), q.device)
    idx = torch.empty((n, budget), dtype=torch.int32, device=q.device)
    count = torch.empty((n,), dtype=torch.int32, device=q.device)
    mass = torch.empty((n, budget), dtype=torch.float32, device=q.device) if want_mass else None
    lse = torch.empty((hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _call("topk_support", ctypes.byref(ad), ctypes.byref(sd), _ptr(q), _ptr(k), _ptr(idx),
          _ptr(count), _ptr(mass), _ptr(lse), _ptr(ws), ws.numel(), _stream(q.device))
    return idx, count, mass, lse


def sparse_attn(q, k, v, idx, count, key_block: int = 1, scale: Optional[float] = None,
                want_lse: bool = False, out=None):
    """Attention on each row's support. Returns (out [N,Hq,d] fp32, lse_sparse [Hq,N] or None)."""
    torch = _torch()
    _check_dev(q, k, v, idx, count)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    ad = attn_desc(q, k, scale)
    n, hq, d = q.shape
    if idx.dim() != 2 or idx.shape[0] != n or count.shape != (n,):
        raise ValueError("idx must be [N, max_units] and count [N]")
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _call("sparse_attn", ctypes.byref(ad), int(key_block), int(idx.shape[1]), _ptr(q), _ptr(k),
          _ptr(v), _ptr(idx), _ptr(count), _ptr(out), _ptr(lse), _stream(q.device))
    return out, lse


def sparse_attn_workspace_bytes(ad) -> int:
    """Scratch bytes of sparse_attn_windowed for the layer shape in ad."""
    nbytes = ctypes.c_size_t(0)
    _call("amtk_sparse_attn_workspace", ctypes.byref(ad), ctypes.byref(nbytes))
    return int(nbytes.value)


def sparse_attn_windowed(q, k, v, idx, count, key_block: int = 1, scale: Optional[float] = None,
                         want_lse: bool = False, out=None, ws=None):
    """sparse_attn walked in key windows (better cache reuse at long N; the
    same result up to rounding order). Returns (out [N,Hq,d] fp32,
    lse_sparse [Hq,N] or None)."""
    torch = _torch()
    _check_dev(q, k, v, idx, count)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    ad = attn_desc(q, k, scale)
    n, hq, d = q.shape
    if idx.dim() != 2 or idx.shape[0] != n or count.shape != (n,):
        raise ValueError("idx must be [N, max_units] and count [N]")
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(sparse_attn_workspace_bytes(ad), q.device)
    lse = torch.empty((hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _call("sparse_attn_windowed", ctypes.byref(ad), int(key_block), int(idx.shape[1]), _ptr(q),
          _ptr(k), _ptr(v), _ptr(idx), _ptr(count), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(),
          _stream(q.device))
    return out, lse


def sparse_attn_windowed_static(q, k, v, idx, count, key_block: int = 1,
                                scale: Optional[float] = None, want_lse: bool = False, out=None):
    """sparse_attn_windowed with its scratch in the library's static device
    array (no workspace; the C call allocates nothing). Outputs are allocated
    here unless `out` is given. Returns (out [N,Hq,d] fp32, lse_sparse [Hq,N]
    or None)."""
    torch = _torch()
    _check_dev(q, k, v, idx, count)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    ad = attn_desc(q, k, scale)
    n, hq, d = q.shape
    if idx.dim() != 2 or idx.shape[0] != n or count.shape != (n,):
        raise ValueError("idx must be [N, max_units] and count [N]")
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _call("sparse_attn_windowed_static", ctypes.byref(ad), int(key_block), int(idx.shape[1]),
          _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(count), _ptr(out), _ptr(lse),
          _stream(q.device))
    return out, lse


def sparse_attn_blocks(q, k, v, idx, count, query_block: int = 64, key_block: int = 1,
                       scale: Optional[float] = None, want_lse: bool = False, out=None):
    """Attention of each selection block of query_block rows on the support in
    the block's first row (rows skip ids after themselves). Returns
    (out [N,Hq,d] fp32, lse_sparse [Hq,N] or None)."""
    torch = _torch()
    _check_dev(q, k, v, idx, count)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    if idx.dtype != torch.int32 or count.dtype != torch.int32:
        raise TypeError("idx and count must be int32")
    ad = attn_desc(q, k, scale)
    n, hq, d = q.shape
    if idx.dim() != 2 or idx.shape[0] != n or count.shape != (n,):
        raise ValueError("idx must be [N, max_units] and count [N]")
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _call("sparse_attn_blocks", ctypes.byref(ad), int(key_block), int(query_block),
          int(idx.shape[1]), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(count), _ptr(out),
          _ptr(lse), _stream(q.device))
    return out, lse


def captured_mass(lse_dense, lse_support, out=None):
    """Per row, the head-averaged dense mass a support keeps, from the dense
    per-head LSE [Hq,N] and the LSE over the support [Hq,N]. Returns [N] fp32."""
    torch = _torch()
    _check_dev(lse_dense, lse_support)
    if lse_dense.dtype != torch.float32 or lse_support.dtype != torch.float32:
        raise TypeError("LSE arrays must be float32")
    if lse_dense.dim() != 2 or lse_support.shape != lse_dense.shape:
        raise ValueError("lse_dense and lse_support must both be [Hq, N]")
    hq, n = lse_dense.shape
    if out is None:
        out = torch.empty((n,), dtype=torch.float32, device=lse_dense.device)
    _call("captured_mass", n, hq, _ptr(lse_dense), _ptr(lse_support), _ptr(out),
          _stream(lse_dense.device))
    return out


def support_overlap(idx_a, count_a, idx_b, count_b, out=None):
    """Per row, the number of ids two supports share (ids ascending within
    each row's count). Returns [N] int32."""
    torch = _torch()
    _check_dev(idx_a, count_a, idx_b, count_b)
    for t in (idx_a, count_a, idx_b, count_b):
        if t.dtype != torch.int32:
            raise TypeError("ids and counts must be int32")
    n = idx_a.shape[0]
    if idx_a.dim() != 2 or idx_b.dim() != 2 or idx_b.shape[0] != n or count_a.shape != (n,) \
            or count_b.shape != (n,):
        raise ValueError("idx_a/idx_b must be [N, max] and counts [N]")
    if out is None:
        out = torch.empty((n,), dtype=torch.int32, device=idx_a.device)
    _call("support_overlap", n, int(idx_a.shape[1]), _ptr(idx_a), _ptr(count_a),
          int(idx_b.shape[1]), _ptr(idx_b), _ptr(count_b), _ptr(out), _stream(idx_a.device))
    return out


def kl_workspace_bytes(ad, d_idx: int) -> int:
    nbytes = ctypes.c_size_t(0)
    _call("amtk_kl_workspace", ctypes.byref(ad), int(d_idx), ctypes.byref(nbytes))
    return nbytes.value


def kl_distill(q, k, q_idx, k_idx, scale: Optional[float] = None,
               idx_scale: Optional[float] = None, ws=None):
    """KL-distillation loss of the indexer (q_idx, k_idx) against the dense
    head-averaged mass of (q, k), with the gradients of the mean loss.
    Returns (kl_row [N] fp32, loss [1] fp32, dq_idx [N,d_idx] fp32,
    dk_idx [N,d_idx] fp32)."""
    torch = _torch()
    _check_dev(q, k, q_idx, k_idx)
    if q_idx.dtype != torch.bfloat16 or k_idx.dtype != torch.bfloat16:
        raise TypeError("q_idx and k_idx must be bfloat16")
    n = q.shape[0]
    if q_idx.dim() != 2 or q_idx.shape[0] != n or k_idx.shape != q_idx.shape:
        raise ValueError("q_idx and k_idx must both be [N, d_idx]")
    ad = attn_desc(q, k, scale)
    d_idx = q_idx.shape[1]
    if ws is None:
        ws = workspace(kl_workspace_bytes(ad, d_idx), q.device)
    dev = q.device
    kl = torch.empty((n,), dtype=torch.float32, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    dq = torch.empty((n, d_idx), dtype=torch.float32, device=dev)
    dk = torch.empty((n, d_idx), dtype=torch.float32, device=dev)
    _call("kl_distill", ctypes.byref(ad), int(d_idx), ctypes.c_float(idx_scale or 0.0), _ptr(q),
          _ptr(k), _ptr(q_idx), _ptr(k_idx), _ptr(kl), _ptr(loss), _ptr(dq), _ptr(dk), _ptr(ws),
          ws.numel(), _stream(dev))
    return kl, loss, dq, dk


def oracle_prefill(q, k, v, budget: int, key_block: int = 1, scale: Optional[float] = None,
                   candidate_cap: int = 0, want_mass: bool = True, want_lse: bool = True,
                   ws=None, query_block: int = 1):
    """topk_support + sparse_attn. Returns (out, idx, count, mass, lse)."""
    torch = _torch()
    _check_dev(q, k, v)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    ad, sd = attn_desc(q, k, scale), support_desc(budget, key_block, candidate_cap, query_block)
    n, hq, d = q.shape
    if ws is None:
        ws = workspace(topk_workspace_bytes(ad, sd), q.device)
    out = torch.empty((n, hq, d), dtype=torch.float32, device=q.device)
    idx = torch.empty((n, budget), dtype=torch.int32, device=q.device)
    count = torch.empty((n,), dtype=torch.int32, device=q.device)
    mass = torch.empty((n, budget), dtype=torch.float32, device=q.device) if want_mass else None
    lse = torch.empty((hq, n), dtype=torch.float32, device=q.device) if want_lse else None
    _call("oracle_prefill", ctypes.byref(ad), ctypes.byref(sd), _ptr(q), _ptr(k), _ptr(v),
          _ptr(out), _ptr(idx), _ptr(count), _ptr(mass), _ptr(lse), _ptr(ws), ws.numel(),
          _stream(q.device))
    return out, idx, count, mass, lse


def indexer_topk(q_idx, k_idx, budget: int, key_block: int = 64, scale: Optional[float] = None,
                 candidate_cap: int = 0, want_mass: bool = True, ws=None, query_block: int = 1):
    """Head-collapsed indexer top-k. Returns (idx [N,k], count [N], mass [N,k] or None).
    query_block = 64 shares one support among each block of 64 queries."""
    torch = _torch()
    _check_dev(q_idx, k_idx)
    if q_idx.dim() != 2 or q_idx.shape != k_idx.shape or q_idx.dtype != k_idx.dtype:
        raise ValueError("q_idx and k_idx must both be [N, d_idx] with one dtype")
    n, di = q_idx.shape
    code = _dtype_code(q_idx)
    sd = support_desc(budget, key_block, candidate_cap, query_block)
    if ws is None:
        ws = workspace(indexer_workspace_bytes(n, di, code, sd), q_idx.device)
    idx = torch.empty((n, budget), dtype=torch.int32, device=q_idx.device)
    count = torch.empty((n,), dtype=torch.int32, device=q_idx.device)
    mass = torch.empty((n, budget), dtype=torch.float32, device=q_idx.device) if want_mass else None
    _call("indexer_topk", n, di, code, ctypes.c_float(float(scale) if scale else 0.0),
          ctypes.byref(sd), _ptr(q_idx), _ptr(k_idx), _ptr(idx), _ptr(count), _ptr(mass),
          _ptr(ws), ws.numel(), _stream(q_idx.device))
    return idx, count, mass


def indexer_prefill(q, k, v, q_idx, k_idx, budget: int, key_block: int = 64,
                    query_block: int = 1, scale: Optional[float] = None,
                    idx_scale: Optional[float] = None, want_mass: bool = True, ws=None, out=None):
    """Indexer-driven sparse prefill: the indexer's support, then attention on
    it. query_block = 1: per query (indexer_topk + sparse_attn); 64: the fused
    realisation (one kernel per block of 64 queries scores, selects and
    attends; other head layouts and token units: the block support, then the
    per-row gather). Returns (out [N,Hq,d] fp32, idx, count, mass or None)."""
    torch = _torch()
    _check_dev(q, k, v, q_idx, k_idx)
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("v must match k in shape and dtype")
    if q_idx.dim() != 2 or q_idx.shape != k_idx.shape or q_idx.dtype != q.dtype:
        raise ValueError("q_idx and k_idx must both be [N, d_idx] in the layer's dtype")
    ad = attn_desc(q, k, scale)
    n, hq, d = q.shape
    di = q_idx.shape[1]
    sd = support_desc(budget, key_block, 0, query_block)
    dev = q.device
    if ws is None:
        ws = workspace(indexer_workspace_bytes(n, di, _dtype_code(q_idx), sd), dev)
    if out is None:
        out = torch.empty((n, hq, d), dtype=torch.float32, device=dev)
    idx = torch.empty((n, budget), dtype=torch.int32, device=dev)
    count = torch.empty((n,), dtype=torch.int32, device=dev)
    mass = torch.empty((n, budget), dtype=torch.float32, device=dev) if want_mass else None
    _call("indexer_prefill", ctypes.byref(ad), int(di), ctypes.c_float(idx_scale or 0.0),
          ctypes.byref(sd), _ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), _ptr(k_idx), _ptr(out),
          _ptr(idx), _ptr(count), _ptr(mass), _ptr(ws), ws.numel(), _stream(dev))
    return out, idx, count, mass


def pool_stats(ad: AttnDesc, sd: SupportDesc, ws, device=None):
    """(max candidates in a row, rows recomputed densely, capacity) of the last run on ws."""
    mx, ov, cap = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int64(0)
    _call("amtk_pool_stats", ctypes.byref(ad), ctypes.byref(sd), _ptr(ws), ws.numel(),
          ctypes.byref(mx), ctypes.byref(ov), ctypes.byref(cap), _stream(ws.device))
    return mx.value, ov.value, cap.value


__all__ = ["load", "topk_support", "sparse_attn", "sparse_attn_windowed", "sparse_attn_blocks",
           "sparse_attn_workspace_bytes", "oracle_prefill",
           "indexer_topk", "indexer_prefill", "captured_mass", "support_overlap", "kl_distill",
           "kl_workspace_bytes",
           "topk_workspace_bytes", "indexer_workspace_bytes", "workspace", "pool_stats",
           "attn_desc", "support_desc", "AmtkError", "AttnDesc", "SupportDesc"]


class PrefillPlan:
    """Preallocated outputs + workspace for repeated oracle prefills of one layer shape.

    run() enqueues topk_support stages 1-3 and the gather (sparse_attn_windowed,
    or sparse_attn with windowed=False; sparse_attn_blocks for selection
    blocks) on the current stream; stage(s) / attn() enqueue one piece (for
    timing). The indexer variant (q_idx, k_idx given) runs indexer_topk
    instead of topk_support, then the gather over 64-token key blocks.
    """

    def __init__(self, q, k, v, budget, key_block=1, q_idx=None, k_idx=None, candidate_cap=0,
                 query_block=1, windowed=True):
        torch = _torch()
        _check_dev(q, k, v)
        self.q, self.k, self.v = q, k, v
        self.n, self.hq, self.d = q.shape
        self.budget, self.key_block = int(budget), int(key_block)
        self.indexer = q_idx is not None
        self.ad = attn_desc(q, k)
        self.sd = support_desc(budget, key_block, candidate_cap, query_block)
        dev = q.device
        if self.indexer:
            _check_dev(q_idx, k_idx)
            self.q_idx, self.k_idx = q_idx, k_idx
            nbytes = indexer_workspace_bytes(self.n, q_idx.shape[1], _dtype_code(q_idx), self.sd)
        else:
            nbytes = topk_workspace_bytes(self.ad, self.sd)
        self.ws = workspace(nbytes, dev)
        # the per-row gather runs in key windows (sparse_attn_windowed) unless
        # windowed=False asks for the one-pass sparse_attn
        self.windowed = windowed
        self.attn_ws = workspace(sparse_attn_workspace_bytes(self.ad), dev) if windowed else None
        self.idx = torch.empty((self.n, budget), dtype=torch.int32, device=dev)
        self.count = torch.empty((self.n,), dtype=torch.int32, device=dev)
        self.mass = torch.empty((self.n, budget), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.hq, self.n), dtype=torch.float32, device=dev)
        self.out = torch.empty((self.n, self.hq, self.d), dtype=torch.float32, device=dev)
        # the block tile kernel's shapes (sparse_attn_blocks); elsewhere the
        # per-row kernel reads the rows' copies of their block's support
        self.shared_tiles = (q.dtype == torch.bfloat16 and self.d == 128 and self.hq == 32
                             and k.shape[1] == 8 and query_block == 64)

    def stage(self, s):
        if self.indexer:
            raise ValueError("the indexer path runs as one call (indexer())")
        _call("topk_support_stage", ctypes.byref(self.ad), ctypes.byref(self.sd), int(s),
              _ptr(self.q), _ptr(self.k), _ptr(self.idx), _ptr(self.count), _ptr(self.mass),
              _ptr(self.lse), _ptr(self.ws), self.ws.numel(), _stream(self.q.device))

    def indexer_call(self):
        _call("indexer_topk", self.n, self.q_idx.shape[1], _dtype_code(self.q_idx),
              ctypes.c_float(0.0), ctypes.byref(self.sd), _ptr(self.q_idx), _ptr(self.k_idx),
              _ptr(self.idx), _ptr(self.count), _ptr(self.mass), _ptr(self.ws), self.ws.numel(),
              _stream(self.q.device))

    def attn(self):
        qb = self.sd.query_block
        if qb != 1 and self.shared_tiles:
            _call("sparse_attn_blocks", ctypes.byref(self.ad), self.key_block, qb, self.budget,
                  _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.idx), _ptr(self.count),
                  _ptr(self.out), None, _stream(self.q.device))
            return
        if self.windowed:
            _call("sparse_attn_windowed", ctypes.byref(self.ad), self.key_block, self.budget,
                  _ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.idx), _ptr(self.count),
                  _ptr(self.out), None, _ptr(self.attn_ws), self.attn_ws.numel(),
                  _stream(self.q.device))
            return
        _call("sparse_attn", ctypes.byref(self.ad), self.key_block, self.budget, _ptr(self.q),
              _ptr(self.k), _ptr(self.v), _ptr(self.idx), _ptr(self.count), _ptr(self.out), None,
              _stream(self.q.device))

    def run(self):
        if self.indexer:
            self.indexer_call()
        else:
            for s in (1, 2, 3):
                self.stage(s)
        self.attn()


__all__.append("PrefillPlan")
