"""ctypes declarations of libamtk.so's C ABI (include/amtk.h)."""
import ctypes
import os

# AMTK_LIBRARY may point at another build of the same library (e.g. a variant
# compiled with different flags); by default the in-tree libamtk.so is used.
LIB_PATH = os.environ.get("AMTK_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libamtk.so")

AMTK_OK = 0
AMTK_E_INVALID = -1
AMTK_E_UNSUPPORTED = -2
AMTK_E_WORKSPACE = -3
AMTK_E_HIP = -4
AMTK_STATIC_SCRATCH_BYTES = 32 << 20
AMTK_BF16 = 0
AMTK_F32 = 1


class AttnDesc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class SupportDesc(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("key_block", ctypes.c_int32),
                ("query_block", ctypes.c_int32), ("candidate_cap", ctypes.c_int32)]


_P = ctypes.c_void_p
_A = ctypes.POINTER(AttnDesc)
_S = ctypes.POINTER(SupportDesc)
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

SIGNATURES = {
    "amtk_topk_workspace": (ctypes.c_int, [_A, _S, ctypes.POINTER(_SZ)]),
    "amtk_workspace_bytes": (_SZ, [_A, _S]),
    "topk_support": (ctypes.c_int, [_A, _S, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "topk_support_stage": (ctypes.c_int, [_A, _S, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sparse_attn": (ctypes.c_int, [_A, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "sparse_attn_windowed_static": (ctypes.c_int, [_A, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                                                   _P]),
    "sparse_attn_blocks": (ctypes.c_int, [_A, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "amtk_sparse_attn_workspace": (ctypes.c_int, [_A, ctypes.POINTER(_SZ)]),
    "sparse_attn_windowed": (ctypes.c_int, [_A, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                            _P]),
    "indexer_prefill": (ctypes.c_int, [_A, _I32, ctypes.c_float, _S, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, ctypes.c_size_t, _P]),
    "captured_mass": (ctypes.c_int, [_I64, _I32, _P, _P, _P, _P]),
    "amtk_kl_workspace": (ctypes.c_int, [_A, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "kl_distill": (ctypes.c_int, [_A, _I32, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
    "support_overlap": (ctypes.c_int, [_I64, _I32, _P, _P, _I32, _P, _P, _P, _P]),
    "oracle_prefill": (ctypes.c_int, [_A, _S, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "amtk_indexer_workspace": (ctypes.c_int, [_I64, _I32, _I32, _S, ctypes.POINTER(_SZ)]),
    "indexer_topk": (ctypes.c_int, [_I64, _I32, _I32, ctypes.c_float, _S, _P, _P, _P, _P, _P,
                                    _P, _SZ, _P]),
    "amtk_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "amtk_last_hip_error": (ctypes.c_int, []),
    "amtk_pool_stats": (ctypes.c_int, [_A, _S, _P, _SZ, ctypes.POINTER(_I64),
                                       ctypes.POINTER(_I64), ctypes.POINTER(_I64), _P]),
}


def open_library(path=LIB_PATH):
    """dlopen libamtk.so and attach the C signatures. Raises if it was not built."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(or python sparse_long_context_causal_amd/build.py)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
