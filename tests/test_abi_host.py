"""Host-side checks of the C ABI: the library loads, exports exactly what
include/amtk.h declares, and rejects bad arguments before launching anything.
No call here reaches a GPU: every argument set fails validation on the host.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "amtk.h")


@pytest.fixture(scope="module")
def lib():
    from sparse_long_context_causal_amd import _abi, build
    if not os.path.exists(_abi.LIB_PATH):
        build.build(verbose=False)
    return _abi.open_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("oracle_prefill", "topk_support", "sparse_attn", "indexer_topk"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from sparse_long_context_causal_amd import _abi
    names = declared_functions()
    assert set(names) == set(_abi.SIGNATURES), (names, sorted(_abi.SIGNATURES))
    for n in names:
        assert getattr(lib, n) is not None
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    # nothing else of ours leaks out
    ours = {s for s in exported if "amtk" in s or s in names}
    assert ours == set(names), sorted(ours - set(names))


def test_workspace_bytes_matches_the_status_form(lib):
    for kw in (dict(), dict(n=1000, hq=32, hkv=8, d=128, k=82), dict(k=4, kb=64), dict(qb=64)):
        a, s = _descs(**kw)
        need = ctypes.c_size_t(0)
        assert lib.amtk_topk_workspace(ctypes.byref(a), ctypes.byref(s), ctypes.byref(need)) == 0
        assert need.value > 0
        assert lib.amtk_workspace_bytes(ctypes.byref(a), ctypes.byref(s)) == need.value
    for kw in (dict(n=0), dict(causal=0), dict(k=0), dict(kb=2)):
        a, s = _descs(**kw)
        assert lib.amtk_workspace_bytes(ctypes.byref(a), ctypes.byref(s)) == 0
    assert lib.amtk_workspace_bytes(None, None) == 0


def test_strerror_covers_codes(lib):
    for c in (0, -1, -2, -3, -4, -99):
        assert lib.amtk_strerror(c)


def _descs(n=64, hq=8, hkv=2, d=64, dtype=0, causal=1, scale=0.0, k=4, kb=1, qb=1, cap=0):
    from sparse_long_context_causal_amd._abi import AttnDesc, SupportDesc
    return AttnDesc(n, hq, hkv, d, dtype, causal, scale), SupportDesc(k, kb, qb, cap)


FAKE = ctypes.c_void_p(0x100000)   # 256-aligned, never dereferenced on the host


def _topk(lib, a, s, ws_bytes=1, q=FAKE, ws=FAKE, idx=FAKE):
    return lib.topk_support(ctypes.byref(a) if a is not None else None, ctypes.byref(s),
                            q, FAKE, idx, FAKE, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), -1), (dict(hq=6, hkv=4), -1), (dict(dtype=7), -1), (dict(scale=float("nan")), -1),
    (dict(k=0), -1), (dict(cap=-1), -1),
    (dict(causal=0), -2), (dict(d=96), -2), (dict(kb=2), -2), (dict(qb=32), -2), (dict(qb=64, kb=64), -2),
    (dict(k=9000), -2),
    (dict(hq=32, hkv=2), -2),          # 16 query heads per KV head
    (dict(hkv=16, hq=16), -2),         # more KV heads than pass waves
    (dict(dtype=1, d=128, hq=8, hkv=2), -2),   # fp32 group tile too large for registers
    (dict(dtype=1, d=128, hq=16, hkv=8), -2),  # fp32 key slots of 8 waves exceed the LDS
])
def test_invalid_arguments_are_rejected(lib, kw, code):
    a, s = _descs(**kw)
    assert _topk(lib, a, s) == code


def test_null_and_misaligned_pointers(lib):
    a, s = _descs()
    assert _topk(lib, None, s) == -1
    assert _topk(lib, a, s, q=None) == -1
    assert _topk(lib, a, s, q=ctypes.c_void_p(0x100004)) == -1     # q not 16-byte aligned
    assert _topk(lib, a, s, ws=ctypes.c_void_p(0x100010)) == -1    # ws not 256-byte aligned


def test_workspace_too_small(lib):
    a, s = _descs()
    need = ctypes.c_size_t(0)
    assert lib.amtk_topk_workspace(ctypes.byref(a), ctypes.byref(s), ctypes.byref(need)) == 0
    assert need.value > 0
    assert _topk(lib, a, s, ws_bytes=need.value - 1) == -3


def test_workspace_sizes_grow_with_n_and_cap(lib):
    prev = 0
    for n in (1, 33, 512, 4096):
        a, s = _descs(n=n)
        need = ctypes.c_size_t(0)
        assert lib.amtk_topk_workspace(ctypes.byref(a), ctypes.byref(s), ctypes.byref(need)) == 0
        assert need.value > prev
        prev = need.value
    a, s1 = _descs(n=4096, cap=10)
    _, s2 = _descs(n=4096, cap=100)
    b1, b2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    lib.amtk_topk_workspace(ctypes.byref(a), ctypes.byref(s1), ctypes.byref(b1))
    lib.amtk_topk_workspace(ctypes.byref(a), ctypes.byref(s2), ctypes.byref(b2))
    assert b2.value - b1.value >= 4096 * 90 * 8


def test_selection_block_workspace_and_pool_stats(lib):
    """query_block = 64 keeps the LSE and the 32-row tiles' column sums
    ((n+31)/32 x n floats) instead of candidate pools, and has no pool stats."""
    n, hq = 4096, 8
    a, s = _descs(n=n, hq=hq, qb=64)
    need = ctypes.c_size_t(0)
    assert lib.amtk_topk_workspace(ctypes.byref(a), ctypes.byref(s), ctypes.byref(need)) == 0
    assert need.value >= (n + 31) // 32 * n * 4 + hq * n * 4
    assert need.value < (n + 31) // 32 * n * 4 + hq * n * 4 + 4096
    # bf16, d = 128, 32/8 heads: plus pass 1's copy of K in MFMA operand order
    from sparse_long_context_causal_amd import _abi
    b = _abi.AttnDesc(n, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    need_b = ctypes.c_size_t(0)
    assert lib.amtk_topk_workspace(ctypes.byref(b), ctypes.byref(s), ctypes.byref(need_b)) == 0
    base = (n + 31) // 32 * n * 4 + 32 * n * 4 + (n + 31) // 32 * 32 * 8 * 128 * 2
    assert base <= need_b.value < base + 4096
    z = ctypes.c_int64(0)
    assert lib.amtk_pool_stats(ctypes.byref(a), ctypes.byref(s), FAKE, need.value, ctypes.byref(z),
                               ctypes.byref(z), ctypes.byref(z), None) == -2


def test_sparse_attn_validation(lib):
    a, _ = _descs()
    f = lib.sparse_attn
    assert f(ctypes.byref(a), 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert f(ctypes.byref(a), 3, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert f(ctypes.byref(a), 1, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == -1


def test_sparse_attn_windowed_validation(lib):
    from sparse_long_context_causal_amd import _abi
    f = lib.sparse_attn_windowed
    b = _abi.AttnDesc(100000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    need = ctypes.c_size_t(0)
    assert lib.amtk_sparse_attn_workspace(ctypes.byref(b), ctypes.byref(need)) == 0
    # window starts [n][windows + 1] int32 (13 windows of 8192 at 100000) + the running LSE
    starts = (100000 * 14 * 4 + 255) // 256 * 256
    assert need.value == starts + (32 * 100000 * 4 + 255) // 256 * 256
    assert lib.amtk_sparse_attn_workspace(ctypes.byref(b), None) == -1
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert f(ctypes.byref(b), 1, 0, *args, FAKE, need.value, None) == -1        # max_units
    assert f(ctypes.byref(b), 3, 4, *args, FAKE, need.value, None) == -2        # key_block
    assert f(ctypes.byref(b), 1, 4, *args, None, need.value, None) == -1        # no scratch
    assert f(ctypes.byref(b), 1, 4, *args, FAKE, need.value - 1, None) == -3    # too small
    odd = ctypes.c_void_p(0x100080)   # scratch must be 256-byte aligned
    assert f(ctypes.byref(b), 1, 4, *args, odd, need.value, None) == -1


def test_sparse_attn_blocks_validation(lib):
    f = lib.sparse_attn_blocks
    a, _ = _descs()
    assert f(ctypes.byref(a), 1, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -1
    # head layouts other than the tile kernel's (fp32 8/2 here) run the per-row
    # gather on the blocks' first rows: the shape passes, the null v fails
    assert f(ctypes.byref(a), 1, 64, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == -1
    assert f(ctypes.byref(a), 64, 64, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1
    from sparse_long_context_causal_amd import _abi
    g3 = _abi.AttnDesc(1000, 24, 8, 128, _abi.AMTK_BF16, 1, 0.0)   # 3 query heads per KV head
    assert f(ctypes.byref(g3), 1, 64, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    b = _abi.AttnDesc(1000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    assert f(ctypes.byref(b), 1, 32, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert f(ctypes.byref(b), 16, 64, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == -2
    assert f(ctypes.byref(b), 64, 64, 4, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None) == -1
    odd = ctypes.c_void_p(0x100004)   # o must be 16-byte aligned
    assert f(ctypes.byref(b), 1, 64, 4, FAKE, FAKE, FAKE, FAKE, FAKE, odd, None, None) == -1


def test_indexer_prefill_validation(lib):
    from sparse_long_context_causal_amd import _abi
    f = lib.indexer_prefill
    b = _abi.AttnDesc(1000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    s_fused = _abi.SupportDesc(16, 64, 64, 0)
    need = ctypes.c_size_t(0)
    assert lib.amtk_indexer_workspace(1000, 64, _abi.AMTK_BF16, ctypes.byref(s_fused),
                                      ctypes.byref(need)) == 0
    args = [FAKE] * 5                                   # q, k, v, q_idx, k_idx
    outs = [FAKE, FAKE, FAKE, None]                     # o, idx, count, mass
    ok = lambda sd, **kw: f(ctypes.byref(kw.get("a", b)), kw.get("di", 64), 0.0, ctypes.byref(sd),
                            *kw.get("args", args), *kw.get("outs", outs), FAKE,
                            kw.get("ws", need.value), None)
    assert ok(s_fused, ws=need.value - 1) == -3
    assert ok(s_fused, di=32) == -2                     # indexer heads of 64 or 128 only
    # token units: the indexer's column-sum top-k, then the per-row gather
    # (stopped here by its workspace check, before any launch)
    assert ok(_abi.SupportDesc(16, 1, 64, 0), ws=0) == -3
    assert ok(_abi.SupportDesc(2000, 64, 64, 0)) == -2  # more winners than the block kernel's LDS holds
    a, _ = _descs()
    assert ok(s_fused, a=a, ws=0) == -3                 # other layouts: the two-step realisation
    g3 = _abi.AttnDesc(1000, 24, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    assert ok(s_fused, a=g3) == -2                      # a layout no gather takes
    assert ok(s_fused, outs=[None, FAKE, FAKE, None]) == -1
    assert ok(s_fused, args=[FAKE, FAKE, FAKE, None, FAKE]) == -1
    # the per-query realisation checks the backbone q and k before any launch
    odd = ctypes.c_void_p(0x100002)
    s_query = _abi.SupportDesc(16, 1, 1, 0)
    for bad in ([None, FAKE, FAKE, FAKE, FAKE], [FAKE, None, FAKE, FAKE, FAKE],
                [odd, FAKE, FAKE, FAKE, FAKE], [FAKE, odd, FAKE, FAKE, FAKE]):
        assert ok(s_query, args=bad) == -1
        assert ok(_abi.SupportDesc(16, 64, 1, 0), args=bad) == -1
        assert ok(s_fused, args=bad) == -1


def test_static_windowed_validation(lib):
    from sparse_long_context_causal_amd import _abi
    f = lib.sparse_attn_windowed_static
    ok = lambda a, kb=1, mu=16, ptrs=None: f(ctypes.byref(a), kb, mu, *(ptrs or [FAKE] * 7), None,
                                            None)
    big = _abi.AttnDesc(400000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    assert ok(big) == -3                                # more scratch than the static array
    need = ctypes.c_size_t(0)
    assert lib.amtk_sparse_attn_workspace(ctypes.byref(big), ctypes.byref(need)) == 0
    assert need.value > _abi.AMTK_STATIC_SCRATCH_BYTES
    fits = _abi.AttnDesc(150000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    assert lib.amtk_sparse_attn_workspace(ctypes.byref(fits), ctypes.byref(need)) == 0
    assert need.value <= _abi.AMTK_STATIC_SCRATCH_BYTES
    assert ok(fits, kb=2) == -2
    assert ok(fits, mu=0) == -1
    for j in range(7):                                  # q, k, v, idx, count, o, (lse optional)
        ptrs = [FAKE] * 7
        ptrs[j] = None if j < 6 else ctypes.c_void_p(0x100002)
        assert ok(fits, ptrs=ptrs) == -1, j
    assert ok(_abi.AttnDesc(1000, 32, 8, 128, _abi.AMTK_BF16, 0, 0.0)) == -2


def test_diagnostics_validation(lib):
    odd = ctypes.c_void_p(0x100002)
    assert lib.captured_mass(0, 8, FAKE, FAKE, FAKE, None) == -1
    assert lib.captured_mass(10, 0, FAKE, FAKE, FAKE, None) == -1
    assert lib.captured_mass(10, 8, None, FAKE, FAKE, None) == -1
    assert lib.captured_mass(10, 8, FAKE, FAKE, odd, None) == -1
    assert lib.support_overlap(0, 4, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.support_overlap(10, 0, FAKE, FAKE, 4, FAKE, FAKE, FAKE, None) == -1
    assert lib.support_overlap(10, 4, FAKE, FAKE, 4, FAKE, None, FAKE, None) == -1
    assert lib.support_overlap(10, 4, FAKE, FAKE, 4, FAKE, FAKE, odd, None) == -1


def test_kl_distill_validation(lib):
    from sparse_long_context_causal_amd import _abi
    a, _ = _descs()                                     # fp32, d = 64: not the kernel's shape
    need = ctypes.c_size_t(0)
    assert lib.amtk_kl_workspace(ctypes.byref(a), 64, ctypes.byref(need)) == -2
    b = _abi.AttnDesc(1000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    assert lib.amtk_kl_workspace(ctypes.byref(b), 32, ctypes.byref(need)) == -2
    assert lib.amtk_kl_workspace(ctypes.byref(b), 0, ctypes.byref(need)) == -1
    assert lib.amtk_kl_workspace(ctypes.byref(b), 64, ctypes.byref(need)) == 0
    # dense LSE, student LSE, the key gradient's 8 per-KV-group shares and the
    # teacher pass's copy of K in MFMA operand order: linear in n (no n x
    # n-sized array)
    kops = (1000 + 31) // 32 * 32 * 8 * 128 * 2
    assert 1000 * (32 + 1 + 8 * 64) * 4 + kops <= need.value <= 1000 * (32 + 1 + 8 * 64) * 4 + kops + 4096
    big = _abi.AttnDesc(100000, 32, 8, 128, _abi.AMTK_BF16, 1, 0.0)
    need_big = ctypes.c_size_t(0)
    assert lib.amtk_kl_workspace(ctypes.byref(big), 64, ctypes.byref(need_big)) == 0
    assert need_big.value <= 100000 * (32 + 1 + 8 * 64) * 4 + (100000 + 31) // 32 * 65536 + 4096   # 423 MB at 100K
    # 4 query heads per KV head with fewer KV heads: one key-gradient share per KV head
    for hq, hkv in ((16, 4), (8, 2), (4, 1)):
        c = _abi.AttnDesc(1000, hq, hkv, 128, _abi.AMTK_BF16, 1, 0.0)
        assert lib.amtk_kl_workspace(ctypes.byref(c), 64, ctypes.byref(need)) == 0
        base = 1000 * (hq + 1 + hkv * 64) * 4 + (1000 + 31) // 32 * 32 * hkv * 128 * 2   # + key copy
        assert base <= need.value <= base + 4096
    for hq, hkv in ((16, 8), (32, 4), (8, 8)):   # other group sizes: not covered
        c = _abi.AttnDesc(1000, hq, hkv, 128, _abi.AMTK_BF16, 1, 0.0)
        assert lib.amtk_kl_workspace(ctypes.byref(c), 64, ctypes.byref(need)) == -2
    f = lib.kl_distill
    args = [FAKE] * 8
    assert f(ctypes.byref(b), 64, 0.0, *args, FAKE, need.value - 1, None) == -3
    assert f(ctypes.byref(b), 64, float("nan"), *args, FAKE, need.value, None) == -1
    bad = list(args)
    bad[4] = None                                       # kl_row
    assert f(ctypes.byref(b), 64, 0.0, *bad, FAKE, need.value, None) == -1


def test_indexer_validation(lib):
    _, s = _descs(kb=64, k=16)
    f = lib.indexer_topk
    assert f(0, 64, 0, 0.0, ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, None) == -1
    assert f(100, 32, 0, 0.0, ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, None) == -2
    need = ctypes.c_size_t(0)
    assert lib.amtk_indexer_workspace(100, 64, 0, ctypes.byref(s), ctypes.byref(need)) == 0
    assert f(100, 64, 0, 0.0, ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, FAKE,
             need.value - 1, None) == -3


def test_binding_fails_loudly_without_library(tmp_path):
    from sparse_long_context_causal_amd import _abi
    with pytest.raises(RuntimeError):
        _abi.open_library(str(tmp_path / "missing.so"))


def test_calibration_library_exports_its_two_kernels():
    """bench.py's measured ceilings come from libamtk_calib.so: the L2 read
    calibration and the passes' inner-loop compute ceiling."""
    from sparse_long_context_causal_amd import build
    if not os.path.exists(build.CALIB_LIB):
        build.build(verbose=False)
    out = subprocess.run(["nm", "-D", "--defined-only", build.CALIB_LIB], capture_output=True,
                         text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {"amtk_calib_l2_read", "amtk_calib_mix"} <= exported
    cal = ctypes.CDLL(build.CALIB_LIB)
    cal.amtk_calib_mix.restype = ctypes.c_int
    cal.amtk_calib_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    # rejected on the host before any HIP call
    assert cal.amtk_calib_mix(2, 1, 1, ctypes.c_void_p(16), None) != 0
    assert cal.amtk_calib_mix(0, 0, 1, ctypes.c_void_p(16), None) != 0
    assert cal.amtk_calib_mix(0, 1, 1, None, None) != 0
