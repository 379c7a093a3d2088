"""Every output element is written: outputs are poisoned (NaN for floats, a
sentinel for ints) before each call through the C ABI, and no poison may
survive in the region the contract says is written (padding included).
Shapes with ragged tails (N not a multiple of 32 or 64)."""
import ctypes

import numpy as np
import pytest

from synth import random_inputs, round_bf16

pytestmark = pytest.mark.gpu

SENT = -777777


def _bf(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).cuda()


def _poisoned(shape, dtype):
    import torch
    if dtype == torch.int32:
        return torch.full(shape, SENT, dtype=torch.int32, device="cuda")
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def _clean(t):
    import torch
    t = t.cpu()
    if t.dtype == torch.int32:
        return not bool((t == SENT).any())
    return not bool(torch.isnan(t).any())


def _layer(n, seed):
    x = random_inputs(n, 32, 8, 128, "bf16", seed=seed, sink=True)
    return x, _bf(x["q"]), _bf(x["k"]), _bf(x["v"])


@pytest.mark.parametrize("n,k,kb,qb", [(1000, 40, 1, 1), (1000, 3, 64, 1), (1000, 40, 1, 64),
                                       (77, 100, 1, 1)])
def test_topk_support_writes_every_element(gpu_lib, n, k, kb, qb):
    import torch
    amtk = gpu_lib
    _, q, kk, _ = _layer(n, n + k)
    ad, sd = amtk.attn_desc(q, kk), amtk.support_desc(k, kb, 0, qb)
    ws = amtk.workspace(amtk.topk_workspace_bytes(ad, sd), q.device)
    idx, cnt = _poisoned((n, k), torch.int32), _poisoned((n,), torch.int32)
    mass, lse = _poisoned((n, k), torch.float32), _poisoned((32, n), torch.float32)
    amtk._call("topk_support", ctypes.byref(ad), ctypes.byref(sd), amtk._ptr(q), amtk._ptr(kk),
               amtk._ptr(idx), amtk._ptr(cnt), amtk._ptr(mass), amtk._ptr(lse), amtk._ptr(ws),
               ws.numel(), amtk._stream(q.device))
    torch.cuda.synchronize()
    for t in (idx, cnt, mass, lse):
        assert _clean(t)
    ii, cc = idx.cpu().numpy(), cnt.cpu().numpy()
    for i in range(n):
        assert np.all(ii[i, cc[i]:] == -1)


@pytest.mark.parametrize("kb", [1, 64])
def test_sparse_attn_writes_every_element(gpu_lib, kb):
    import torch
    amtk = gpu_lib
    n, k = 300, 8
    _, q, kk, v = _layer(n, 11 + kb)
    rng = np.random.default_rng(kb)
    units = n if kb == 1 else (n + 63) // 64
    idx = np.full((n, k), -1, dtype=np.int32)
    cnt = rng.integers(0, k + 1, n).astype(np.int32)
    for i in range(n):
        top = i if kb == 1 else i // 64
        idx[i, : cnt[i]] = rng.integers(0, top + 1, cnt[i])
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    ad = amtk.attn_desc(q, kk)
    o, lse = _poisoned((n, 32, 128), torch.float32), _poisoned((32, n), torch.float32)
    amtk._call("sparse_attn", ctypes.byref(ad), kb, k, amtk._ptr(q), amtk._ptr(kk), amtk._ptr(v),
               amtk._ptr(ti), amtk._ptr(tc), amtk._ptr(o), amtk._ptr(lse), amtk._stream(q.device))
    torch.cuda.synchronize()
    assert _clean(o)
    lc = lse.cpu()
    assert not bool(torch.isnan(lc).any())
    o2, lse2 = _poisoned((n, 32, 128), torch.float32), _poisoned((32, n), torch.float32)
    amtk._call("sparse_attn_blocks", ctypes.byref(ad), kb, 64, k, amtk._ptr(q), amtk._ptr(kk),
               amtk._ptr(v), amtk._ptr(ti), amtk._ptr(tc), amtk._ptr(o2), amtk._ptr(lse2),
               amtk._stream(q.device))
    torch.cuda.synchronize()
    assert _clean(o2) and not bool(torch.isnan(lse2.cpu()).any())


@pytest.mark.parametrize("kb", [1, 64])
def test_sparse_attn_windowed_writes_every_element(gpu_lib, kb):
    """Two key windows (N = 9000): rows with empty supports, rows whose ids all
    lie in the second window, rows in random order."""
    import torch
    amtk = gpu_lib
    n, k = 9000, 8
    _, q, kk, v = _layer(n, 41 + kb)
    rng = np.random.default_rng(40 + kb)
    idx = np.full((n, k), -1, dtype=np.int32)
    cnt = rng.integers(0, k + 1, n).astype(np.int32)
    for i in range(n):
        top = i if kb == 1 else i // 64
        lo = 8192 // kb if (i % 3 == 0 and top >= 8192 // kb) else 0   # second window only
        idx[i, : cnt[i]] = np.sort(rng.integers(lo, top + 1, cnt[i]))
        if i % 7 == 0:
            rng.shuffle(idx[i, : cnt[i]])
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    ad = amtk.attn_desc(q, kk)
    ws = amtk.workspace(amtk.sparse_attn_workspace_bytes(ad), q.device)
    o, lse = _poisoned((n, 32, 128), torch.float32), _poisoned((32, n), torch.float32)
    amtk._call("sparse_attn_windowed", ctypes.byref(ad), kb, k, amtk._ptr(q), amtk._ptr(kk),
               amtk._ptr(v), amtk._ptr(ti), amtk._ptr(tc), amtk._ptr(o), amtk._ptr(lse),
               amtk._ptr(ws), ws.numel(), amtk._stream(q.device))
    torch.cuda.synchronize()
    assert _clean(o) and not bool(torch.isnan(lse.cpu()).any())
    o1, _ = amtk.sparse_attn(q, kk, v, ti, tc, kb)
    torch.cuda.synchronize()
    assert float((o1 - o).abs().max()) <= 1.5e-4


@pytest.mark.parametrize("qb", [1, 64])
def test_indexer_paths_write_every_element(gpu_lib, qb):
    import torch
    amtk = gpu_lib
    n, k = 700, 4
    _, q, kk, v = _layer(n, 21 + qb)
    rng = np.random.default_rng(qb)
    qi = _bf(round_bf16(rng.standard_normal((n, 64)).astype(np.float32)))
    ki = _bf(round_bf16(rng.standard_normal((n, 64)).astype(np.float32)))
    sd = amtk.support_desc(k, 64, 0, qb)
    ws = amtk.workspace(amtk.indexer_workspace_bytes(n, 64, 0, sd), q.device)
    idx, cnt, mass = _poisoned((n, k), torch.int32), _poisoned((n,), torch.int32), _poisoned((n, k), torch.float32)
    amtk._call("indexer_topk", n, 64, 0, ctypes.c_float(0.0), ctypes.byref(sd), amtk._ptr(qi),
               amtk._ptr(ki), amtk._ptr(idx), amtk._ptr(cnt), amtk._ptr(mass), amtk._ptr(ws),
               ws.numel(), amtk._stream(q.device))
    torch.cuda.synchronize()
    assert _clean(idx) and _clean(cnt) and _clean(mass)
    ad = amtk.attn_desc(q, kk)
    o = _poisoned((n, 32, 128), torch.float32)
    idx2, cnt2, mass2 = _poisoned((n, k), torch.int32), _poisoned((n,), torch.int32), _poisoned((n, k), torch.float32)
    amtk._call("indexer_prefill", ctypes.byref(ad), 64, ctypes.c_float(0.0), ctypes.byref(sd),
               amtk._ptr(q), amtk._ptr(kk), amtk._ptr(v), amtk._ptr(qi), amtk._ptr(ki), amtk._ptr(o),
               amtk._ptr(idx2), amtk._ptr(cnt2), amtk._ptr(mass2), amtk._ptr(ws), ws.numel(),
               amtk._stream(q.device))
    torch.cuda.synchronize()
    for t in (o, idx2, cnt2, mass2):
        assert _clean(t)


def test_kl_and_diagnostics_write_every_element(gpu_lib):
    import torch
    amtk = gpu_lib
    n = 161
    _, q, kk, v = _layer(n, 31)
    rng = np.random.default_rng(31)
    qi = _bf(round_bf16(rng.standard_normal((n, 64)).astype(np.float32)))
    ki = _bf(round_bf16(rng.standard_normal((n, 64)).astype(np.float32)))
    ad = amtk.attn_desc(q, kk)
    ws = amtk.workspace(amtk.kl_workspace_bytes(ad, 64), q.device)
    kl, loss = _poisoned((n,), torch.float32), _poisoned((1,), torch.float32)
    dq, dk = _poisoned((n, 64), torch.float32), _poisoned((n, 64), torch.float32)
    amtk._call("kl_distill", ctypes.byref(ad), 64, ctypes.c_float(0.0), amtk._ptr(q), amtk._ptr(kk),
               amtk._ptr(qi), amtk._ptr(ki), amtk._ptr(kl), amtk._ptr(loss), amtk._ptr(dq),
               amtk._ptr(dk), amtk._ptr(ws), ws.numel(), amtk._stream(q.device))
    torch.cuda.synchronize()
    for t in (kl, loss, dq, dk):
        assert _clean(t)
    idx, cnt, _, lse = amtk.topk_support(q, kk, 9)
    _, lse_s = amtk.sparse_attn(q, kk, v, idx, cnt, 1, want_lse=True)
    cap, ov = _poisoned((n,), torch.float32), _poisoned((n,), torch.int32)
    amtk._call("captured_mass", n, 32, amtk._ptr(lse), amtk._ptr(lse_s), amtk._ptr(cap),
               amtk._stream(q.device))
    amtk._call("support_overlap", n, 9, amtk._ptr(idx), amtk._ptr(cnt), 9, amtk._ptr(idx),
               amtk._ptr(cnt), amtk._ptr(ov), amtk._stream(q.device))
    torch.cuda.synchronize()
    assert _clean(cap) and _clean(ov)
    assert np.array_equal(ov.cpu().numpy(), cnt.cpu().numpy())   # a support overlaps itself fully
