"""GPU parity of the indexer's selection-block-shared support and of the
fused realisation (indexer_prefill with query_block = 64).

Supports: every row of a block must hold the same ids and count; the ids
pass the near-tie check (1e-6 band) against the oracle's block scores; the
masses are those scores (|diff| <= 1e-7 + 2e-4 * score). Outputs: each row
against the oracle's attention on the shared tokens up to the row (2e-3 max
abs, the bf16 output bar). The fused kernel must give exactly what its two
unfused halves give (indexer_topk + sparse_attn_blocks): same ids, same
outputs, bit for bit.
"""
import numpy as np
import pytest

from oracle import IndexerOracle, OracleLayer, tokens_of_blocks
from synth import WORKLOADS, generate, random_inputs, round_bf16
from tests.gpu_helpers import BAND, TOL_OUT, upload
from tests.support_rules import check_row

pytestmark = pytest.mark.gpu


def _idx_inputs(n, seed):
    rng = np.random.default_rng(seed)
    qi = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    ki = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    return qi, ki


def _t(a):
    import torch
    return torch.from_numpy(a).to(torch.bfloat16).cuda()


def _check_blocks(idx, cnt, mass, ix, n, k, blocks=None, key_block=64):
    nblk = (n + 63) // 64
    res = {}
    for t in (range(nblk) if blocks is None else blocks):
        r = ix.query_block(int(t), k, key_block, 64)
        rows = list(r["rows"])
        i0 = rows[0]
        for i in rows:
            assert cnt[i] == cnt[i0] and np.array_equal(idx[i], idx[i0]), f"row {i}"
        ok, msg, _ = check_row(idx[i0], cnt[i0], r["score"], r["kth"], k, BAND)
        assert ok, f"block {t}: {msg}"
        sel = idx[i0, : cnt[i0]]
        want = r["score"][sel]
        assert np.all(np.abs(mass[i0, : cnt[i0]] - want) <= 1e-7 + 2e-4 * want), f"block {t} mass"
        res[t] = sel
    return res


@pytest.mark.parametrize("n,k", [(200, 2), (650, 4), (130, 5), (64, 1)])
def test_indexer_query_blocks_small(gpu_lib, n, k):
    qi, ki = _idx_inputs(n, n + k)
    idx, cnt, mass = gpu_lib.indexer_topk(_t(qi), _t(ki), k, 64, query_block=64)
    _check_blocks(idx.cpu().numpy(), cnt.cpu().numpy(), mass.cpu().numpy(), IndexerOracle(qi, ki),
                  n, k)


def test_sparse_attn_blocks_key_blocks_oracle_supports(gpu_lib):
    """The block tile kernel over 64-token key blocks, driven by the oracle's
    indexer supports (the first row of each block only), every row checked."""
    import torch
    n, k = 300, 3
    x = random_inputs(n, 32, 8, 128, "bf16", seed=51, sink=True)
    qi, ki = _idx_inputs(n, 52)
    ix = IndexerOracle(qi, ki)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = np.full((n, k), -3, dtype=np.int32)
    cnt = np.full(n, 1, dtype=np.int32)
    sup = {}
    for t in range((n + 63) // 64):
        r = ix.query_block(t, k, 64, 64)
        idx[64 * t] = -1
        idx[64 * t, : r["units"].size] = r["units"]
        cnt[64 * t] = r["units"].size
        sup.update(r["support"])
    d = upload(x, "bf16")
    out, lse = gpu_lib.sparse_attn_blocks(d["q"], d["k"], d["v"], torch.from_numpy(idx).cuda(),
                                          torch.from_numpy(cnt).cuda(), 64, key_block=64,
                                          want_lse=True)
    out = out.cpu().numpy()
    for i in range(n):
        o_ref, _ = layer.attention_on(i, sup[i])
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"


@pytest.mark.parametrize("n,k", [(330, 3), (1000, 6)])
def test_indexer_prefill_fused_equals_unfused_and_oracle(gpu_lib, n, k):
    import torch
    amtk = gpu_lib
    x = random_inputs(n, 32, 8, 128, "bf16", seed=n + 7, sink=True)
    qi, ki = _idx_inputs(n, n + 8)
    d = upload(x, "bf16")
    tq, tk = _t(qi), _t(ki)
    out_f, idx_f, cnt_f, mass_f = amtk.indexer_prefill(d["q"], d["k"], d["v"], tq, tk, k, 64,
                                                       query_block=64)
    idx_u, cnt_u, mass_u = amtk.indexer_topk(tq, tk, k, 64, query_block=64)
    out_u, _ = amtk.sparse_attn_blocks(d["q"], d["k"], d["v"], idx_u, cnt_u, 64, key_block=64)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_u) and torch.equal(cnt_f, cnt_u) and torch.equal(mass_f, mass_u)
    assert torch.equal(out_f, out_u)
    ix = IndexerOracle(qi, ki)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    ii, cc = idx_f.cpu().numpy(), cnt_f.cpu().numpy()
    _check_blocks(ii, cc, mass_f.cpu().numpy(), ix, n, k)
    out = out_f.cpu().numpy()
    for i in range(0, n, 7):
        toks = tokens_of_blocks(ii[i, : cc[i]], 64, i)
        o_ref, _ = layer.attention_on(i, toks)
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"


def test_indexer_prefill_per_query_equals_its_parts(gpu_lib):
    import torch
    amtk = gpu_lib
    n, k = 400, 4
    x = random_inputs(n, 32, 8, 128, "bf16", seed=91, sink=True)
    qi, ki = _idx_inputs(n, 92)
    d = upload(x, "bf16")
    tq, tk = _t(qi), _t(ki)
    out_p, idx_p, cnt_p, _ = amtk.indexer_prefill(d["q"], d["k"], d["v"], tq, tk, k, 64)
    idx_u, cnt_u, _ = amtk.indexer_topk(tq, tk, k, 64)
    out_u, _ = amtk.sparse_attn(d["q"], d["k"], d["v"], idx_u, cnt_u, 64)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx_u) and torch.equal(cnt_p, cnt_u)
    assert torch.equal(out_p, out_u)


def test_indexer_prefill_fused_indexer_bf16_32k_sampled(gpu_lib):
    """The fused realisation on the indexer workload at its full size: seeded
    blocks' supports against the oracle, and rows of them against the oracle's
    attention on the shared tokens."""
    amtk = gpu_lib
    w = WORKLOADS["indexer_bf16_32k"]
    x = generate(w)
    d = upload(x, "bf16")
    out, idx, cnt, mass = amtk.indexer_prefill(d["q"], d["k"], d["v"], _t(x["q_idx"]),
                                               _t(x["k_idx"]), w.k, w.key_block, query_block=64)
    ii, cc = idx.cpu().numpy(), cnt.cpu().numpy()
    blocks = [0, 1, 100, 377, 511]
    ix = IndexerOracle(x["q_idx"], x["k_idx"])
    _check_blocks(ii, cc, mass.cpu().numpy(), ix, w.n, w.k, blocks)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    out = out.cpu().numpy()
    for t in blocks:
        for i in (64 * t, 64 * t + 17, 64 * t + 63):
            toks = tokens_of_blocks(ii[i, : cc[i]], 64, i)
            o_ref, _ = layer.attention_on(i, toks)
            err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
            assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"


@pytest.mark.parametrize("hq,hkv,kb,k", [
    (16, 2, 64, 4),     # 8 query heads per KV head, key blocks
    (8, 8, 64, 3),      # one query head per KV head
    (32, 8, 1, 100),    # the tile kernel's layout, but token units
])
def test_indexer_prefill_blocks_two_step(gpu_lib, hq, hkv, kb, k):
    """indexer_prefill with selection blocks where the fused kernel does not
    apply: the block support (as indexer_topk writes it), then the per-row
    gather. Bit for bit against those two calls; the supports against the
    oracle's block scores, the outputs against its attention on the shared
    tokens up to each row."""
    import torch
    amtk = gpu_lib
    n = 330
    x = random_inputs(n, hq, hkv, 128, "bf16", seed=hq + hkv + kb, sink=True)
    qi, ki = _idx_inputs(n, hq * 3 + kb)
    d = upload(x, "bf16")
    tq, tk = _t(qi), _t(ki)
    out_f, idx_f, cnt_f, mass_f = amtk.indexer_prefill(d["q"], d["k"], d["v"], tq, tk, k, kb,
                                                       query_block=64)
    idx_u, cnt_u, mass_u = amtk.indexer_topk(tq, tk, k, kb, query_block=64)
    out_u, _ = amtk.sparse_attn(d["q"], d["k"], d["v"], idx_u, cnt_u, kb)
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx_u) and torch.equal(cnt_f, cnt_u) and torch.equal(mass_f, mass_u)
    assert torch.equal(out_f, out_u)
    ix = IndexerOracle(qi, ki)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    ii, cc = idx_f.cpu().numpy(), cnt_f.cpu().numpy()
    _check_blocks(ii, cc, mass_f.cpu().numpy(), ix, n, k, key_block=kb)
    out = out_f.cpu().numpy()
    for i in range(0, n, 7):
        units = ii[i, : cc[i]]
        toks = tokens_of_blocks(units, kb, i) if kb > 1 else units[units <= i]
        o_ref, _ = layer.attention_on(i, toks)
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"


@pytest.mark.parametrize("hq,hkv,d,dtype", [
    (16, 2, 128, "bf16"),   # MFMA gather over key blocks, 8 query heads per KV head
    (8, 2, 64, "f32"),      # VALU gather
])
def test_sparse_attn_blocks_key_blocks_other_layouts(gpu_lib, hq, hkv, d, dtype):
    """sparse_attn_blocks over 64-token key blocks on layouts outside the tile
    kernel (the per-row gather reading each block's first index row), driven by
    the oracle's indexer supports: every row against the oracle's attention on
    the block's tokens up to the row, and bit for bit against sparse_attn on
    per-row copies."""
    import torch
    n, k = 300, 3
    x = random_inputs(n, hq, hkv, d, dtype, seed=53 + hq, sink=True)
    qi, ki = _idx_inputs(n, 54)
    ix = IndexerOracle(qi, ki)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = np.full((n, k), -3, dtype=np.int32)
    cnt = np.full(n, 1, dtype=np.int32)
    per_idx = np.full((n, k), -1, dtype=np.int32)
    per_cnt = np.zeros(n, dtype=np.int32)
    units = {}
    for t in range((n + 63) // 64):
        u = ix.query_block(t, k, 64, 64)["units"]
        units[t] = u
        idx[64 * t] = -1
        idx[64 * t, : u.size] = u
        cnt[64 * t] = u.size
        per_idx[64 * t: 64 * t + 64] = idx[64 * t]
        per_cnt[64 * t: 64 * t + 64] = u.size
    dv = upload(x, dtype)
    out, lse = gpu_lib.sparse_attn_blocks(dv["q"], dv["k"], dv["v"], torch.from_numpy(idx).cuda(),
                                          torch.from_numpy(cnt).cuda(), 64, key_block=64,
                                          want_lse=True)
    out_r, lse_r = gpu_lib.sparse_attn(dv["q"], dv["k"], dv["v"], torch.from_numpy(per_idx).cuda(),
                                       torch.from_numpy(per_cnt).cuda(), 64, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_r) and torch.equal(lse, lse_r)
    out = out.cpu().numpy()
    for i in range(n):
        o_ref, _ = layer.attention_on(i, tokens_of_blocks(units[i // 64], 64, i))
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        assert err <= TOL_OUT[dtype], f"row {i}: max abs err {err}"
