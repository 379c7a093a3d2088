"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Index sets must match except within 1e-6 of the k-th mass; outputs on
identical supports within 2e-3 (bf16 inputs) / 1e-5 (fp32 inputs) max abs;
per-head LSE within 1e-4 / 1e-5; masses within 1e-7 + 2e-4 * P.
Small shapes are compared on every row (several 32-row tiles and a ragged
tail); the full-size workloads on the seeded oracle row samples, in the same
launch configuration the benchmark times.
"""
import math

import numpy as np
import pytest

from oracle import OracleLayer, IndexerOracle, tokens_of_blocks
from synth import WORKLOADS, generate, random_inputs, round_bf16, sample_rows
from tests.support_rules import check_row
from tests.gpu_helpers import (BAND, TOL_LSE, TOL_OUT, check_outputs_on_gpu_support,
                               check_support_rows, upload)

pytestmark = pytest.mark.gpu


def _run_oracle_prefill(amtk, x, dtype, k, key_block=1, cap=0):
    import torch
    d = upload(x, dtype)
    out, idx, count, mass, lse = amtk.oracle_prefill(d["q"], d["k"], d["v"], k, key_block,
                                                     candidate_cap=cap)
    torch.cuda.synchronize()
    return {"out": out.cpu().numpy(), "idx": idx.cpu().numpy(), "count": count.cpu().numpy(),
            "mass": mass.cpu().numpy(), "lse": lse.cpu().numpy()}


def _full_check(amtk, x, dtype, k, key_block=1, rows=None, cap=0):
    layer = OracleLayer(x["q"], x["k"], x["v"])
    res = _run_oracle_prefill(amtk, x, dtype, k, key_block, cap)
    n = x["q"].shape[0]
    rows = np.arange(n) if rows is None else rows
    for i in rows:
        r = layer.row(int(i), k, key_block)
        assert np.max(np.abs(res["lse"][:, i] - r["lse"])) <= TOL_LSE[dtype], f"lse row {i}"
        sel = res["idx"][i][: res["count"][i]]
        want = r["score"][sel]
        assert np.all(np.abs(res["mass"][i][: res["count"][i]] - want) <= 1e-7 + 2e-4 * want), \
            f"mass row {i}"
    check_support_rows(res["idx"], res["count"], layer, rows, k, key_block)
    check_outputs_on_gpu_support(res["out"], None, layer, rows, res["idx"], res["count"],
                                 key_block, dtype)
    return res, layer


# ------------------------------------------------------------ small shapes
@pytest.mark.parametrize("n,hq,hkv,d,dtype,k", [
    (1, 8, 2, 64, "f32", 4),        # one token
    (33, 8, 2, 64, "f32", 5),       # ragged second tile
    (200, 8, 2, 64, "f32", 32),
    (150, 32, 8, 128, "bf16", 12),
    (300, 4, 1, 128, "bf16", 20),   # MQA
    (130, 4, 4, 128, "bf16", 7),    # MHA (G = 1)
    (97, 16, 8, 128, "bf16", 9),    # G = 2
    (161, 8, 1, 64, "bf16", 11),    # G = 8, d = 64
    (90, 4, 2, 128, "f32", 6),      # fp32, d = 128
    (110, 8, 4, 128, "bf16", 8),    # G = 2, four KV heads
    (99, 8, 8, 128, "bf16", 10),    # G = 1 with eight KV heads (key tiles loaded straight to registers)
])
def test_small_shapes_all_rows(gpu_lib, n, hq, hkv, d, dtype, k):
    x = random_inputs(n, hq, hkv, d, dtype, seed=n * 7 + hq, sink=True)
    _full_check(gpu_lib, x, dtype, k)


def test_budget_at_least_row_length_is_dense(gpu_lib):
    import torch
    n = 96
    x = random_inputs(n, 8, 2, 128, "bf16", seed=5, sink=True)
    res = _run_oracle_prefill(gpu_lib, x, "bf16", n)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in range(n):
        assert res["count"][i] == i + 1
        assert res["idx"][i][: i + 1].tolist() == list(range(i + 1))
        assert np.all(res["idx"][i][i + 1:] == -1)
        assert np.max(np.abs(res["out"][i] - layer.dense(i))) <= TOL_OUT["bf16"]


@pytest.mark.parametrize("n,hq,hkv,d,dtype", [
    (9000, 32, 8, 128, "bf16"),   # MFMA passes with direct key tiles, windowed MFMA gather (2 windows)
    (8300, 8, 2, 64, "f32"),      # fp32 passes, VALU gather
])
def test_largest_budget(gpu_lib, n, hq, hkv, d, dtype):
    """The largest budget the select sorts (k = 8192 tokens): rows up to
    8191 keep every visible key, later rows the exact top 8192 of up to
    9000, which the select's LDS cannot stage (global-memory radix path)."""
    k = 8192                      # the header's upper limit of k
    x = random_inputs(n, hq, hkv, d, dtype, seed=n + hq, sink=True)
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([[0, 1, 31, k - 2, k - 1, k, k + 1, n - 2, n - 1],
                                     rng.integers(k, n, 5), rng.integers(0, k, 3)]))
    res, _ = _full_check(gpu_lib, x, dtype, k, rows=rows)
    for i in rows:
        assert res["count"][i] == min(i + 1, k)
        if i < k:
            assert res["idx"][i][: i + 1].tolist() == list(range(i + 1))
            assert np.all(res["idx"][i][i + 1:] == -1)


@pytest.mark.parametrize("n", [120, 3000])   # 3000: rows keep more than the select's LDS holds
def test_equal_keys_tie_to_smallest_ids(gpu_lib, n):
    hq, hkv, d = 8, 2, 64
    rng = np.random.default_rng(3)
    q = rng.standard_normal((n, hq, d)).astype(np.float32)
    k = np.broadcast_to(rng.standard_normal((1, hkv, d)), (n, hkv, d)).astype(np.float32).copy()
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    res = _run_oracle_prefill(gpu_lib, {"q": q, "k": k, "v": v}, "f32", 10)
    for i in range(n):
        assert res["idx"][i][: res["count"][i]].tolist() == list(range(min(10, i + 1)))


def _class_keys(n, hq, hkv, d, probs, logits, seed):
    """Every key is one of a few class vectors (a class per token), and every
    query head points along its KV head's direction, so row i's logits are
    about logits[c] for a key of class c, identical within a class, and the
    classes' masses sit a factor e apart."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((hkv, d))
    w /= np.linalg.norm(w, axis=1, keepdims=True)
    cls = rng.choice(len(probs), size=n, p=probs)
    t = np.asarray(logits, dtype=np.float64)
    k = (t[cls][:, None, None] * w[None]).astype(np.float32)
    g_of_h = np.arange(hq) // (hq // hkv)
    q = (np.sqrt(d) * w[g_of_h][None] + 0.05 * rng.standard_normal((n, hq, d))).astype(np.float32)
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    return {"q": q, "k": k, "v": v}, cls


@pytest.mark.parametrize("n,k,probs", [
    (4000, 300, [0.02, 0.03, 0.45, 0.5]),
    (5000, 700, [0.02, 0.10, 0.45, 0.43]),
])
def test_key_classes_exact_supports(gpu_lib, n, k, probs):
    """Supports follow from the construction: whole classes in order of
    logit, then the smallest ids of the class holding the k-th unit. Long
    rows keep whole classes beyond what the select's LDS holds, short ones
    fit; both select paths see several distinct masses and exact ties."""
    logits = [3.0, 2.0, 1.0, 0.0]
    x, cls = _class_keys(n, 8, 2, 64, probs, logits, seed=n + k)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in (n // 3, n - 1):   # the construction's class order holds in the oracle
        sc = layer.row(i, k)["score"]
        per = [sc[np.nonzero(cls[: i + 1] == c)[0]] for c in range(4)]
        assert all(p.size and np.ptp(p) <= 1e-12 * p.max() for p in per)
        assert per[0][0] > per[1][0] > per[2][0] > per[3][0]
    res = _run_oracle_prefill(gpu_lib, x, "f32", k)
    for i in range(n):
        want = []
        for c in range(4):
            ids = np.nonzero(cls[: i + 1] == c)[0]
            want.extend(ids[: k - len(want)].tolist())
            if len(want) == k:
                break
        want = sorted(want)
        assert res["count"][i] == len(want), f"row {i}"
        assert res["idx"][i][: len(want)].tolist() == want, f"row {i}"


@pytest.mark.parametrize("dtype,hq,hkv,d", [
    ("f32", 8, 2, 64),
    ("bf16", 8, 2, 64),
    ("bf16", 32, 8, 128),   # pass 1 from the keys in operand order (its redo path)
])
def test_lse_far_above_first_key_tile(gpu_lib, dtype, hq, hkv, d):
    """One key (id 100) scores about 180 log2 units above every key of the
    first 32-key tile, so a sum referenced to the first tile's maximum would
    overflow; rows that see it must still match the oracle (their LSE is
    about 125, so fp32 keeps ~1e-5 there: the check allows 4 ulp on top)."""
    n = 200
    rng = np.random.default_rng(77)
    e0 = np.zeros(d)
    e0[0] = 1.0
    q = (25.0 * e0 + 0.01 * rng.standard_normal((n, hq, d))).astype(np.float32)
    k = rng.standard_normal((n, hkv, d)).astype(np.float32)
    k[100] = 40.0 * math.sqrt(d / 64) * e0   # the same logit, 125 (180 log2 units), at any d
    v = rng.standard_normal((n, hkv, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    x = {"q": q, "k": k, "v": v}
    layer = OracleLayer(q, k, v)
    res = _run_oracle_prefill(gpu_lib, x, dtype, 8)
    for i in range(n):
        ref = layer.row(i, 8)["lse"]
        tol = TOL_LSE[dtype] + 4 * np.spacing(np.abs(ref).astype(np.float32))
        assert np.all(np.abs(res["lse"][:, i] - ref) <= tol), f"lse row {i}"
    assert np.all(res["idx"][100:, :8] >= 0) and np.all(np.any(res["idx"][100:] == 100, axis=1))
    check_support_rows(res["idx"], res["count"], layer, np.arange(n), 8)
    check_outputs_on_gpu_support(res["out"], None, layer, np.arange(0, n, 3), res["idx"],
                                 res["count"], 1, dtype)


def test_overflow_path_gives_same_supports(gpu_lib):
    """A tiny candidate capacity forces the dense per-row recompute."""
    x = random_inputs(260, 8, 2, 128, "bf16", seed=11, sink=True)
    a = _run_oracle_prefill(gpu_lib, x, "bf16", 16)
    b = _run_oracle_prefill(gpu_lib, x, "bf16", 16, cap=17)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    check_support_rows(b["idx"], b["count"], layer, np.arange(260), 16)
    assert np.array_equal(a["count"], b["count"])
    same = np.mean([np.array_equal(a["idx"][i], b["idx"][i]) for i in range(260)])
    assert same > 0.98
    check_outputs_on_gpu_support(b["out"], None, layer, np.arange(0, 260, 7), b["idx"],
                                 b["count"], 1, "bf16")


def test_overflow_path_eight_kv_heads(gpu_lib):
    """The same with 8 KV heads, bf16, d = 128 (pass 2's key tiles come from the
    workspace copy in operand order; rows whose pools overflow are redone densely)."""
    x = random_inputs(230, 32, 8, 128, "bf16", seed=13, sink=True)
    a = _run_oracle_prefill(gpu_lib, x, "bf16", 12)
    b = _run_oracle_prefill(gpu_lib, x, "bf16", 12, cap=13)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    check_support_rows(b["idx"], b["count"], layer, np.arange(230), 12)
    assert np.array_equal(a["count"], b["count"])
    same = np.mean([np.array_equal(a["idx"][i], b["idx"][i]) for i in range(230)])
    assert same > 0.98


def test_overflow_rows_are_reported(gpu_lib):
    import torch
    amtk = gpu_lib
    x = random_inputs(300, 8, 2, 64, "bf16", seed=12)
    d = upload(x, "bf16")
    ad, sd = amtk.attn_desc(d["q"], d["k"]), amtk.support_desc(8, 1, 9)
    ws = amtk.workspace(amtk.topk_workspace_bytes(ad, sd), d["q"].device)
    amtk.topk_support(d["q"], d["k"], 8, 1, candidate_cap=9, ws=ws)
    mx, ov, cap = amtk.pool_stats(ad, sd, ws)
    assert cap == 9 and mx > 9 and ov > 0
    sd2 = amtk.support_desc(8, 1, 0)
    ws2 = amtk.workspace(amtk.topk_workspace_bytes(ad, sd2), d["q"].device)
    amtk.topk_support(d["q"], d["k"], 8, 1, ws=ws2)
    mx2, ov2, cap2 = amtk.pool_stats(ad, sd2, ws2)
    assert ov2 == 0 and mx2 <= cap2


def test_key_block_support(gpu_lib):
    x = random_inputs(700, 8, 2, 128, "bf16", seed=21, sink=True)
    _full_check(gpu_lib, x, "bf16", 3, key_block=64)


def test_key_block_support_overflow_path(gpu_lib):
    x = random_inputs(700, 8, 2, 64, "f32", seed=22, sink=True)
    _full_check(gpu_lib, x, "f32", 2, key_block=64, cap=2)


def test_repeatable_bitwise(gpu_lib):
    x = random_inputs(400, 32, 8, 128, "bf16", seed=31, sink=True)
    a = _run_oracle_prefill(gpu_lib, x, "bf16", 24)
    for _ in range(2):
        b = _run_oracle_prefill(gpu_lib, x, "bf16", 24)
        for key in a:
            assert np.array_equal(a[key], b[key]), key


def test_sparse_attn_given_oracle_supports(gpu_lib):
    """K3 alone, driven by the oracle's supports (independent of K1/K2)."""
    import torch
    amtk = gpu_lib
    n, k = 257, 19
    x = random_inputs(n, 32, 8, 128, "bf16", seed=41, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = -np.ones((n, k), dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    for i in range(n):
        u = layer.row(i, k)["units"]
        idx[i, : u.size] = u
        cnt[i] = u.size
    d = upload(x, "bf16")
    out, lse_s = amtk.sparse_attn(d["q"], d["k"], d["v"], torch.from_numpy(idx).cuda(),
                                  torch.from_numpy(cnt).cuda(), 1, want_lse=True)
    check_outputs_on_gpu_support(out.cpu().numpy(), lse_s.cpu().numpy(), layer, range(n), idx,
                                 cnt, 1, "bf16")


def test_sparse_attn_one_token_and_empty(gpu_lib):
    import torch
    amtk = gpu_lib
    n = 40
    x = random_inputs(n, 8, 2, 64, "f32", seed=42)
    idx = np.full((n, 3), -1, dtype=np.int32)
    cnt = np.ones(n, dtype=np.int32)
    idx[:, 0] = np.arange(n) // 2
    cnt[5] = 0
    d = upload(x, "f32")
    out, lse = amtk.sparse_attn(d["q"], d["k"], d["v"], torch.from_numpy(idx).cuda(),
                                torch.from_numpy(cnt).cuda(), 1, want_lse=True)
    out = out.cpu().numpy()
    for i in range(n):
        if i == 5:
            assert np.all(out[i] == 0) and np.all(np.isneginf(lse.cpu().numpy()[:, i]))
            continue
        for h in range(8):
            np.testing.assert_array_equal(out[i, h], x["v"][i // 2, h // 4])


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (16, 8), (64, 8), (8, 1), (64, 16), (16, 16)])
@pytest.mark.parametrize("key_block,max_units", [(1, 48), (64, 48), (1, 200)])
def test_sparse_attn_mfma_unsorted_invalid_and_clamped(gpu_lib, key_block, max_units, hq, hkv):
    """The MFMA path (bf16, d=128; 1, 2, 4 or 8 query heads per KV head) on
    hand-made supports: ids in random order (the running maximum moves late),
    negative ids and ids past the row mixed in, counts above max_units
    (clamped), empty rows. Every row is checked against the oracle on the ids
    the contract keeps. Token supports of up to 48 units take 16-token
    chunks; 200 units take 32-token chunks (ids two chunks ahead), with every
    chunk count from 0 to 7 among the rows."""
    import torch
    amtk = gpu_lib
    n = 300
    rng = np.random.default_rng(77 + key_block)
    x = random_inputs(n, hq, hkv, 128, "bf16", seed=43 + hq + hkv, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = np.full((n, max_units), -1, dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    for i in range(n):
        top = i if key_block == 1 else i // key_block
        m = int(rng.integers(0, max_units + 12))          # up to 11 past max_units
        ids = rng.permutation(top + 1)[: max(0, m - 3)].tolist()
        ids += [-1, top + 1 + int(rng.integers(0, 5)), -7][: m - len(ids)]
        ids = rng.permutation(np.asarray(ids, dtype=np.int64)).tolist() if ids else []
        idx[i, : min(len(ids), max_units)] = ids[:max_units]
        cnt[i] = m
    cnt[7] = 0
    cnt[150] = 0
    d = upload(x, "bf16")
    out, lse = amtk.sparse_attn(d["q"], d["k"], d["v"], torch.from_numpy(idx).cuda(),
                                torch.from_numpy(cnt).cuda(), key_block, want_lse=True)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in range(n):
        kept = [int(u) for u in idx[i, : min(int(cnt[i]), max_units)] if u >= 0]
        if key_block == 1:
            toks = [j for j in kept if j <= i]
        else:
            toks = [j for b in kept for j in range(b * 64, b * 64 + 64) if j <= i]
        if not toks:
            assert np.all(out[i] == 0) and np.all(np.isneginf(lse[:, i])), f"row {i}"
            continue
        o_ref, l_ref = layer.attention_on(i, toks)
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"
        assert np.max(np.abs(lse[:, i] - l_ref)) <= TOL_LSE["bf16"], f"row {i} lse"


# ------------------------------------------------ selection-block-shared support
def _check_query_blocks(amtk, x, dtype, k, blocks=None, b_sel=64):
    """oracle_prefill with query_block = b_sel against the oracle's block
    supports: every row of a block carries the block's support, the support
    passes the near-tie check against the block scores, the masses are the
    block scores, and each row's output matches the oracle on the shared
    keys up to that row."""
    from tests.support_rules import check_row
    layer = OracleLayer(x["q"], x["k"], x["v"])
    d_ = upload(x, dtype)
    out, idx, count, mass, _ = amtk.oracle_prefill(d_["q"], d_["k"], d_["v"], k,
                                                   query_block=b_sel)
    out, idx = out.cpu().numpy(), idx.cpu().numpy()
    count, mass = count.cpu().numpy(), mass.cpu().numpy()
    n = x["q"].shape[0]
    nblk = (n + b_sel - 1) // b_sel
    for t in (range(nblk) if blocks is None else blocks):
        r = layer.query_block(int(t), k, b_sel)
        rows = list(r["rows"])
        i0 = rows[0]
        for i in rows:
            assert count[i] == count[i0] and np.array_equal(idx[i], idx[i0]), f"row {i}"
        ok, msg, _ = check_row(idx[i0], count[i0], r["score"], r["kth"], k)
        assert ok, f"block {t}: {msg}"
        sel = idx[i0, : count[i0]]
        np.testing.assert_allclose(mass[i0, : count[i0]], r["score"][sel], rtol=2e-4, atol=1e-7)
        for i in rows:
            sup = sel[sel <= i]
            if sup.size == 0:
                assert np.all(out[i] == 0), f"row {i}"
                continue
            o_ref, _ = layer.attention_on(i, sup)
            err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
            assert err <= TOL_OUT[dtype], f"row {i}: max abs err {err}"


@pytest.mark.parametrize("n,hq,hkv,d,dtype,k", [
    (200, 8, 2, 64, "f32", 12),      # 4 blocks, the last with 8 rows
    (330, 32, 8, 128, "bf16", 40),   # the MFMA attention path, last block 10 rows
    (129, 4, 4, 64, "bf16", 70),     # budgets above the first blocks' key counts
    (64, 2, 1, 128, "f32", 5),       # one block
])
def test_query_blocks_small_shapes(gpu_lib, n, hq, hkv, d, dtype, k):
    x = random_inputs(n, hq, hkv, d, dtype, seed=n + k, sink=True)
    _check_query_blocks(gpu_lib, x, dtype, k)


def test_query_blocks_mid_bf16_4k_sampled(gpu_lib):
    w = WORKLOADS["mid_bf16_4k"]
    x = generate(w)
    _check_query_blocks(gpu_lib, x, "bf16", w.k, blocks=[0, 1, 7, 30, 63])


def test_query_blocks_long_bf16_32k_sampled(gpu_lib):
    w = WORKLOADS["long_bf16_32k"]
    x = generate(w)
    _check_query_blocks(gpu_lib, x, "bf16", w.k, blocks=[3, 170, 511])


def test_sparse_attn_blocks_oracle_supports(gpu_lib):
    """The block tile kernel alone, on the oracle's own block supports: every
    row against the oracle's output and support LSE. Only the first row of a
    block carries the support (the others hold junk the kernel must not read)."""
    import torch
    amtk = gpu_lib
    n, k = 330, 40                      # 6 blocks, the last with 10 rows; 2 chunks of keys
    x = random_inputs(n, 32, 8, 128, "bf16", seed=44, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = np.full((n, k), -5, dtype=np.int32)
    cnt = np.full(n, 7, dtype=np.int32)
    res = {}
    for t in range((n + 63) // 64):
        r = layer.query_block(t, k, 64)
        res[t] = r
        u = r["units"]
        idx[64 * t, :] = -1
        idx[64 * t, : u.size] = u
        cnt[64 * t] = u.size
    d = upload(x, "bf16")
    out, lse = amtk.sparse_attn_blocks(d["q"], d["k"], d["v"], torch.from_numpy(idx).cuda(),
                                       torch.from_numpy(cnt).cuda(), 64, want_lse=True)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in range(n):
        r = res[i // 64]
        err = float(np.max(np.abs(out[i].astype(np.float64) - r["out"][i])))
        assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"
        if np.all(np.isneginf(r["lse_s"][i])):
            assert np.all(np.isneginf(lse[:, i])), f"row {i} lse"
        else:
            assert np.max(np.abs(lse[:, i] - r["lse_s"][i])) <= TOL_LSE["bf16"], f"row {i} lse"


@pytest.mark.parametrize("hq,hkv,d,dtype", [
    (16, 2, 128, "bf16"),   # MFMA gather, 8 query heads per KV head
    (8, 8, 128, "bf16"),    # MFMA gather, one query head per KV head
    (8, 2, 64, "f32"),      # VALU gather
])
def test_sparse_attn_blocks_other_layouts(gpu_lib, hq, hkv, d, dtype):
    """Head layouts outside the block tile kernel run the per-row gather, each
    row reading its block's first index row (the other rows hold junk): every
    row against the oracle's block outputs and support LSE, and bit for bit
    against sparse_attn on per-row copies of the block supports."""
    import torch
    amtk = gpu_lib
    n, k = 330, 40                      # 6 blocks, the last with 10 rows
    x = random_inputs(n, hq, hkv, d, dtype, seed=hq * 10 + hkv, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = np.full((n, k), -5, dtype=np.int32)
    cnt = np.full(n, 7, dtype=np.int32)
    per_idx = np.full((n, k), -1, dtype=np.int32)
    per_cnt = np.zeros(n, dtype=np.int32)
    res = {}
    for t in range((n + 63) // 64):
        r = layer.query_block(t, k, 64)
        res[t] = r
        u = r["units"]
        idx[64 * t, :] = -1
        idx[64 * t, : u.size] = u
        cnt[64 * t] = u.size
        per_idx[64 * t: 64 * t + 64] = idx[64 * t]
        per_cnt[64 * t: 64 * t + 64] = u.size
    dv = upload(x, dtype)
    out, lse = amtk.sparse_attn_blocks(dv["q"], dv["k"], dv["v"], torch.from_numpy(idx).cuda(),
                                       torch.from_numpy(cnt).cuda(), 64, want_lse=True)
    out_r, lse_r = amtk.sparse_attn(dv["q"], dv["k"], dv["v"], torch.from_numpy(per_idx).cuda(),
                                    torch.from_numpy(per_cnt).cuda(), want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_r) and torch.equal(lse, lse_r)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in range(n):
        r = res[i // 64]
        err = float(np.max(np.abs(out[i].astype(np.float64) - r["out"][i])))
        assert err <= TOL_OUT[dtype], f"row {i}: max abs err {err}"
        if np.all(np.isneginf(r["lse_s"][i])):
            assert np.all(np.isneginf(lse[:, i])), f"row {i} lse"
        else:
            assert np.max(np.abs(lse[:, i] - r["lse_s"][i])) <= TOL_LSE[dtype], f"row {i} lse"


def test_sparse_attn_blocks_unsorted_invalid_and_clamped(gpu_lib):
    """The block tile kernel on hand-made block supports: ids in random order,
    negative ids, ids past n and past the rows mixed in, a count above
    max_units (clamped), an empty block, a block whose keys all lie after
    its first 40 rows (those rows get zeros), a single-chunk block. Every row
    against the oracle on the ids the contract keeps."""
    import torch
    amtk = gpu_lib
    n, max_units = 300, 100             # 5 blocks, the last with 44 rows; up to 4 chunks
    rng = np.random.default_rng(91)
    x = random_inputs(n, 32, 8, 128, "bf16", seed=45, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    idx = np.full((n, max_units), -1, dtype=np.int32)
    cnt = np.zeros(n, dtype=np.int32)
    blocks = {}
    for t in range(5):
        i0, i1 = 64 * t, min(64 * t + 63, n - 1)
        if t == 0:
            ids = rng.permutation(i1 + 1)[:20].tolist()                     # one chunk
        elif t == 2:
            ids = (i0 + 40 + rng.permutation(i1 - i0 - 39)).tolist()        # after row i0+39
        else:
            ids = rng.permutation(i1 + 1)[:90].tolist() + [-1, n + 3, -7, i1 + 1, 2 ** 30]
            ids = rng.permutation(np.asarray(ids, dtype=np.int64)).tolist()
        c = len(ids)
        if t == 3:
            c = max_units + 9                                               # clamped
        if t == 4:
            ids, c = [], 0
        idx[i0, : min(len(ids), max_units)] = ids[:max_units]
        cnt[i0] = c
        blocks[t] = [int(u) for u in idx[i0, : min(c, max_units)] if 0 <= u < n]
    d = upload(x, "bf16")
    out, lse = amtk.sparse_attn_blocks(d["q"], d["k"], d["v"], torch.from_numpy(idx).cuda(),
                                       torch.from_numpy(cnt).cuda(), 64, want_lse=True)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for i in range(n):
        toks = [j for j in blocks[i // 64] if j <= i]
        if not toks:
            assert np.all(out[i] == 0) and np.all(np.isneginf(lse[:, i])), f"row {i}"
            continue
        o_ref, l_ref = layer.attention_on(i, toks)
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        assert err <= TOL_OUT["bf16"], f"row {i}: max abs err {err}"
        assert np.max(np.abs(lse[:, i] - l_ref)) <= TOL_LSE["bf16"], f"row {i} lse"


# ------------------------------------------------------------ the workloads
_GEN_CACHE = {}


def _generated(name):
    """Each workload's inputs are generated once per test session (the 100K
    layer takes seconds to build); only the latest one is kept."""
    if name not in _GEN_CACHE:
        _GEN_CACHE.clear()
        _GEN_CACHE[name] = generate(WORKLOADS[name])
    return _GEN_CACHE[name]


def _workload_check(amtk, name, k=None):
    """The whole seeded oracle row sample of a workload (every row at 512 and
    4096 tokens, 256 rows at 32K, 128 at 100K), in the launch configuration
    the benchmark times (oracle_prefill): per-head LSE, selected masses,
    supports by the near-tie rule, outputs on the GPU's own supports, and
    every surviving planted needle of a checked row selected."""
    w = WORKLOADS[name]
    x = _generated(name)
    rows = sample_rows(w)
    k = w.k if k is None else k
    res, layer = _full_check(amtk, x, w.dtype, k, w.key_block, rows=rows)
    owners = x["owner"]
    lost = []
    n_needles = 0
    for i in rows:
        mine = np.nonzero(owners == i)[0]
        n_needles += mine.size
        sel = set(res["idx"][i][: res["count"][i]].tolist())
        if not set(mine.tolist()) <= sel:
            lost.append(int(i))
    assert not lost, f"rows {lost[:8]} lost a needle"
    return res, rows, n_needles


def test_workload_tiny_fp32_512_all_rows(gpu_lib):
    _, rows, nn = _workload_check(gpu_lib, "tiny_fp32_512")
    assert rows.size == 512 and nn > 0


def test_workload_mid_bf16_4k_all_rows(gpu_lib):
    _, rows, nn = _workload_check(gpu_lib, "mid_bf16_4k")
    assert rows.size == 4096 and nn > 0


def test_workload_long_bf16_32k_sample(gpu_lib):
    _, rows, _ = _workload_check(gpu_lib, "long_bf16_32k")
    assert rows.size == 256


@pytest.mark.parametrize("k", [512, 1024, 2048])
def test_workload_vlong_bf16_100k_sample(gpu_lib, k):
    """The budget sweep of the 100K layer; oracle_prefill runs the windowed
    gather here (13 key windows)."""
    _, rows, _ = _workload_check(gpu_lib, "vlong_bf16_100k", k=k)
    assert rows.size == 128


# ----------------------------------------------------------------- indexer
def _indexer_run(amtk, qi, ki, k, key_block):
    import torch
    idx, cnt, mass = amtk.indexer_topk(torch.from_numpy(qi).to(torch.bfloat16).cuda(),
                                       torch.from_numpy(ki).to(torch.bfloat16).cuda(), k,
                                       key_block)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy(), mass.cpu().numpy()


# n = 1, 31 and 97 put fewer key tiles than waves in the split LSE pass (one
# head: four waves per 32-row tile) and leave ragged last tiles
@pytest.mark.parametrize("n,k,kb", [(1000, 4, 64), (300, 16, 1), (64, 2, 64), (65, 1, 64),
                                    (1, 3, 1), (31, 5, 1), (97, 7, 1), (97, 1, 64)])
def test_indexer_small(gpu_lib, n, k, kb):
    rng = np.random.default_rng(n + k)
    from synth import round_bf16
    qi = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    ki = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    idx, cnt, mass = _indexer_run(gpu_lib, qi, ki, k, kb)
    ix = IndexerOracle(qi, ki)
    for i in range(n):
        r = ix.row(i, k, kb)
        from tests.support_rules import check_row
        ok, msg, _ = check_row(idx[i], cnt[i], r["score"], r["kth"], k, BAND)
        assert ok, f"row {i}: {msg}"
        sel = idx[i][: cnt[i]]
        assert np.all(np.abs(mass[i][: cnt[i]] - r["score"][sel]) <= 1e-7 + 2e-4 * r["score"][sel])


def test_indexer_zero_queries_tie_by_block_size(gpu_lib):
    n = 500
    qi = np.zeros((n, 64), dtype=np.float32)
    ki = np.random.default_rng(1).standard_normal((n, 64)).astype(np.float32)
    from synth import round_bf16
    idx, cnt, _ = _indexer_run(gpu_lib, qi, round_bf16(ki), 2, 64)
    for i in range(n):
        nb = i // 64 + 1
        if nb <= 2:
            assert idx[i][: cnt[i]].tolist() == list(range(nb))
        elif (i + 1) % 64 == 0:
            assert idx[i][:2].tolist() == [0, 1]          # all blocks full: smallest ids
        else:
            assert idx[i][:2].tolist() == [0, 1]          # full blocks outweigh the partial one


def test_workload_indexer_bf16_32k_sample(gpu_lib):
    """The indexer workload on its whole seeded row sample (256 rows): the
    indexer's top-16 key blocks by the near-tie rule, their block masses,
    and the gather on them (one pass and windowed) against the oracle."""
    import torch
    amtk = gpu_lib
    w = WORKLOADS["indexer_bf16_32k"]
    x = _generated("indexer_bf16_32k")
    rows = sample_rows(w)
    assert rows.size == 256
    idx, cnt, mass = _indexer_run(amtk, x["q_idx"], x["k_idx"], w.k, w.key_block)
    ix = IndexerOracle(x["q_idx"], x["k_idx"])
    for i in rows:
        r = ix.row(int(i), w.k, w.key_block)
        ok, msg, _ = check_row(idx[i], cnt[i], r["score"], r["kth"], w.k, BAND)
        assert ok, f"row {i}: {msg}"
        sel = idx[i][: cnt[i]]
        want = r["score"][sel]
        assert np.all(np.abs(mass[i][: cnt[i]] - want) <= 1e-7 + 2e-4 * want), f"mass row {i}"
    d = upload(x, "bf16")
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    out, lse_s = amtk.sparse_attn(d["q"], d["k"], d["v"], ti, tc, 64, want_lse=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    check_outputs_on_gpu_support(out.cpu().numpy(), lse_s.cpu().numpy(), layer, rows, idx, cnt,
                                 64, "bf16")
    # the windowed gather (four 8192-token windows) on the same supports
    out_w, _ = amtk.sparse_attn_windowed(d["q"], d["k"], d["v"], ti, tc, 64)
    torch.cuda.synchronize()
    assert float((out_w - out).abs().max()) <= 1.5e-4
    check_outputs_on_gpu_support(out_w.cpu().numpy(), None, layer, rows, idx, cnt, 64, "bf16")
