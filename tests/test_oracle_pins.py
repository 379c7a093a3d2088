"""Pins for the CPU oracle: things the pages and the mathematics fix on their own.

Each test would fail for a plausible slip in the oracle: a dropped or wrong
scale, a transposed operand, a wrong GQA routing, logits instead of
probabilities, a missing renormalisation, a wrong tie-break or sort direction.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleLayer, IndexerOracle
from synth import WORKLOADS, generate, random_inputs
from tests import brute_force as bf

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(expr):
    """Evaluate a golden-file entry: a fraction, or a small ln-expression."""
    expr = str(expr)
    if "ln" in expr:
        if "*" in expr:
            a, b = expr.split("*")
            return float(a) * math.log(float(b[2:]))
        return math.log(float(expr[2:]))
    return float(Fraction(expr))


# ----------------------------------------------------------------- golden rows
def _worked_layer():
    g = json.load(open(os.path.join(GOLDEN, "worked_rows.json")))
    k = np.array([[_num(x) for x in row] for row in g["k_rows"]])[:, None, :]
    qh = np.array(g["q_head_rows"], dtype=np.float64)
    q = np.broadcast_to(qh, (4, 2, 4)).copy()
    v = np.eye(4)[:, None, :]
    return g, OracleLayer(q, k, v)


def test_worked_rows_mass_lse_topk():
    g, layer = _worked_layer()
    assert layer.scale == 0.5
    for i_s, exp in g["rows"].items():
        i = int(i_s)
        for kk, top in exp["top"].items():
            r = layer.row(i, int(kk))
            np.testing.assert_allclose(r["lse"], [_num(x) for x in exp["lse"]], atol=1e-12)
            np.testing.assert_allclose(r["p"], [_num(x) for x in exp["mass"]], atol=1e-12)
            assert r["units"].tolist() == top


def test_worked_row3_outputs_and_blocks():
    g, layer = _worked_layer()
    exp = g["rows"]["3"]
    r = layer.row(3, 2, dense=True)
    np.testing.assert_allclose(r["out"], [[_num(x) for x in row] for row in exp["out_top2"]],
                               atol=1e-12)
    np.testing.assert_allclose(r["lse_s"], [_num(x) for x in exp["lse_top2"]], atol=1e-12)
    np.testing.assert_allclose(r["dense_out"], [[_num(x) for x in row] for row in exp["dense_out"]],
                               atol=1e-12)
    rb = layer.row(3, 1, key_block=2)
    np.testing.assert_allclose(rb["score"], [_num(x) for x in exp["block2_mass"]], atol=1e-12)
    assert rb["units"].tolist() == exp["block2_top1"]
    assert rb["support"].tolist() == [2, 3]


def _num_or_inf(expr):
    return -math.inf if str(expr) == "-inf" else _num(expr)


def test_worked_rows_kth_mass():
    """The selection boundary (k-th largest mass) of every worked row and budget,
    read off the hand-sorted masses; -inf where the row keeps all its units."""
    g, layer = _worked_layer()
    for i_s, exp in g["rows"].items():
        i = int(i_s)
        for kk, want in exp["kth"].items():
            r = layer.row(i, int(kk))
            want = _num_or_inf(want)
            if want == -math.inf:
                assert r["kth"] == -math.inf, (i, kk)
            else:
                assert r["kth"] == pytest.approx(want, abs=1e-12), (i, kk)
            assert oracle.kth_score(r["p"], int(kk)) == r["kth"]
    exp3 = g["rows"]["3"]
    for kk, want in exp3["block2_kth"].items():
        rb = layer.row(3, int(kk), key_block=2)
        want = _num_or_inf(want)
        if want == -math.inf:
            assert rb["kth"] == -math.inf
        else:
            assert rb["kth"] == pytest.approx(want, abs=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_kth_score_is_the_order_statistic(seed):
    """kth_score(x, k) is the value m with #(x > m) < k <= #(x >= m), the
    definition of the k-th largest element, on rows with repeated values."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    x = rng.integers(0, 6, size=n).astype(np.float64) / 7.0
    for kk in range(1, n + 3):
        m = oracle.kth_score(x, kk)
        if n <= kk:
            assert m == -math.inf
            continue
        assert m in set(x.tolist())
        assert int(np.sum(x > m)) < kk <= int(np.sum(x >= m))
        # the top-k set is exactly what lies above m plus the first equals
        top = oracle.top_units(x, kk)
        assert top.size == kk
        assert np.all(x[top] >= m)
        above = np.nonzero(x > m)[0]
        assert set(above.tolist()) <= set(top.tolist())
        eq_taken = sorted(set(top.tolist()) - set(above.tolist()))
        assert eq_taken == np.nonzero(x == m)[0][: kk - above.size].tolist()


# ---------------------------------------------------------- pages' sparsity
def test_sparsity_matches_pages_sweep_ends():
    g = json.load(open(os.path.join(GOLDEN, "sparsity_sweep.json")))
    for c in g["cases"]:
        got = 100.0 * oracle.causal_sparsity(c["n"], c["k"])
        assert abs(got - c["sparsity_pct"]) <= g["tolerance_pct"], (c, got)
        # the non-causal count 1 - k/N does not reproduce the printed figures
        assert abs(100.0 * (1 - c["k"] / c["n"]) - c["sparsity_pct"]) > 1.0


def test_sparsity_of_two_percent_budgets():
    # 2 % budgets at 4K and 32K sit at the top of the pages' range
    assert abs(100 * oracle.causal_sparsity(4096, 82) - 96.04) < 0.01
    assert abs(100 * oracle.causal_sparsity(32768, 655) - 96.04) < 0.01
    assert oracle.causal_sparsity(100, 100) == 0.0


# ------------------------------------------------------------- brute force
@pytest.mark.parametrize("shape", [(48, 8, 2, 16), (33, 4, 4, 8), (40, 6, 3, 32), (17, 2, 1, 64)])
@pytest.mark.parametrize("kk", [1, 5, 12])
def test_against_brute_force(shape, kk):
    n, hq, hkv, d = shape
    x = random_inputs(n, hq, hkv, d, "f32", seed=7 * n + kk, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    P, probs, logits = bf.full_mass(x["q"], x["k"], 1 / math.sqrt(d))
    supports = []
    for i in range(n):
        r = layer.row(i, kk, dense=True)
        np.testing.assert_allclose(r["p"], P[i, : i + 1], atol=1e-12, rtol=0)
        assert abs(P[i].sum() - 1) < 1e-12
        np.testing.assert_allclose(probs[:, i, : i + 1].sum(-1), 1.0, atol=1e-12)
        assert r["units"].tolist() == bf.full_topk(P[i], i, kk).tolist()
        supports.append(r["units"])
    o_bf = bf.full_sparse_out(logits, x["v"], supports)
    for i in range(n):
        np.testing.assert_allclose(layer.row(i, kk)["out"], o_bf[i], atol=1e-12)


@pytest.mark.parametrize("shape,b_sel", [((70, 8, 2, 16), 16), ((45, 4, 1, 8), 64),
                                         ((64, 6, 3, 32), 8)])
@pytest.mark.parametrize("kk", [1, 6, 20])
def test_query_blocks_against_brute_force(shape, b_sel, kk):
    """Selection-block-shared support: block scores, shared top-k and every
    row's output against the full-tensor formulation (masked softmax, mean
    over heads, column mean over the block's rows, stable argsort)."""
    n, hq, hkv, d = shape
    x = random_inputs(n, hq, hkv, d, "f32", seed=11 * n + kk + b_sel, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    P, probs, logits = bf.full_mass(x["q"], x["k"], 1 / math.sqrt(d))
    supports = []
    for t in range((n + b_sel - 1) // b_sel):
        r = layer.query_block(t, kk, b_sel)
        rows = list(r["rows"])
        assert rows == list(range(t * b_sel, min(n, (t + 1) * b_sel)))
        score, units = bf.full_block_topk(P, rows, kk)
        np.testing.assert_allclose(r["score"], score, atol=1e-12, rtol=0)
        assert abs(r["score"].sum() - 1) < 1e-12
        assert r["units"].tolist() == units.tolist()
        for i in rows:
            supports.append(units[units <= i])
    o_bf = bf.full_sparse_out(logits, x["v"], supports)
    for t in range((n + b_sel - 1) // b_sel):
        r = layer.query_block(t, kk, b_sel)
        for i in r["rows"]:
            np.testing.assert_allclose(r["out"][i], o_bf[i], atol=1e-12)


def test_query_block_of_one_row_is_per_query_and_full_budget_is_dense():
    n, hq, hkv, d = 40, 4, 2, 16
    x = random_inputs(n, hq, hkv, d, "f32", seed=5, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in range(n):
        a, b = layer.query_block(i, 7, 1), layer.row(i, 7)
        assert a["units"].tolist() == b["units"].tolist()
        np.testing.assert_array_equal(a["score"], b["p"])
        np.testing.assert_array_equal(a["out"][i], b["out"])
    # a budget covering the block's last row keeps every key: each row's
    # output is then its dense attention
    for t in range(3):
        r = layer.query_block(t, n, 16)
        assert r["units"].tolist() == list(range(r["rows"][-1] + 1))
        for i in r["rows"]:
            np.testing.assert_allclose(r["out"][i], layer.dense(i), atol=1e-12)


def test_query_block_equal_keys_closed_form():
    """All keys equal: row i spreads 1/(i+1) over keys 0..i, so the block
    score of key j is the mean over the block's rows i >= j of 1/(i+1)
    (keys after a row count 0 for it), and ties go to the smallest ids."""
    n, hq, hkv, d, b_sel = 50, 4, 2, 8, 16
    x = random_inputs(n, hq, hkv, d, "f32", seed=9)
    x["k"][:] = x["k"][0]
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for t in range(4):
        r = layer.query_block(t, 5, b_sel)
        rows = list(r["rows"])
        want = np.array([sum(1.0 / (i + 1) for i in rows if i >= j) / len(rows)
                         for j in range(rows[-1] + 1)])
        np.testing.assert_allclose(r["score"], want, rtol=1e-12, atol=0)
        assert r["units"].tolist() == list(range(5))


def test_dense_against_torch_sdpa():
    n, hq, hkv, d = 64, 8, 2, 32
    x = random_inputs(n, hq, hkv, d, "f32", seed=3, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    q = torch.from_numpy(x["q"]).double().permute(1, 0, 2)[None]
    k = torch.from_numpy(x["k"]).double().permute(1, 0, 2)[None].repeat_interleave(hq // hkv, 1)
    v = torch.from_numpy(x["v"]).double().permute(1, 0, 2)[None].repeat_interleave(hq // hkv, 1)
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)[0]
    ref = ref.permute(1, 0, 2).numpy()
    for i in range(n):
        np.testing.assert_allclose(layer.dense(i), ref[i], atol=1e-12)
        # k >= i+1 keeps every key, so the sparse output is the dense one
        r = layer.row(i, i + 1)
        assert r["units"].tolist() == list(range(i + 1))
        np.testing.assert_allclose(r["out"], ref[i], atol=1e-12)


# ------------------------------------------------------------- closed forms
def test_equal_keys_give_log_count():
    n, hq, hkv, d = 20, 4, 2, 16
    rng = np.random.default_rng(5)
    q = rng.standard_normal((n, hq, d))
    kap = rng.standard_normal((hkv, d))
    k = np.broadcast_to(kap, (n, hkv, d)).copy()
    v = rng.standard_normal((n, hkv, d))
    layer = OracleLayer(q, k, v)
    for i in range(n):
        r = layer.row(i, 3)
        for h in range(hq):
            dot = sum(q[i, h, c] * kap[h // 2, c] for c in range(d))
            assert abs(r["lse"][h] - (dot / math.sqrt(d) + math.log(i + 1))) < 1e-12
        # all keys tie: the smallest indices win
        assert r["units"].tolist() == list(range(min(3, i + 1)))
        np.testing.assert_allclose(r["p"], 1.0 / (i + 1), atol=1e-15)


def test_gqa_routing_contiguous_groups():
    # KV head 1 carries zero keys: only heads 2,3 (g = h // 2) see flat logits
    n, hq, hkv, d = 12, 4, 2, 8
    rng = np.random.default_rng(11)
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((n, hkv, d))
    k[:, 1, :] = 0.0
    v = rng.standard_normal((n, hkv, d))
    layer = OracleLayer(q, k, v)
    for i in range(1, n):
        lse = layer.row(i, 2)["lse"]
        np.testing.assert_allclose(lse[2:], math.log(i + 1), atol=1e-12)
        assert np.all(np.abs(lse[:2] - math.log(i + 1)) > 1e-6)
    assert [oracle.kv_head(h, 4, 2) for h in range(4)] == [0, 0, 1, 1]


def test_single_head_topk_is_topk_of_logits():
    n, d = 64, 16
    x = random_inputs(n, 1, 1, d, "f32", seed=9)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in range(n):
        raw = [float(np.dot(x["q"][i, 0].astype(np.float64), x["k"][j, 0].astype(np.float64)))
               for j in range(i + 1)]
        want = sorted(sorted(range(i + 1), key=lambda j: -raw[j])[:7])
        assert layer.row(i, 7)["units"].tolist() == want


def test_identical_heads_reduce_to_single_head():
    n, d = 40, 16
    x = random_inputs(n, 1, 1, d, "f32", seed=13)
    one = OracleLayer(x["q"], x["k"], x["v"])
    many = OracleLayer(np.repeat(x["q"], 4, axis=1), x["k"], x["v"])
    for i in range(n):
        a, b = one.row(i, 5), many.row(i, 5)
        assert a["units"].tolist() == b["units"].tolist()
        np.testing.assert_allclose(a["p"], b["p"], atol=1e-15)


def test_one_token_support_returns_its_value_row():
    x = random_inputs(30, 4, 2, 16, "f32", seed=21)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in [0, 5, 29]:
        for j in [0, i]:
            out, lse_s = layer.attention_on(i, [j])
            for h in range(4):
                np.testing.assert_array_equal(out[h], x["v"][j, h // 2].astype(np.float64))
                assert abs(lse_s[h] - layer.logits(i)[h, j]) < 1e-12


def test_scaling_values_scales_output_and_weights_sum_to_one():
    x = random_inputs(30, 4, 2, 16, "f32", seed=22)
    a = OracleLayer(x["q"], x["k"], x["v"])
    b = OracleLayer(x["q"], x["k"], 2.5 * x["v"].astype(np.float64))
    ones = OracleLayer(x["q"], x["k"], np.ones_like(x["v"]))
    for i in [3, 17, 29]:
        np.testing.assert_allclose(b.row(i, 4)["out"], 2.5 * a.row(i, 4)["out"], atol=1e-12)
        np.testing.assert_allclose(ones.row(i, 4)["out"], 1.0, atol=1e-12)


def test_nesting_causality_and_capture_bound():
    x = random_inputs(200, 8, 2, 32, "f32", seed=23, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in range(0, 200, 7):
        prev = set()
        for kk in (4, 16, 64):
            r = layer.row(i, kk)
            s = set(r["units"].tolist())
            assert prev <= s
            assert max(s) <= i and len(s) == min(kk, i + 1)
            assert r["captured"] >= min(kk, i + 1) / (i + 1) - 1e-12
            prev = s


# ------------------------------------------------------------ diagnostics
def test_captured_mass_of_full_support_is_one_and_of_top_k_is_brute_force_top_sum():
    """Captured mass pins: the whole causal prefix keeps all of the mass (P
    sums to 1); the oracle's top-k keeps the sum of the k largest entries of
    the brute-force mass row; it never decreases with k."""
    for (n, hq, hkv, d), seed in (((40, 4, 2, 8), 1), ((64, 6, 3, 16), 2)):
        x = random_inputs(n, hq, hkv, d, "f32", seed=seed + 50, sink=True)
        layer = OracleLayer(x["q"], x["k"], x["v"])
        P, _, _ = bf.full_mass(x["q"], x["k"], oracle.default_scale(d))
        for i in range(0, n, 3):
            assert abs(layer.captured(i, np.arange(i + 1)) - 1.0) <= 1e-12
            prev = 0.0
            for kk in (1, 3, 8, 20, n):
                r = layer.row(i, kk)
                top = np.sort(P[i, : i + 1])[::-1][: min(kk, i + 1)].sum()
                assert abs(layer.captured(i, r["units"]) - top) <= 1e-12
                assert abs(r["captured"] - top) <= 1e-12
                assert r["captured"] >= prev - 1e-15
                prev = r["captured"]


def test_captured_mass_from_support_lse_identity():
    """The identity the GPU's captured mass rests on:
    sum_{j in S} P(j) = (1/Hq) sum_h exp(LSE^S_h - LSE_h), checked between the
    oracle's support attention (LSE over S) and its mass row, on random
    supports, including an empty one (LSE^S = -inf contributes 0)."""
    x = random_inputs(90, 8, 2, 32, "f32", seed=57, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    rng = np.random.default_rng(5)
    for i in (0, 1, 17, 60, 89):
        s = layer.logits(i)
        lse = oracle.log_sum_exp(s)
        for m in (0, 1, 5, i + 1):
            sup = np.sort(rng.permutation(i + 1)[:m])
            want = layer.captured(i, sup)
            if sup.size == 0:
                assert want == 0.0
                continue
            _, lse_s = oracle.support_attention(s, layer.v_t, sup)
            got = float(np.mean(np.exp(lse_s - lse)))
            assert abs(got - want) <= 1e-12 * max(1.0, want)


def test_support_overlap_against_sets():
    rng = np.random.default_rng(8)
    assert oracle.support_overlap([1, 4, 9], [1, 4, 9]) == 3
    assert oracle.support_overlap([1, 4, 9], [0, 2, 10]) == 0
    assert oracle.support_overlap([-1, 3, -1], [-1, 3]) == 1
    assert oracle.support_overlap([], [1]) == 0
    for _ in range(50):
        a = rng.choice(100, size=int(rng.integers(0, 40)), replace=False)
        b = rng.choice(100, size=int(rng.integers(0, 40)), replace=False)
        want = len(set(a.tolist()) & set(b.tolist()))
        assert oracle.support_overlap(a, b) == want


# ------------------------------------------------------- KL distillation
def _kl_inputs(n, hq, hkv, d, d_idx, seed):
    x = random_inputs(n, hq, hkv, d, "f32", seed=seed, sink=True)
    rng = np.random.default_rng(seed + 1)
    qi = rng.standard_normal((n, d_idx)).astype(np.float32)
    ki = rng.standard_normal((n, d_idx)).astype(np.float32)
    return x, qi, ki


@pytest.mark.parametrize("shape", [(30, 4, 2, 8, 6), (45, 6, 3, 16, 8)])
def test_kl_distill_against_autograd_brute_force(shape):
    """Per-row KL, loss and both gradients against a second formulation: the
    brute-force teacher mass tensor, the student's masked log_softmax over a
    full [N, N] score matrix and torch fp64 autograd for the gradients."""
    n, hq, hkv, d, d_idx = shape
    x, qi, ki = _kl_inputs(n, hq, hkv, d, d_idx, seed=n)
    P, _, _ = bf.full_mass(x["q"], x["k"], oracle.default_scale(d))
    tq = torch.tensor(qi, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(ki, dtype=torch.float64, requires_grad=True)
    T = (tq @ tk.T) / math.sqrt(d_idx)
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool))
    logq = torch.log_softmax(T.masked_fill(~mask, float("-inf")), dim=-1)
    Pt = torch.tensor(P)
    pos = Pt > 0
    terms = torch.where(pos, Pt * (torch.log(torch.where(pos, Pt, torch.ones_like(Pt)))
                                   - torch.where(mask, logq, torch.zeros_like(logq))),
                        torch.zeros_like(Pt))
    kl = terms.sum(dim=1)
    loss = kl.mean()
    gq, gk = torch.autograd.grad(loss, (tq, tk))
    kd = oracle.KLDistillOracle(OracleLayer(x["q"], x["k"], x["v"]), qi, ki).full()
    np.testing.assert_allclose(kd["kl"], kl.detach().numpy(), rtol=1e-10, atol=1e-12)
    assert abs(kd["loss"] - float(loss.detach())) <= 1e-12
    np.testing.assert_allclose(kd["dq"], gq.numpy(), rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(kd["dk"], gk.numpy(), rtol=1e-9, atol=1e-13)


def test_kl_distill_is_zero_when_the_student_is_the_teacher():
    """One query head, one KV head, d_idx = d and the same temperature: the
    student's distribution is the teacher's, so every KL and gradient is 0."""
    n, d = 40, 16
    x = random_inputs(n, 1, 1, d, "f32", seed=61, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    kd = oracle.KLDistillOracle(layer, x["q"][:, 0, :], x["k"][:, 0, :]).full()
    assert np.max(np.abs(kd["kl"])) <= 1e-13
    assert np.max(np.abs(kd["dq"])) <= 1e-15 and np.max(np.abs(kd["dk"])) <= 1e-15


def test_kl_distill_invariances():
    """KL >= 0; a vector u added to every k_idx row shifts each student row by
    a constant, so the loss is unchanged and the key gradients sum to 0;
    sum_i <q_i, dq_i> = sum_j <k_j, dk_j> (both are sum_ij dL/dt_ij t_ij)."""
    n, d_idx = 50, 8
    x, qi, ki = _kl_inputs(n, 8, 2, 16, d_idx, seed=67)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    a = oracle.KLDistillOracle(layer, qi, ki).full()
    u = np.random.default_rng(3).standard_normal(d_idx)
    b = oracle.KLDistillOracle(layer, qi, ki + u).full()
    assert np.all(a["kl"] >= -1e-15)
    np.testing.assert_allclose(a["kl"], b["kl"], rtol=1e-10, atol=1e-12)
    assert np.max(np.abs(a["dk"].sum(axis=0))) <= 1e-12 * max(1.0, np.abs(a["dk"]).max() * n)
    lhs = float(np.sum(qi.astype(np.float64) * a["dq"]))
    rhs = float(np.sum(ki.astype(np.float64) * a["dk"]))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_kl_distill_row_and_key_subsets_match_the_full_pass():
    n = 36
    x, qi, ki = _kl_inputs(n, 4, 2, 8, 6, seed=71)
    kd = oracle.KLDistillOracle(OracleLayer(x["q"], x["k"], x["v"]), qi, ki)
    full = kd.full()
    for i in (0, 7, 35):
        assert abs(kd.row(i)["kl"] - full["kl"][i]) <= 1e-14
        np.testing.assert_allclose(kd.dq(i), full["dq"][i], rtol=1e-12, atol=1e-16)
    keys = [3, 20, 35]
    np.testing.assert_allclose(kd.dk(keys), full["dk"][keys], rtol=1e-12, atol=1e-16)


# ------------------------------------------- indexer, selection-block shared
@pytest.mark.parametrize("n,kb,b_sel,kk", [(150, 16, 32, 3), (200, 1, 64, 9), (97, 8, 64, 5)])
def test_indexer_query_blocks_against_brute_force(n, kb, b_sel, kk):
    """The indexer's block-shared support against a full-tensor formulation:
    masked [N, N] indexer softmax, column mean over the block's rows, sums
    over aligned key blocks, one stable argsort; supports clipped to j <= i."""
    from scipy.special import softmax
    rng = np.random.default_rng(n + kb)
    qi = rng.standard_normal((n, 12)).astype(np.float32)
    ki = rng.standard_normal((n, 12)).astype(np.float32)
    ix = IndexerOracle(qi, ki)
    T = (qi.astype(np.float64) @ ki.astype(np.float64).T) / math.sqrt(12)
    T = np.where(np.tril(np.ones((n, n), dtype=bool)), T, -np.inf)
    P = softmax(T, axis=1)
    for t in range((n + b_sel - 1) // b_sel):
        r = ix.query_block(t, kk, kb, b_sel)
        rows = list(range(t * b_sel, min(n, (t + 1) * b_sel)))
        assert list(r["rows"]) == rows
        last = rows[-1]
        col = P[rows, : last + 1].mean(axis=0)
        nb = (last + 1 + kb - 1) // kb
        score = np.array([col[b * kb:(b + 1) * kb].sum() for b in range(nb)])
        np.testing.assert_allclose(r["score"], score, atol=1e-12, rtol=0)
        order = np.argsort(-score, kind="stable")
        units = np.sort(order[: min(kk, nb)])
        assert r["units"].tolist() == units.tolist()
        for i in rows:
            toks = sorted(j for b in units for j in range(b * kb, min((b + 1) * kb, i + 1)))
            assert r["support"][i].tolist() == toks


def test_indexer_query_block_of_one_row_is_the_per_row_indexer():
    rng = np.random.default_rng(4)
    qi = rng.standard_normal((70, 8))
    ki = rng.standard_normal((70, 8))
    ix = IndexerOracle(qi, ki)
    for i in (0, 5, 63, 64, 69):
        a = ix.query_block(i, 3, 16, 1)
        b = ix.row(i, 3, 16)
        assert a["units"].tolist() == b["units"].tolist()
        np.testing.assert_allclose(a["score"], b["score"], atol=1e-14, rtol=0)
        assert a["support"][i].tolist() == b["support"].tolist()


def test_needles_are_selected_on_tiny_workload():
    w = WORKLOADS["tiny_fp32_512"]
    x = generate(w)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    owners = x["owner"]
    hits = 0
    for j in np.nonzero(owners >= 0)[0]:
        i = int(owners[j])
        assert j in set(layer.row(i, w.k)["units"].tolist()), (i, j)
        hits += 1
    assert hits > 300


# -------------------------------------------------------------- key blocks
def test_block_size_one_is_token_support():
    x = random_inputs(50, 4, 2, 16, "f32", seed=31)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in range(0, 50, 3):
        a, b = layer.row(i, 6), layer.row(i, 6, key_block=1)
        assert a["units"].tolist() == b["units"].tolist()


def test_block_masses_sum_to_one_and_clip_causally():
    x = random_inputs(100, 4, 2, 16, "f32", seed=32)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in [0, 9, 63, 64, 70, 99]:
        r = layer.row(i, 2, key_block=8)
        assert abs(r["score"].sum() - 1) < 1e-12
        assert r["score"].shape[0] == i // 8 + 1
        assert r["support"].max() <= i
        manual = [sum(r["p"][j] for j in range(b * 8, min(b * 8 + 8, i + 1)))
                  for b in range(i // 8 + 1)]
        np.testing.assert_allclose(r["score"], manual, atol=1e-15)


def test_indexer_zero_query_ties_by_block_size():
    n, di, blk = 300, 64, 64
    rng = np.random.default_rng(41)
    qi = np.zeros((n, di))
    ki = rng.standard_normal((n, di))
    ix = IndexerOracle(qi, ki)
    for i in [0, 63, 64, 200, 299]:
        r = ix.row(i, 2, blk)
        sizes = np.array([min(blk, i + 1 - b * blk) for b in range(i // blk + 1)])
        np.testing.assert_allclose(r["score"], sizes / (i + 1), atol=1e-15)
        full = np.nonzero(sizes == blk)[0]
        if full.size >= 2 and sizes.size > 2:
            assert r["units"].tolist() == [0, 1]


def test_indexer_equals_single_head_oracle():
    n, di = 150, 64
    x = random_inputs(n, 1, 1, di, "bf16", seed=43)
    ix = IndexerOracle(x["q"][:, 0], x["k"][:, 0])
    layer = OracleLayer(x["q"], x["k"], x["v"])
    for i in range(0, n, 11):
        a, b = ix.row(i, 2, 16), layer.row(i, 2, key_block=16)
        assert a["units"].tolist() == b["units"].tolist()
        np.testing.assert_allclose(a["score"], b["score"], atol=1e-14)
