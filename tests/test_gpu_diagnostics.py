"""GPU parity of the support diagnostics (captured mass, support overlap).

captured_mass is compared with the oracle's head-averaged mass on the GPU's
own support (|diff| <= 1e-6 + 2e-4 * captured: the support and dense LSEs
carry about 1e-4 absolute error each, see the sparse-attention bar);
support_overlap, integer work, must equal the host intersection of the same
arrays exactly. Cases: small shapes on every row, a budget sweep, the
indexer workload (indexer support against the oracle's block support), and
selection-block supports (the realization side).
"""
import numpy as np
import pytest

from oracle import OracleLayer, tokens_of_blocks
from synth import WORKLOADS, generate, random_inputs, sample_rows
from tests.gpu_helpers import upload

pytestmark = pytest.mark.gpu


def _tol(c):
    return 1e-6 + 2e-4 * abs(c)


def _host_overlap(ia, ca, ib, cb):
    out = np.zeros(ia.shape[0], dtype=np.int64)
    for i in range(ia.shape[0]):
        a = ia[i, : ca[i]]
        b = ib[i, : cb[i]]
        out[i] = np.intersect1d(a[a >= 0], b[b >= 0]).size
    return out


def _captured_on_gpu(amtk, d, idx, cnt, lse_dense, key_block=1):
    _, lse_s = amtk.sparse_attn(d["q"], d["k"], d["v"], idx, cnt, key_block, want_lse=True)
    return amtk.captured_mass(lse_dense, lse_s)


@pytest.mark.parametrize("n,hq,hkv,d,dtype,k1,k2", [
    (150, 32, 8, 128, "bf16", 24, 9),
    (97, 8, 2, 64, "f32", 16, 5),
])
def test_captured_mass_and_overlap_all_rows(gpu_lib, n, hq, hkv, d, dtype, k1, k2):
    import torch
    amtk = gpu_lib
    x = random_inputs(n, hq, hkv, d, dtype, seed=n + k1, sink=True)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    dd = upload(x, dtype)
    idx1, cnt1, _, lse = amtk.topk_support(dd["q"], dd["k"], k1)
    idx2, cnt2, _, _ = amtk.topk_support(dd["q"], dd["k"], k2)
    cap = _captured_on_gpu(amtk, dd, idx1, cnt1, lse).cpu().numpy()
    ov = amtk.support_overlap(idx1, cnt1, idx2, cnt2).cpu().numpy()
    torch.cuda.synchronize()
    i1, c1 = idx1.cpu().numpy(), cnt1.cpu().numpy()
    i2, c2 = idx2.cpu().numpy(), cnt2.cpu().numpy()
    assert np.array_equal(ov, _host_overlap(i1, c1, i2, c2))
    for i in range(n):
        want = layer.captured(i, i1[i, : c1[i]])
        assert abs(cap[i] - want) <= _tol(want), f"row {i}: {cap[i]} vs {want}"
        if c1[i] == i + 1:
            assert abs(cap[i] - 1.0) <= _tol(1.0)


def test_overlap_unsorted_counts_and_negative_ids(gpu_lib):
    """Clamped counts, -1 entries inside the count, empty rows; supports of
    different widths. Support a ascends (the contract); b may come in any
    order."""
    import torch
    amtk = gpu_lib
    n, ma, mb = 200, 40, 70
    rng = np.random.default_rng(3)
    ia = np.full((n, ma), -1, dtype=np.int32)
    ib = np.full((n, mb), -1, dtype=np.int32)
    ca = rng.integers(0, ma + 5, n).astype(np.int32)
    cb = rng.integers(0, mb + 5, n).astype(np.int32)
    for i in range(n):
        a = np.sort(rng.choice(300, size=min(ca[i], ma), replace=False))
        ia[i, : a.size] = a
        b = rng.choice(300, size=min(cb[i], mb), replace=False)
        if b.size > 3:
            b[1] = -1
        ib[i, : b.size] = b
    ca[5] = 0
    cb[6] = 0
    t = lambda a: torch.from_numpy(a).cuda()
    ov = amtk.support_overlap(t(ia), t(ca), t(ib), t(cb)).cpu().numpy()
    want = _host_overlap(ia, np.minimum(ca, ma), ib, np.minimum(cb, mb))
    assert np.array_equal(ov, want)


def test_captured_mass_budget_sweep_mid_bf16_4k(gpu_lib):
    """Captured mass against the budget (the oracle-feasibility side of the
    diagnostics) on seeded rows of the 4K workload: per row against the
    oracle on the GPU's support, and the sample mean non-decreasing in k."""
    amtk = gpu_lib
    w = WORKLOADS["mid_bf16_4k"]
    x = generate(w)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    rows = sample_rows(w)[::16]
    dd = upload(x, "bf16")
    prev = 0.0
    for k in (16, 82, 512):
        idx, cnt, _, lse = amtk.topk_support(dd["q"], dd["k"], k)
        cap = _captured_on_gpu(amtk, dd, idx, cnt, lse).cpu().numpy()
        ii, cc = idx.cpu().numpy(), cnt.cpu().numpy()
        for i in rows:
            want = layer.captured(int(i), ii[i, : cc[i]])
            assert abs(cap[i] - want) <= _tol(want), f"k={k} row {i}"
        assert cap.mean() >= prev - 1e-6
        prev = float(cap.mean())


def test_indexer_against_oracle_blocks_indexer_bf16_32k(gpu_lib):
    """The indexer gap's layer-level analogue on the indexer workload: the
    overlap of the indexer's top-16 blocks with the oracle's top-16 blocks
    (every row, exact), and the oracle mass the indexer's support captures
    (seeded rows, against the oracle)."""
    import torch
    amtk = gpu_lib
    w = WORKLOADS["indexer_bf16_32k"]
    x = generate(w)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    dd = upload(x, "bf16")
    qi = torch.from_numpy(x["q_idx"]).to(torch.bfloat16).cuda()
    ki = torch.from_numpy(x["k_idx"]).to(torch.bfloat16).cuda()
    ind, cind, _ = amtk.indexer_topk(qi, ki, w.k, w.key_block)
    orc, corc, _, lse = amtk.topk_support(dd["q"], dd["k"], w.k, w.key_block)
    cap = _captured_on_gpu(amtk, dd, ind, cind, lse, w.key_block).cpu().numpy()
    ov = amtk.support_overlap(orc, corc, ind, cind).cpu().numpy()
    a, ca = orc.cpu().numpy(), corc.cpu().numpy()
    b, cb = ind.cpu().numpy(), cind.cpu().numpy()
    assert np.array_equal(ov, _host_overlap(a, ca, b, cb))
    for i in sample_rows(w)[::8]:
        toks = tokens_of_blocks(b[i, : cb[i]], w.key_block, int(i))
        want = layer.captured(int(i), toks)
        assert abs(cap[i] - want) <= _tol(want), f"row {i}: {cap[i]} vs {want}"


def test_captured_mass_of_selection_blocks_mid_bf16_4k(gpu_lib):
    """The realization side: the mass each row keeps on its selection block's
    shared support (keys up to the row), from sparse_attn_blocks' LSE."""
    amtk = gpu_lib
    w = WORKLOADS["mid_bf16_4k"]
    x = generate(w)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    dd = upload(x, "bf16")
    idx, cnt, _, lse = amtk.topk_support(dd["q"], dd["k"], w.k, query_block=64)
    _, lse_s = amtk.sparse_attn_blocks(dd["q"], dd["k"], dd["v"], idx, cnt, 64, want_lse=True)
    cap = amtk.captured_mass(lse, lse_s).cpu().numpy()
    ii, cc = idx.cpu().numpy(), cnt.cpu().numpy()
    for i in list(range(0, 64, 5)) + [int(r) for r in sample_rows(w)[::32]]:
        sup = ii[i, : cc[i]]
        want = layer.captured(i, sup[sup <= i])
        assert abs(cap[i] - want) <= _tol(want), f"row {i}: {cap[i]} vs {want}"
