"""GPU parity of the KL-distillation loss kernel (kl_distill) against the oracle.

Bars, from the arithmetic: the teacher masses carry about 1e-6 relative
error (fp32 sums of exact bf16 products, v_exp_f32), the student logits are
exact bf16 products summed in fp32, and dS = Q - P enters the gradient
products split into two bf16 halves (2^-16 relative). Hence
  KL_i:     |diff| <= 1e-4 * max(1, KL_i)
  dq_idx:   |diff| <= 1e-4 * (tau/N) * sum_j (P_ij + Q_ij) |k_idx[j]|_max
  dk_idx:   |diff| <= 1e-4 * (tau/N) * sum_i (P_ij + Q_ij) |q_idx[i]|_max
(the sums are taken from the oracle), plus 1e-3 relative to the value.
Small shapes are compared in full; the 4K and 32K indexer layers on seeded
rows (KL, dq), on their last keys (dk: those need only the last rows), and
through properties that hold at any size: sum_i <q_i, dq_i> = sum_j <k_j,
dk_j>, sum_j dk_j = 0 (the loss ignores a shift of every k_idx row), and
the loss as the mean of the rows. The query-major pass forms dS = Q - P per
pair for KL and dq; the key gradient is built per KV group (each group's
share of the head sum), so dq and dk round dS differently and the
identities hold within bounds derived from the same per-pair bar.
"""
import math

import numpy as np
import pytest

from oracle import KLDistillOracle, OracleLayer
from synth import WORKLOADS, generate, random_inputs, round_bf16, sample_rows

pytestmark = pytest.mark.gpu


def _upload(x, qi, ki):
    import torch
    t = {key: torch.from_numpy(x[key]).to(torch.bfloat16).cuda() for key in ("q", "k")}
    t["qi"] = torch.from_numpy(qi).to(torch.bfloat16).cuda()
    t["ki"] = torch.from_numpy(ki).to(torch.bfloat16).cuda()
    return t


def _run(amtk, t):
    import torch
    kl, loss, dq, dk = amtk.kl_distill(t["q"], t["k"], t["qi"], t["ki"])
    torch.cuda.synchronize()
    return kl.cpu().numpy(), float(loss.cpu().numpy()[0]), dq.cpu().numpy(), dk.cpu().numpy()


def _idx_inputs(n, seed):
    rng = np.random.default_rng(seed)
    qi = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    ki = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    return qi, ki


def _check_rows(kd, rows, kl, dq, qi, ki):
    n = kd.n
    tau = kd.scale
    kmax = float(np.max(np.abs(ki)))
    for i in rows:
        r = kd.row(int(i))
        want_kl = r["kl"]
        assert abs(kl[i] - want_kl) <= 1e-4 * max(1.0, abs(want_kl)), f"row {i}: KL {kl[i]} vs {want_kl}"
        want = kd.dq(int(i))
        mass = float(np.sum(r["p"] + np.exp(r["log_q"])))
        tol = 1e-4 * tau / n * mass * kmax + 1e-3 * np.abs(want)
        err = np.abs(dq[i] - want)
        assert np.all(err <= tol), f"row {i}: dq err {err.max()} (tol {tol.min()})"


def _check_keys(kd, keys, dk, qi):
    n = kd.n
    tau = kd.scale
    want = kd.dk(keys)
    colmass = np.zeros(len(keys))
    for i in range(int(min(keys)), n):
        r = kd.row(i)
        pq = r["p"] + np.exp(r["log_q"])
        for a, j in enumerate(keys):
            if j <= i:
                colmass[a] += pq[j]
    qmax = float(np.max(np.abs(qi)))
    for a, j in enumerate(keys):
        tol = 1e-4 * tau / n * colmass[a] * qmax + 1e-3 * np.abs(want[a])
        err = np.abs(dk[j] - want[a])
        assert np.all(err <= tol), f"key {j}: dk err {err.max()} (tol {tol.min()})"


def _check_properties(kl, loss, dq, dk, qi, ki, tau):
    """Identities of the exact gradients. dq and dk are computed from two
    roundings of dS = Q - P (the query-major pass forms Q - P per pair; the
    key gradient adds the KV groups' shares of P separately), each within
    eps (P_ij + Q_ij) of the exact dS with eps = 1e-4, the same bar as the
    element-wise checks. Summed over all pairs, with sum_j (P_ij + Q_ij) = 2
    per row:
      |sum_i <q_i, dq_i> - sum_j <k_j, dk_j>| <= 4 eps tau max|q_i| max|k_j|,
      |sum_j dk_j[d]| <= 2 eps (tau/N) sum_i |q_i[d]|."""
    n = qi.shape[0]
    eps = 1e-4
    q64, k64 = qi.astype(np.float64), ki.astype(np.float64)
    assert abs(loss - float(np.mean(kl.astype(np.float64)))) <= 1e-6 * max(1.0, abs(loss))
    lhs = float(np.sum(q64 * dq))
    rhs = float(np.sum(k64 * dk))
    qn = float(np.max(np.linalg.norm(q64, axis=1)))
    kn = float(np.max(np.linalg.norm(k64, axis=1)))
    assert abs(lhs - rhs) <= 4 * eps * tau * qn * kn, (lhs, rhs)
    tot = dk.astype(np.float64).sum(axis=0)
    bound = 2 * eps * tau / n * np.abs(q64).sum(axis=0)
    assert np.all(np.abs(tot) <= bound), (tot, bound)


@pytest.mark.parametrize("n", [1, 32, 100, 161])
def test_kl_distill_small_shapes_every_row_and_key(gpu_lib, n):
    x = random_inputs(n, 32, 8, 128, "bf16", seed=300 + n, sink=True)
    qi, ki = _idx_inputs(n, 400 + n)
    kl, loss, dq, dk = _run(gpu_lib, _upload(x, qi, ki))
    kd = KLDistillOracle(OracleLayer(x["q"], x["k"], x["v"]), qi, ki)
    _check_rows(kd, range(n), kl, dq, qi, ki)
    _check_keys(kd, list(range(n)), dk, qi)
    full = kd.full()
    assert abs(loss - full["loss"]) <= 1e-4 * max(1.0, abs(full["loss"]))
    _check_properties(kl, loss, dq, dk, qi, ki, kd.scale)


@pytest.mark.parametrize("n,hq,hkv", [
    (100, 16, 4),   # 4 KV heads: 4 of the tile kernel's 8 waves score the teacher
    (161, 8, 2),
    (70, 4, 1),     # one KV head (MQA-style groups of 4)
    (33, 8, 2),     # a ragged second tile
    (600, 16, 4),   # three 256-key blocks of the key-gradient kernel, the last partial
])
def test_kl_distill_other_head_layouts_every_row_and_key(gpu_lib, n, hq, hkv):
    """4 query heads per KV head with 1, 2 or 4 KV heads: every row and key
    against the oracle, the loss, and the gradient identities."""
    import torch
    x = random_inputs(n, hq, hkv, 128, "bf16", seed=500 + n + hkv, sink=True)
    qi, ki = _idx_inputs(n, 600 + n + hkv)
    t = _upload(x, qi, ki)
    kl, loss, dq, dk = _run(gpu_lib, t)
    kd = KLDistillOracle(OracleLayer(x["q"], x["k"], x["v"]), qi, ki)
    _check_rows(kd, range(n), kl, dq, qi, ki)
    _check_keys(kd, list(range(n)), dk, qi)
    full = kd.full()
    assert abs(loss - full["loss"]) <= 1e-4 * max(1.0, abs(full["loss"]))
    _check_properties(kl, loss, dq, dk, qi, ki, kd.scale)
    again = gpu_lib.kl_distill(t["q"], t["k"], t["qi"], t["ki"])   # deterministic
    torch.cuda.synchronize()
    for a, b in zip(again, (kl, np.array([loss], dtype=np.float32), dq, dk)):
        assert np.array_equal(a.cpu().numpy(), b)


def test_kl_distill_student_equals_teacher_gives_zero(gpu_lib):
    """Four identical query heads per KV head and identical KV heads make the
    head-averaged mass one head's softmax; with q_idx, k_idx the first 64
    dims of that head and zeros elsewhere, and idx_scale = 1/sqrt(128), the
    student equals the teacher: KL and both gradients vanish (to rounding)."""
    import torch
    n = 96
    rng = np.random.default_rng(5)
    q1 = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    k1 = round_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    q = np.zeros((n, 32, 128), np.float32)
    k = np.zeros((n, 8, 128), np.float32)
    q[:, :, :64] = q1[:, None, :]
    k[:, :, :64] = k1[:, None, :]
    t = {"q": torch.from_numpy(q).to(torch.bfloat16).cuda(),
         "k": torch.from_numpy(k).to(torch.bfloat16).cuda(),
         "qi": torch.from_numpy(q1).to(torch.bfloat16).cuda(),
         "ki": torch.from_numpy(k1).to(torch.bfloat16).cuda()}
    kl, loss, dq, dk = gpu_lib.kl_distill(t["q"], t["k"], t["qi"], t["ki"],
                                          idx_scale=1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    assert float(kl.abs().max()) <= 1e-5
    assert float(dq.abs().max()) <= 1e-7 and float(dk.abs().max()) <= 1e-7


def test_kl_distill_repeatable_bitwise(gpu_lib):
    n = 200
    x = random_inputs(n, 32, 8, 128, "bf16", seed=77, sink=True)
    qi, ki = _idx_inputs(n, 78)
    t = _upload(x, qi, ki)
    a = _run(gpu_lib, t)
    b = _run(gpu_lib, t)
    for u, v in zip(a, b):
        assert np.array_equal(np.asarray(u), np.asarray(v))


@pytest.mark.parametrize("n", [4096, 32768])
def test_kl_distill_indexer_workload(gpu_lib, n):
    """The indexer workload's layer (main Q/K with the sink and needles, the
    correlated q_idx/k_idx) at 4K and at its full 32K."""
    w = WORKLOADS["indexer_bf16_32k"]
    x = generate(w, n=n)
    qi, ki = x["q_idx"], x["k_idx"]
    kl, loss, dq, dk = _run(gpu_lib, _upload(x, qi, ki))
    kd = KLDistillOracle(OracleLayer(x["q"], x["k"], x["v"]), qi, ki)
    rows = sample_rows(w, n=n)[:: (8 if n == 4096 else 32)]
    _check_rows(kd, rows, kl, dq, qi, ki)
    _check_keys(kd, list(range(n - 40, n, 3)), dk, qi)
    _check_properties(kl, loss, dq, dk, qi, ki, kd.scale)
