"""Helpers shared by the GPU parity tests: upload inputs, run the HIP path,
compare with the oracle row by row."""
import numpy as np

from tests.support_rules import check_row

TOL_OUT = {"bf16": 2e-3, "f32": 1e-5}     # outputs on identical supports (max abs)
TOL_LSE = {"bf16": 1e-4, "f32": 1e-5}     # per-head log-sum-exp, dense or on a support (max abs)
BAND = 1e-6                               # near-tie band around the k-th mass


def to_dev(arr, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def upload(x, dtype):
    return {k: to_dev(x[k], dtype) for k in ("q", "k", "v") if k in x}


def check_support_rows(res_units, res_count, oracle, rows, k, key_block=1, band=BAND,
                       scores=None):
    """Near-tie check of GPU supports against the oracle on the given rows.

    Returns (n_rows, total in-band entries). Raises AssertionError on a failure.
    """
    in_band = 0
    for i in rows:
        if scores is not None:
            sc, kth = scores(i)
        else:
            r = oracle.row(int(i), k, key_block)
            sc, kth = r["score"], r["kth"]
        ok, msg, nb = check_row(res_units[i], res_count[i], sc, kth, k, band)
        assert ok, f"row {i}: {msg}"
        in_band += nb
    return len(rows), in_band


def check_outputs_on_gpu_support(out, lse_s, oracle, rows, units, counts, key_block, dtype):
    """GPU sparse output vs the oracle's attention on the GPU's own support."""
    from oracle import tokens_of_blocks
    worst = 0.0
    for i in rows:
        sel = units[i][: counts[i]]
        sup = sel if key_block == 1 else tokens_of_blocks(np.asarray(sel), key_block, int(i))
        o_ref, l_ref = oracle.attention_on(int(i), sup)
        err = float(np.max(np.abs(out[i].astype(np.float64) - o_ref)))
        worst = max(worst, err)
        assert err <= TOL_OUT[dtype], f"row {i}: max abs err {err}"
        if lse_s is not None:
            assert np.max(np.abs(lse_s[:, i] - l_ref)) <= TOL_LSE[dtype], f"row {i} lse_s"
    return worst
