#!/usr/bin/env python3
"""Oracle + sparse prefill throughput of one GQA layer on one MI355X.

A step is one pass of the whole hot path over the layer: per-head dense LSE
pass, head-averaged mass pass with the streaming top-k filter, exact select,
and the gather sparse attention on the selected supports (for the indexer
workload: indexer scoring + block top-k, then block sparse attention).
Inputs are seeded synthetic tensors already resident in HBM. Prints one JSON
line on stdout; everything else goes to stderr.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--k K]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = {
    "pass1_lse": ("sparse_long_context_causal_amd/csrc/passes.hip",
                  "sparse_long_context_causal_amd/csrc/pass1_direct.hip"),
    "pass2_filter": "sparse_long_context_causal_amd/csrc/passes.hip",
    "select": "sparse_long_context_causal_amd/csrc/select.hip",
    "sparse_attn": "sparse_long_context_causal_amd/csrc/sparse_attn.hip",
    "pass2_colsum": "sparse_long_context_causal_amd/csrc/passes.hip",
    "block_topk": "sparse_long_context_causal_amd/csrc/block_select.hip",
    "sparse_attn_blocks": "sparse_long_context_causal_amd/csrc/block_attn.hip",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(rel):
    h = hashlib.sha256()
    for r in ((rel,) if isinstance(rel, str) else rel):
        h.update(open(os.path.join(ROOT, r), "rb").read())
    h.update(open(os.path.join(ROOT, "sparse_long_context_causal_amd/csrc/device_common.h"),
                  "rb").read())
    return h.hexdigest()[:16]


def support_tokens(plan, key_block, query_block=1):
    """Tokens gathered by sparse_attn: sum over rows of the selected units' visible keys."""
    import torch
    cnt = plan.count.to(torch.int64)
    if key_block == 1 and query_block == 1:
        return int(cnt.sum().item())
    n, kk = plan.idx.shape
    rows = torch.arange(n, device=plan.idx.device, dtype=torch.int64)[:, None]
    b = plan.idx.to(torch.int64)
    valid = (torch.arange(kk, device=b.device)[None, :] < cnt[:, None]) & (b >= 0)
    if key_block == 1:      # a shared support: each row gathers its ids up to itself
        return int((valid & (b <= rows)).sum().item())
    toks = torch.clamp(rows + 1 - b * key_block, min=0, max=key_block)
    return int(torch.where(valid, toks, torch.zeros_like(toks)).sum().item())


def algorithmic_work(w, n, k, sup, gathered=None, units_read=None):
    """Per-call algorithmic flops / bytes of each stage (one call of a stage is one
    launch, except the windowed gather: its window-start kernel and one launch
    per key window; see the design notes).

    sup: keys attended over all rows; gathered: key rows the sparse kernel
    must fetch (= sup per row; once per selection block when shared);
    units_read: index entries it reads."""
    e = 2 if w.dtype == "bf16" else 4
    gathered = sup if gathered is None else gathered
    units_read = n * k if units_read is None else units_read
    pairs = n * (n + 1) // 2                    # causal query-key pairs
    qk_flops = 2 * w.d * w.hq * pairs           # one QK^T over the causal triangle
    attn_bytes = (gathered * w.hkv * w.d * 2 * e   # gathered K and V rows
                  + n * w.hq * w.d * e          # Q
                  + n * w.hq * w.d * 4          # O (fp32)
                  + units_read * 4 + n * 4)     # idx, count
    return qk_flops, attn_bytes


def traffic_for(kernel, workload):
    """Bytes from beyond L2 per call of a stage (all its launches) from the committed
    counter summary, if still current."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = t.get(workload, {}).get(kernel)
    if not ent or ent.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return ent.get("hbm_bytes_per_call")


CALIB_LIB = os.path.join(ROOT, "sparse_long_context_causal_amd", "libamtk_calib.so")


def l2_read_ceiling(regions_mb=(1, 2, 3), mode=0, grid=2048, pass_bytes=8e9, reps=5):
    """Measured L2 read bandwidth of this GPU (GB/s): every XCD re-reads a region
    of its own that fits its 4 MB L2 (calib/l2_read.hip), timed with HIP events
    on the launch stream; the best median over the region sizes. mode 0 streams
    contiguous 16-byte loads, mode 1 reads 256-byte rows at scattered positions
    (the gather's access shape) into registers, mode 2 the same rows into LDS
    by direct global->LDS loads, 16 KiB per 64-lane workgroup (the gather's
    own staging; grid 2048 runs 8 workgroups per CU, 2560 runs 10, which fill
    the LDS). Returns (GB/s, {region MB: GB/s})."""
    import ctypes
    import numpy as np
    import torch
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(CALIB_LIB)
    fn = lib.amtk_calib_l2_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sink = torch.empty(grid * 256 * 16, dtype=torch.uint8, device=dev)
    res = {}
    for mb in regions_mb:
        region = int(mb * (1 << 20))
        buf = torch.randint(0, 255, (8 * region,), dtype=torch.uint8, device=dev)
        if mode == 0:
            iters = max(1, int(pass_bytes / (8 * region)))
            nbytes = iters * 8 * region
        elif mode == 1:
            per_iter = grid * 16 * 64 * 256          # 64 rows per 16-lane group
            iters = max(1, int(pass_bytes / per_iter))
            nbytes = iters * per_iter
        else:
            per_iter = grid * 16384                  # 64-lane workgroups, 16 KiB rounds
            iters = max(1, int(pass_bytes / per_iter))
            nbytes = iters * per_iter
        times = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn(buf.data_ptr(), region, iters, grid, mode, sink.data_ptr(), stream.cuda_stream)
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"amtk_calib_l2_read returned {rc}")
            torch.cuda.synchronize(dev)
            if r:
                times.append(e0.elapsed_time(e1) * 1e-3)
        res[mb] = nbytes / float(np.median(times)) / 1e9
        del buf
    return max(res.values()), res


def pass_mix_ceiling(iters=3000, reps=3):
    """Measured compute ceilings of the passes' inner loop (calib/mix_ceiling.hip),
    in TFLOP/s of bf16 MFMA work, random operands, one 512-thread workgroup per CU
    (two waves per SIMD, the passes' occupancy): mode 0 the MFMA chains alone
    (the rate the chip sustains under its power limit), mode 1 the same chains
    with each head's fma/exp2/add per logit beside the next head's chain, in the
    pass kernels' order. Timed with HIP events on the launch stream, median of
    reps after one warm-up launch. Returns {"mfma_sustained": ..., "pass_mix": ...}."""
    import ctypes
    import numpy as np
    import torch
    if not os.path.exists(CALIB_LIB):
        raise RuntimeError(f"{CALIB_LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(CALIB_LIB)
    fn = lib.amtk_calib_mix
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    grid = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sink = torch.empty(grid * 512, dtype=torch.float32, device=dev)
    flops = float(grid) * 8 * iters * 64 * 32768   # 8 waves, 8 heads x 8 MFMAs per round
    out = {}
    for mode, name in ((0, "mfma_sustained"), (1, "pass_mix")):
        times = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = fn(mode, iters, grid, sink.data_ptr(), stream.cuda_stream)
            e1.record(stream)
            if rc != 0:
                raise RuntimeError(f"amtk_calib_mix returned {rc}")
            torch.cuda.synchronize(dev)
            if r:
                times.append(e0.elapsed_time(e1) * 1e-3)
        out[name] = flops / float(np.median(times)) / 1e12
    return out


def _host_cpu():
    """(cores this process may run on, CPU model name)."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cores, model


def cpu_baseline(w, x, k, key_block, budget_s=10.0, query_block=1):
    """The fp64 oracle on a seeded row sample of the same layer, extrapolated by row length."""
    cores, model = _host_cpu()
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=cores):      # BLAS threads = the cores we may use
        if query_block > 1:
            res = _cpu_baseline_blocks(w, x, k, query_block, budget_s)
        else:
            res = _cpu_baseline_rows(w, x, k, key_block, budget_s)
    res.update({"cores": cores, "cpu_model": model})
    return res


def _cpu_baseline_rows(w, x, k, key_block, budget_s):
    """The oracle's seeded row sample of the workload (every row at 512 and 4096
    tokens, 256 rows at 32K, 128 at 100K), walked in passes until at least
    budget_s of CPU work is done (at least one whole pass; a pass stops early
    only when a single pass exceeds 3 x budget_s)."""
    import numpy as np
    from oracle import OracleLayer, IndexerOracle
    from synth import sample_rows
    n = x["q"].shape[0]
    rows = np.random.default_rng(w.row_seed + 1).permutation(sample_rows(w, n=n))
    layer = OracleLayer(x["q"], x["k"], x["v"])
    ix = IndexerOracle(x["q_idx"], x["k_idx"]) if w.indexer_d else None
    t_rows, cost, done, passes = 0.0, 0.0, 0, 0
    while t_rows < budget_s:
        for i in rows:
            t0 = time.perf_counter()
            if ix is None:
                layer.row(int(i), k, key_block)
            else:
                r = ix.row(int(i), k, key_block)
                layer.attention_on(int(i), r["support"])
            t_rows += time.perf_counter() - t0
            cost += i + 1
            done += 1
            if t_rows > 3 * budget_s:
                break
        passes += 1
        if t_rows > 3 * budget_s:
            break
    full_s = t_rows * (n * (n + 1) / 2.0) / cost
    return {"value": n / full_s, "unit": "tokens/s", "kind": "oracle",
            "sample": (f"the {rows.size}-row seeded oracle sample of {w.name} "
                       f"({done} row evaluations in {passes} pass(es), {t_rows:.1f} s), full fp64 "
                       f"oracle per row, layer time extrapolated by row length "
                       f"(cost ~ i+1): {full_s:.1f} s"),
            "ms_per_row": 1000.0 * t_rows / max(done, 1)}


def _cpu_baseline_blocks(w, x, k, b_sel, budget_s):
    """The oracle's selection-block path on seeded blocks, extrapolated by the
    blocks' summed row lengths."""
    import numpy as np
    from oracle import OracleLayer, query_block_rows
    n = x["q"].shape[0]
    nblk = (n + b_sel - 1) // b_sel
    order = np.random.default_rng(w.row_seed + 2).permutation(nblk)
    layer = OracleLayer(x["q"], x["k"], x["v"])
    done, cost, t_all = 0, 0.0, 0.0
    for t in order:
        t0 = time.perf_counter()
        layer.query_block(int(t), k, b_sel)
        t_all += time.perf_counter() - t0
        done += 1
        cost += sum(i + 1 for i in query_block_rows(int(t), b_sel, n))
        if t_all > budget_s:
            break
    full_s = t_all * (n * (n + 1) / 2.0) / cost
    return {"value": n / full_s, "unit": "tokens/s", "kind": "oracle",
            "sample": (f"{done} seeded selection blocks of {b_sel} rows (of {nblk}) of {w.name}, "
                       f"full fp64 oracle per block ({t_all:.1f} s), layer time extrapolated by "
                       f"row length (cost ~ i+1): {full_s:.1f} s")}


def diagnostics(amtk, w, x, k):
    """Support diagnostics of one layer (the layer-level analogues of the
    oracle, realization and indexer gaps): the mean head-averaged dense mass
    the oracle's support keeps across budgets, with per-query and with shared
    selection-block supports, and, on the indexer workload, the indexer's
    recall of the oracle's blocks and the oracle mass its support keeps.
    Every per-row figure comes from the library's kernels; the means are
    taken here."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {key: torch.from_numpy(x[key]).to(tdt).to(dev) for key in ("q", "k", "v")}
    rep = {"diagnostics": w.name, "n": w.n, "k": k}

    def mean(a):
        return float(a.to(torch.float64).mean().item())

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if w.indexer_d:
        kb = w.key_block
        qi = torch.from_numpy(x["q_idx"]).to(torch.bfloat16).to(dev)
        ki = torch.from_numpy(x["k_idx"]).to(torch.bfloat16).to(dev)
        ind, cind, _ = amtk.indexer_topk(qi, ki, k, kb)
        orc, corc, _, lse = amtk.topk_support(t["q"], t["k"], k, kb)
        _, lse_i = amtk.sparse_attn(t["q"], t["k"], t["v"], ind, cind, kb, want_lse=True)
        _, lse_o = amtk.sparse_attn(t["q"], t["k"], t["v"], orc, corc, kb, want_lse=True)
        ev0.record()
        cap_i = amtk.captured_mass(lse, lse_i)
        ov = amtk.support_overlap(orc, corc, ind, cind)
        ev1.record()
        cap_o = amtk.captured_mass(lse, lse_o)
        torch.cuda.synchronize(dev)
        rep["indexer_block_recall"] = mean(ov.to(torch.float64) / corc.clamp(min=1))
        rep["indexer_captured_mass"] = mean(cap_i)
        rep["oracle_block_captured_mass"] = mean(cap_o)
        rep["ms_captured_and_overlap"] = ev0.elapsed_time(ev1)
        return rep
    sweep = {}
    for kk in sorted({max(1, k // 4), max(1, k // 2), k, 2 * k, 4 * k}):
        idx, cnt, _, lse = amtk.topk_support(t["q"], t["k"], kk)
        _, lse_s = amtk.sparse_attn(t["q"], t["k"], t["v"], idx, cnt, 1, want_lse=True)
        ev0.record()
        cap = amtk.captured_mass(lse, lse_s)
        ev1.record()
        torch.cuda.synchronize(dev)
        sweep[str(kk)] = {"captured_mass": mean(cap), "min": float(cap.min().item()),
                          "sparsity": 1.0 - float(cnt.to(torch.float64).sum().item())
                          / (w.n * (w.n + 1) / 2.0)}
        if kk == k:
            rep["ms_captured_mass"] = ev0.elapsed_time(ev1)
            per_query = cap
    rep["captured_mass_vs_k"] = sweep
    if w.dtype == "bf16" and w.hq == 32 and w.hkv == 8 and w.d == 128:
        idx, cnt, _, lse = amtk.topk_support(t["q"], t["k"], k, query_block=64)
        _, lse_s = amtk.sparse_attn_blocks(t["q"], t["k"], t["v"], idx, cnt, 64, want_lse=True)
        cap = amtk.captured_mass(lse, lse_s)
        rep["captured_mass_blocks_of_64"] = mean(cap)
        ov = amtk.support_overlap(*amtk.topk_support(t["q"], t["k"], k)[:2], idx, cnt)
        torch.cuda.synchronize(dev)
        rep["per_query_ids_kept_by_block_support"] = mean(
            ov.to(torch.float64) / torch.clamp(torch.arange(1, w.n + 1, device=dev), max=k))
        rep["captured_mass_per_query"] = mean(per_query)
    return rep


def kl_bench(amtk, w, x, steps, warmup):
    """Times kl_distill (teacher LSE pass, student LSE pass, the KL tile
    kernel with both gradients, the key-gradient reduction and the loss) on
    the indexer workload's layer, inputs resident on the device."""
    import torch
    dev = torch.device("cuda:0")
    t = {key: torch.from_numpy(x[key]).to(torch.bfloat16).to(dev)
         for key in ("q", "k", "q_idx", "k_idx")}
    ad = amtk.attn_desc(t["q"], t["k"])
    ws = amtk.workspace(amtk.kl_workspace_bytes(ad, w.indexer_d), dev)
    for _ in range(warmup):
        amtk.kl_distill(t["q"], t["k"], t["q_idx"], t["k_idx"], ws=ws)
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        kl, loss, dq, dk = amtk.kl_distill(t["q"], t["k"], t["q_idx"], t["k_idx"], ws=ws)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1) / steps
    n = w.n
    pairs = n * (n + 1) // 2
    # two teacher QK^T passes (LSE, then mass); student: LSE pass, t, dq, dk
    flops = 2 * (2 * w.d * w.hq * pairs) + 4 * (2 * w.indexer_d * pairs)
    return {"kl_distill": w.name, "n": n, "steps": steps, "ms_per_call": ms,
            "tokens_per_s": n / (ms * 1e-3), "loss": float(loss.item()),
            "algorithmic_tflops": flops / (ms * 1e-3) / 1e12,
            "workspace_bytes": ws.numel()}


def realisation(amtk, w, x, steps, warmup):
    """The indexer-driven sparse prefill three ways on the indexer workload:
    per query (indexer_topk + sparse_attn), selection blocks of 64 as two
    launches (indexer_topk + sparse_attn_blocks) and fused (indexer_prefill:
    one kernel per block scores, selects and attends, after the indexer's
    LSE pass); with the mean dense mass each support keeps (the layer-level
    side of the realization gap)."""
    import torch
    dev = torch.device("cuda:0")
    t = {key: torch.from_numpy(x[key]).to(torch.bfloat16).to(dev)
         for key in ("q", "k", "v", "q_idx", "k_idx")}
    k, kb = w.k, w.key_block

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize(dev)
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / steps

    def blocks_unfused():
        idx, cnt, _ = amtk.indexer_topk(t["q_idx"], t["k_idx"], k, kb, query_block=64)
        return amtk.sparse_attn_blocks(t["q"], t["k"], t["v"], idx, cnt, 64, key_block=kb)

    ms = {
        "per_query": timed(lambda: amtk.indexer_prefill(t["q"], t["k"], t["v"], t["q_idx"],
                                                        t["k_idx"], k, kb)),
        "blocks_of_64_unfused": timed(blocks_unfused),
        "blocks_of_64_fused": timed(lambda: amtk.indexer_prefill(t["q"], t["k"], t["v"], t["q_idx"],
                                                                 t["k_idx"], k, kb, query_block=64)),
    }
    # captured dense mass of each support
    _, _, _, lse = amtk.topk_support(t["q"], t["k"], k, kb)
    ip, cp, _ = amtk.indexer_topk(t["q_idx"], t["k_idx"], k, kb)
    _, lse_p = amtk.sparse_attn(t["q"], t["k"], t["v"], ip, cp, kb, want_lse=True)
    ib, cb, _ = amtk.indexer_topk(t["q_idx"], t["k_idx"], k, kb, query_block=64)
    _, lse_b = amtk.sparse_attn_blocks(t["q"], t["k"], t["v"], ib, cb, 64, key_block=kb,
                                       want_lse=True)
    cap_p = float(amtk.captured_mass(lse, lse_p).to(torch.float64).mean().item())
    cap_b = float(amtk.captured_mass(lse, lse_b).to(torch.float64).mean().item())
    return {"realisation": w.name, "n": w.n, "k": k, "key_block": kb, "steps": steps,
            "ms": ms, "tokens_per_s": {key: w.n / (v * 1e-3) for key, v in ms.items()},
            "captured_mass": {"per_query": cap_p, "blocks_of_64": cap_b}}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_bf16_32k")
    ap.add_argument("--k", type=int, default=None, help="budget (default: the workload's)")
    ap.add_argument("--query-block", type=int, default=1, choices=(1, 64),
                    help="1: a support per query; 64: one support per block of 64 queries")
    ap.add_argument("--diagnostics", action="store_true",
                    help="only print the support diagnostics of the workload and exit")
    ap.add_argument("--kl", action="store_true",
                    help="only time the KL-distillation loss and gradients (indexer workload)")
    ap.add_argument("--realisation", action="store_true",
                    help="only time the indexer path per query, in blocks of 64 and fused "
                         "(indexer workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-l2", action="store_true",
                    help="only measure the L2 read ceiling (streaming and 256-byte rows, "
                         "1-3 MB per XCD) and exit")
    ap.add_argument("--calibrate-mix", action="store_true",
                    help="only measure the passes' compute ceilings (MFMA chains alone, and "
                         "with the per-logit exp/sum work beside them) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run one plain device copy of MB megabytes (to scale HBM "
                         "traffic counters) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        nbytes = args.calibrate_copy * 1000 * 1000
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": nbytes,
                          "bytes_written": nbytes}), flush=True)
        return
    if args.calibrate_mix:
        print(json.dumps({"calibration": "pass inner loop from registers, random bf16 operands",
                          **{k + "_TFLOP/s": v for k, v in pass_mix_ceiling().items()}}),
              flush=True)
        return
    if args.calibrate_l2:
        best, per = l2_read_ceiling(mode=0)
        best_rows, per_rows = l2_read_ceiling(mode=1)
        best_lds, per_lds = l2_read_ceiling(mode=2, grid=2048)
        best_lds10, per_lds10 = l2_read_ceiling(mode=2, grid=2560)
        print(json.dumps({"calibration": "L2 read, every XCD re-reading its own region",
                          "stream_GBs": best, "stream_by_region_MB": per,
                          "rows_256B_GBs": best_rows, "rows_by_region_MB": per_rows,
                          "rows_256B_to_lds_8_per_CU_GBs": best_lds,
                          "rows_to_lds_8_per_CU_by_region_MB": per_lds,
                          "rows_256B_to_lds_10_per_CU_GBs": best_lds10,
                          "rows_to_lds_10_per_CU_by_region_MB": per_lds10}),
              flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU only (asked for --gpus {args.gpus}); the "
              "path shards by query rows across GPUs, which is not built here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import sparse_long_context_causal_amd as amtk
    from synth import WORKLOADS, generate

    amtk.load()
    w = WORKLOADS[args.workload]
    k = args.k or w.k
    log(f"[bench] generating {w.name} (n={w.n}, hq={w.hq}, hkv={w.hkv}, d={w.d}, k={k})")
    x = generate(w)
    if args.diagnostics:
        print(json.dumps(diagnostics(amtk, w, x, k)), flush=True)
        return
    if args.realisation:
        if not w.indexer_d:
            print("bench.py: --realisation needs an indexer workload (indexer_bf16_32k)",
                  file=sys.stderr)
            sys.exit(2)
        print(json.dumps(realisation(amtk, w, x, args.steps, args.warmup)), flush=True)
        return
    if args.kl:
        if not w.indexer_d:
            print("bench.py: --kl needs an indexer workload (indexer_bf16_32k)", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(kl_bench(amtk, w, x, args.steps, args.warmup)), flush=True)
        return
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {key: torch.from_numpy(x[key]).to(tdt).to(dev) for key in ("q", "k", "v")}
    extra = {}
    if w.indexer_d:
        extra = {key: torch.from_numpy(x[key]).to(torch.bfloat16).to(dev)
                 for key in ("q_idx", "k_idx")}
    qb = args.query_block
    if qb != 1 and (w.indexer_d or w.key_block != 1):
        print("bench.py: --query-block 64 applies to the oracle path with key_block 1",
              file=sys.stderr)
        sys.exit(2)
    plan = amtk.PrefillPlan(t["q"], t["k"], t["v"], k, w.key_block, query_block=qb, **extra)
    stream = torch.cuda.current_stream(dev)
    names = ["indexer_topk", "sparse_attn"] if w.indexer_d else \
        ["pass1_lse", "pass2_filter", "select", "sparse_attn"] if qb == 1 else \
        ["pass1_lse", "pass2_colsum", "block_topk", "sparse_attn"]
    pieces = [plan.indexer_call, plan.attn] if w.indexer_d else \
        [lambda: plan.stage(1), lambda: plan.stage(2), lambda: plan.stage(3), plan.attn]

    for _ in range(args.warmup):
        plan.run()
    torch.cuda.synchronize(dev)
    log(f"[bench] warmup done ({args.warmup} steps)")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(pieces) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for j, fn in enumerate(pieces):
            fn()
            ev[s][j + 1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    per = {nm: float(np.mean([ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(args.steps)]))
           for j, nm in enumerate(names)}
    ms_step = 1000.0 * wall / args.steps
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; per stage (ms): "
        + ", ".join(f"{k_}={v:.3f}" for k_, v in per.items()))

    n = w.n
    sup = support_tokens(plan, w.key_block, qb)
    gathered = units_read = None
    attn_name = "sparse_attn"
    if qb != 1 and plan.shared_tiles:   # one gather per selection block
        attn_name = "sparse_attn_blocks"
        first = plan.count[::qb].to(torch.int64)
        gathered = int(first.sum().item())
        units_read = gathered
    qk_flops, attn_bytes = algorithmic_work(w, n, k, sup, gathered, units_read)
    peak_mfma = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    kernels = {}
    if w.indexer_d:
        idx_flops = 2 * w.indexer_d * n * (n + 1) // 2 * 2
        kernels["indexer_topk"] = {"bound": "mfma", "work": idx_flops, "ms": per["indexer_topk"]}
    else:
        kernels["pass1_lse"] = {"bound": "mfma", "work": qk_flops, "ms": per["pass1_lse"]}
        kernels[names[1]] = {"bound": "mfma", "work": qk_flops, "ms": per[names[1]]}
        kernels[names[2]] = {"bound": "alu", "work": None, "ms": per[names[2]]}
    # The gather reads its supports through L2: at 32K the layer's K/V fit the
    # MALL and each key window's rows fit an XCD's L2, so its algorithmic
    # bytes are set against the measured L2 read ceiling; the bytes that came
    # from beyond L2 (FETCH_SIZE counters) are reported beside them.
    l2_gbs, _ = l2_read_ceiling()
    # the staging path's ceiling is taken at its best occupancy: 8 workgroups
    # of 16 KiB per CU run it faster than the 10 that fill the LDS
    stage_gbs = max(l2_read_ceiling(mode=2, grid=g)[0] for g in (2048, 2560))
    log(f"[bench] L2 read ceiling (measured): {l2_gbs:.0f} GB/s; 256-byte rows into LDS by "
        f"direct loads: {stage_gbs:.0f} GB/s")
    kernels[attn_name] = {"bound": "l2", "work": attn_bytes, "ms": per["sparse_attn"]}
    # The passes are bound by MFMA and VALU work together at the clock the
    # chip sustains under that load: their rates are also set against the
    # measured rate of their own inner loop run from registers (bf16 only).
    mix = pass_mix_ceiling() if w.dtype == "bf16" else None
    if mix:
        log(f"[bench] pass inner loop ceilings (measured): MFMA chains alone "
            f"{mix['mfma_sustained']:.0f} TFLOP/s, with the exp/sum work {mix['pass_mix']:.0f} TFLOP/s")
    dom = max((kn for kn in kernels if kernels[kn]["work"]), key=lambda kn: kernels[kn]["ms"])
    kd = kernels[dom]
    tkey = w.name if qb == 1 else f"{w.name}_qb{qb}"
    if kd["bound"] == "l2":
        achieved = kd["work"] / (kd["ms"] * 1e-3) / 1e9
        roof = {"bound": "l2", "achieved": achieved, "peak": l2_gbs, "unit": "GB/s",
                "frac": achieved / l2_gbs, "peak_source": "measured L2 read ceiling"}
    else:
        achieved = kd["work"] / (kd["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": achieved / peak_mfma}
    roof["kernel"] = dom
    roof["traffic"] = traffic_for(dom, tkey) if dom in KERNEL_SOURCES else None

    summary = {}
    for kn, kv in kernels.items():
        ent = {"ms": round(kv["ms"], 4), "bound": kv["bound"]}
        if kv["work"]:
            if kv["bound"] == "l2":
                ent["GB/s"] = round(kv["work"] / (kv["ms"] * 1e-3) / 1e9, 1)
                ent["frac_l2"] = round(ent["GB/s"] / l2_gbs, 4)
                ent["l2_ceiling_GB/s"] = round(l2_gbs, 1)
                # the gather stages its rows in LDS by direct global->LDS
                # loads; that path's own measured ceiling
                ent["lds_staging_ceiling_GB/s"] = round(stage_gbs, 1)
                ent["frac_lds_staging"] = round(ent["GB/s"] / stage_gbs, 4)
                beyond = traffic_for(kn, tkey) if kn in KERNEL_SOURCES else None
                ent["beyond_l2_bytes"] = beyond
                if beyond:
                    bgbs = beyond / (kv["ms"] * 1e-3) / 1e9
                    ent["beyond_l2_GB/s"] = round(bgbs, 1)
                    ent["frac_hbm_of_beyond_l2"] = round(bgbs / PEAK_HBM_GBS, 4)
            else:
                ent["TFLOP/s"] = round(kv["work"] / (kv["ms"] * 1e-3) / 1e12, 1)
                ent["frac_mfma"] = round(ent["TFLOP/s"] / peak_mfma, 4)
                if mix and kn in ("pass1_lse", "pass2_filter", "pass2_colsum"):
                    ent["mfma_sustained_TFLOP/s"] = round(mix["mfma_sustained"], 1)
                    ent["pass_mix_ceiling_TFLOP/s"] = round(mix["pass_mix"], 1)
                    ent["frac_pass_mix_ceiling"] = round(ent["TFLOP/s"] / mix["pass_mix"], 4)
        summary[kn] = ent
    if not w.indexer_d:
        t12 = (per["pass1_lse"] + per[names[1]]) * 1e-3
        summary["passes_1_2_frac_mfma"] = round(2 * qk_flops / t12 / 1e12 / peak_mfma, 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline on a row sample ...")
        cpu = cpu_baseline(w, x, k, w.key_block, args.cpu_seconds, qb)
        log(f"[bench] cpu baseline: {cpu['value']:.1f} tokens/s ({cpu['sample']})")

    line = {
        "metric": "oracle+sparse prefill tokens/s per GQA layer at 32K; % MFMA peak, % HBM BW",
        "value": n / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, sink key, planted needle keys)",
        "config": {"workload": w.name if qb == 1 else f"{w.name}_qb{qb}", "n": n, "hq": w.hq,
                   "hkv": w.hkv, "d": w.d, "k": k,
                   "key_block": w.key_block, "query_block": qb, "support_tokens": sup,
                   "parallelism": "none"},
        "roofline": roof,
        "kernels": summary,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
