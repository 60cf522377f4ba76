#!/usr/bin/env python3
"""Benchmark of interval-mask flex attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: mask_plan_build (GPU planner, one header read-back)
followed by flex_attn_fwd over the plan.  Default workload: sliding window
256 + 64-token sink, B=2, H=16, S=2048, d=128, bf16.

Prints ONE JSON line.  `value` is effective TFLOP/s of the whole step, counting
4*d FLOPs per visible (q, k) pair (unmasked score entries only).  The
attention kernel alone is reported under "fwd" and "roofline": its average
launch duration is measured with HIP events on the launch stream, around
back-to-back launches on one plan (the roofline's figure) and around each
forward of a second pass of the steps (those spans also hold host launch
latency).  The timed steps themselves carry no event markers.
"roofline.traffic" is the kernel's HBM bytes per launch from the committed
counter summary, when that summary was taken on the current kernel source.
The CPU oracle is timed on the host cores as "cpu_baseline" (a reported
baseline, not a target).

  --summarize stats|pmc|counters DIRS  digests rocprofv3 csv output instead.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s (unmasked FLOPs) of masked attn fwd + % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (AMD published)
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def plan_rows_tokens(plan):
    """Tokens per plan row: the tile's rows, or tile_q / G for a PackGQA plan
    (whose tile rows are its G heads of tile_q / G tokens)."""
    return plan.problem.tile_q // plan.info.signature.pack_gqa


def plan_stats(w, plan):
    """Algorithmic counts from the plan (no oracle): visible pairs |E|,
    executed tiles, dense-equivalent pairs."""
    import numpy as np
    ex = plan.export()
    p = plan.problem
    tq = plan_rows_tokens(plan)
    pop = int(np.unpackbits(ex["p_masks"].view(np.uint8)).sum()) if ex["p_masks"].size else 0
    pnnz, fnnz = int(ex["header"][1]), int(ex["header"][2])
    per_mask_head = pop + fnnz * tq * p.tile_k
    rep = w.heads_q // w.mask_heads
    visible = per_mask_head * rep
    executed = (pnnz + fnnz) * tq * p.tile_k * rep
    dense = sum(w.sample_bounds(b)[1] * w.sample_bounds(b)[3] for b in range(w.batch)) * w.heads_q
    return {"visible_pairs": visible, "executed_pairs": executed, "dense_pairs": dense,
            "partial_tiles": pnnz, "full_tiles": fnnz, "rows": int(ex["header"][0]),
            "tasks": int(plan.info.num_tasks)}


def plan_bytes(w, plan):
    """Algorithmic bytes of the forward plan build: the endpoints read once;
    the lists, payload (T_Q*T_KV/8 bytes per partial tile), offsets and
    16 bytes per task written once."""
    h = plan.info.header
    p = plan.problem
    rows, pn, fn = int(h[0]), int(h[1]), int(h[2])
    read = 4 * w.mask_heads * w.nfunc * w.total_q
    write = 4 * (pn + fn) + pn * plan_rows_tokens(plan) * p.tile_k // 8 + \
        8 * (w.mask_heads * rows + 1) + 16 * int(plan.info.num_tasks)
    return read + write


def k2q_bytes(w, plan):
    """Algorithmic bytes of the K2Q view's materialization: the endpoints
    read once, then the lists, offsets, K-row prefixes and the K-major
    payload (T_Q*T_KV/8 bytes per partial pair) written once."""
    h = plan.info.header
    p = plan.problem
    krows, pn, fn = int(h[4]), int(h[5]), int(h[6])
    read = 4 * w.mask_heads * w.nfunc * w.total_q
    write = 4 * (pn + fn) + pn * p.tile_q * p.tile_k // 8 + 8 * (w.mask_heads * krows + 1) + \
        4 * (w.batch + 1)
    return read + write


def attn_bytes(w, plan):
    """Algorithmic bytes of one forward launch: Q, K, V and O once each, the
    LSE (4 bytes per row and head), the predicate payload (T_Q*T_KV/8 bytes
    per partial tile) and 4 bytes per listed tile index."""
    h = plan.info.header
    p = plan.problem
    esz = 2 if w.dtype == 0 else 4
    qo = 2 * w.total_q * w.heads_q * w.head_dim * esz
    kv = 2 * w.total_k * w.heads_k * w.head_dim * esz
    pn, fn = int(h[1]), int(h[2])
    return qo + kv + 4 * w.heads_q * w.total_q + pn * plan_rows_tokens(plan) * p.tile_k // 8 + \
        4 * (pn + fn)


def roofline(flops, nbytes, seconds, peak_tflops):
    """The roof that binds: the larger of the MFMA time (flops at the dense
    peak) and the HBM time (algorithmic bytes at 8 TB/s).  `achieved`/`frac`
    are against that roof; both fractions are reported."""
    t_mfma = flops / (peak_tflops * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    mfma_frac = flops / seconds / 1e12 / peak_tflops
    hbm_frac = nbytes / seconds / 1e9 / PEAK_HBM_GBS
    if t_hbm > t_mfma:
        r = {"bound": "hbm", "achieved": round(nbytes / seconds / 1e9, 2), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(hbm_frac, 5)}
    else:
        r = {"bound": "mfma", "achieved": round(flops / seconds / 1e12, 3), "peak": peak_tflops,
             "unit": "TFLOP/s", "frac": round(mfma_frac, 5)}
    r.update({"mfma_frac": round(mfma_frac, 5), "hbm_frac": round(hbm_frac, 5),
              "roof_us": {"mfma": round(t_mfma * 1e6, 3), "hbm": round(t_hbm * 1e6, 3)},
              "intensity_flop_per_byte": round(flops / nbytes, 2),
              "ridge_flop_per_byte": round(peak_tflops * 1e12 / (PEAK_HBM_GBS * 1e9), 2)})
    return r


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


CONFIG_WORKLOADS = ("tiny_causal", "window_sink", "varlen_doc", "block_sparse",
                    "prefix_softcap")


def oracle_sample_rate(w, seconds):
    """The oracle's attention on a bounded random sample of (token, head)
    rows (about `seconds` of CPU work on all host threads): effective
    TFLOP/s = 4*d per visible pair of the sampled rows / time.  Visible
    pairs are counted from the endpoints (bookkeeping, not attention)."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(7)
    # visible keys per (mask head, token): [0,F0) plus [F1,F2), [F3,F4), ...
    mf = w.mask_func.astype(np.int64)
    vis = mf[:, 0, :] + (mf[:, 2::2, :] - mf[:, 1::2, :]).sum(axis=1)
    n = 64
    t_total, flops, rows_done = 0.0, 0.0, 0
    while t_total < seconds and rows_done < w.total_q * w.heads_q:
        rows = np.stack([rng.integers(0, w.total_q, n), rng.integers(0, w.heads_q, n)], axis=1)
        a = time.perf_counter()
        oracle.attention(w, rows=rows)
        t_total += time.perf_counter() - a
        hm = rows[:, 1] if w.mask_heads > 1 else np.zeros(n, np.int64)
        flops += 4.0 * w.head_dim * float(vis[hm, rows[:, 0]].sum())
        rows_done += n
        n = min(n * 2, 4096)
    return flops / t_total / 1e12, rows_done, t_total


def measure_config(name, args, mpb, W, torch, np):
    """One workload at its full size: the library's tile, steady-state
    forward (HIP events around back-to-back launches), the forward inside a
    plan+forward step, plan build (host clock, and GPU stage events), the
    roofline against the binding roof, and the oracle on a bounded sample."""
    w = W.make(name)
    d = W.to_device(w)
    stream = torch.cuda.current_stream()
    prob = mpb.make_problem(w.layout, w.dtype, w.batch, w.seqlen_q, w.seqlen_k, w.total_q,
                            w.total_k, w.heads_q, w.heads_k, w.head_dim, w.mask_heads, w.nfunc,
                            0, 0)
    kw = dict(scale=w.scale, softcap=w.softcap if w.softcap > 0 else None,
              alibi_slopes=d["slopes"], alibi_before_softcap=w.alibi_before_softcap,
              stream=stream)
    plan = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream)
    out, lse = mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
    kw.update(out=out, lse=lse)
    st = plan_stats(w, plan)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
    e0.record(stream)
    for _ in range(args.config_iters):
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_us = e0.elapsed_time(e1) * 1e3 / args.config_iters
    # whole steps (build + forward), host clock around them
    torch.cuda.synchronize()
    keep = []
    a = time.perf_counter()
    for _ in range(args.config_iters):
        p2 = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream)
        mpb.flex_attn_fwd(p2, d["q"], d["k"], d["v"], **kw)
        keep.append(p2)
        if len(keep) > 2:
            keep.pop(0).close()
    torch.cuda.synchronize()
    step_us = (time.perf_counter() - a) * 1e6 / args.config_iters
    for p2 in keep:
        p2.close()
    builds = []
    for _ in range(5):
        torch.cuda.synchronize()
        a = time.perf_counter()
        p3 = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream)
        torch.cuda.synchronize()
        builds.append((time.perf_counter() - a) * 1e6)
        p3.close()
    runs = []
    for _ in range(5):
        p4 = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream,
                                 time_stages=True)
        runs.append(p4.stage_times())
        p4.close()
    stages = _median_stages(runs)
    gpu_us = sum(v for k, v in stages.items() if k != "span" and v > 0)
    pb = plan_bytes(w, plan)
    eff = 4.0 * w.head_dim * st["visible_pairs"]
    exe = 4.0 * w.head_dim * st["executed_pairs"]
    dense = 4.0 * w.head_dim * st["dense_pairs"]
    peak = PEAK_BF16_TFLOPS if w.dtype == W.DTYPE_BF16 else PEAK_FP32_MFMA_TFLOPS
    t = fwd_us * 1e-6
    res = {"workload": name, "dtype": "bf16" if w.dtype == W.DTYPE_BF16 else "f32",
           "tile": "%dx%d" % (plan.problem.tile_q, plan.problem.tile_k),
           "tasks": st["tasks"], "partial_tiles": st["partial_tiles"],
           "full_tiles": st["full_tiles"],
           "fwd_us": round(fwd_us, 2), "step_us": round(step_us, 2),
           "effective_gflop": round(eff / 1e9, 3), "executed_gflop": round(exe / 1e9, 3),
           "dense_gflop": round(dense / 1e9, 3),
           "effective_tflops": round(eff / t / 1e12, 2), "executed_tflops": round(exe / t / 1e12, 2),
           "pct_peak_effective": round(100 * eff / t / 1e12 / peak, 2),
           "pct_peak_executed": round(100 * exe / t / 1e12 / peak, 2),
           "pct_peak_dense_equiv": round(100 * dense / t / 1e12 / peak, 2),
           "roofline": roofline(eff, attn_bytes(w, plan), t, peak),
           "plan_build_us_host": round(float(np.median(builds)), 1), "plan_stages_us": stages,
           "plan_algorithmic_bytes": pb,
           "planner_gbs_over_stages": round(pb / (gpu_us * 1e-6) / 1e9, 1) if gpu_us > 0 else None}
    if not args.no_cpu_baseline:
        rate, rows, secs = oracle_sample_rate(w, args.config_cpu_seconds)
        import oracle
        res["cpu_baseline"] = {"value": round(rate, 6), "unit": "TFLOP/s",
                               "cores": oracle.default_threads(), "kind": "oracle",
                               "sample": "%d random (token, head) rows of fp64 oracle attention in "
                                         "%.1f s" % (rows, secs)}
    plan.close()
    del d
    torch.cuda.empty_cache()
    return res


def _median_stages(runs):
    import numpy as np
    return {k: round(float(np.median([r[k] for r in runs])), 2) for k in runs[0]}


def cpu_baseline(w, tile_q, tile_k, min_seconds=10.0):
    """The oracle, as it is, on the host cores: whole-workload passes of the
    fp64 plan (expand + classify + pack) and attention until min_seconds
    have elapsed.  Returns (total s, passes, threads, plan s, attention s)."""
    import oracle
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    passes = 0
    t_plan = t_attn = 0.0
    while True:
        a = time.perf_counter()
        oracle.build_plan(w, tile_q, tile_k, nthreads=threads)
        b = time.perf_counter()
        oracle.attention(w, nthreads=threads)
        c = time.perf_counter()
        t_plan += b - a
        t_attn += c - b
        passes += 1
        if c - t0 >= min_seconds:
            break
    return time.perf_counter() - t0, passes, threads, t_plan, t_attn


PROBE_LIB = os.path.join(ROOT, "mask_planned_block_amd", "libmpb_probe.so")


def mfma_probe(workgroups, iters, out, stream):
    """Launches the MFMA throughput probe of libmpb_probe.so (include/mpb_probe.h,
    a measurement helper beside the library); returns the launch's flops."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.mpb_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.mpb_mfma_probe.restype = ctypes.c_int
    if out.numel() < workgroups * 256:
        raise ValueError("out needs workgroups*256 floats")
    st = lib.mpb_mfma_probe(int(workgroups), int(iters), ctypes.c_void_p(out.data_ptr()),
                            ctypes.c_void_p(stream.cuda_stream))
    if st != 0:
        raise RuntimeError("mpb_mfma_probe failed with status %d" % st)
    return workgroups * 4 * iters * 8 * 32768


def mfma_peak(torch, iters=4000):
    """Dense bf16 MFMA rate the device sustains: the MFMA probe (independent
    v_mfma_f32_32x32x16_bf16 chains on register operands) on 8 workgroups
    per CU, timed with HIP events; median of 5 launches."""
    import numpy as np
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wg = 8 * cus
    out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    flops = mfma_probe(wg, 200, out, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rates = []
    for _ in range(5):
        e0.record(stream)
        flops = mfma_probe(wg, iters, out, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return {"tflops": round(float(np.median(rates)), 1), "workgroups": wg,
            "pct_of_published": round(100 * float(np.median(rates)) / PEAK_BF16_TFLOPS, 1)}


ATTN_SOURCE = os.path.join(ROOT, "mask_planned_block_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_window_sink_pmc.txt")


def source_digest(path=ATTN_SOURCE):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _kernel_group(name):
    for key in ("attn_fwd_kernel", "plan_single_pass_tail_kernel", "plan_single_pass_kernel",
                "plan_classify_kernel", "plan_schedule_kernel",
                "plan_materialize_kernel", "plan_geometry_kernel", "plan_finish_kernel",
                "plan_k2q_count_kernel", "plan_k2q_materialize_kernel", "attn_bwd_dkdv",
                "attn_bwd_dq_kernel", "attn_bwd_dot_kernel", "elementwise"):
        if key in name:
            return key
    return None


def summarize(kind, dirs, copy_mb=0):
    """Digest of rocprofv3 csv output under the comma-separated `dirs`:
    per-kernel duration statistics (kind "stats") or per-dispatch counter
    averages (kind "pmc": FETCH_SIZE and WRITE_SIZE, in KiB as read).  For
    pmc, the calibration pass (a streaming elementwise kernel that reads and
    writes copy_mb MiB: the largest elementwise dispatch) gives the factor
    between each counter and the bytes it moved; the attention kernel's
    averages scaled by it give its HBM traffic per launch."""
    import csv
    import glob
    paths = lambda pat: sorted(p for d in dirs.split(",") for p in glob.glob(os.path.join(d, pat)))
    if kind == "counters":
        summarize_counters(paths)
        return
    if kind == "stats":
        for path in paths("*kernel_stats.csv"):
            print("# %s" % os.path.basename(path))
            print("%-44s %7s %10s %10s %10s" % ("kernel", "calls", "avg_us", "min_us", "max_us"))
            for r in csv.DictReader(open(path)):
                tmpl = r["Name"].replace("(anonymous namespace)::", "").replace(
                    "mpb::", "").replace("void ", "").split("(")[0]
                print("%-44s %7s %10.2f %10.2f %10.2f" % (
                    tmpl[:44], r["Calls"], float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
        return
    per = {}
    for path in paths("*counter_collection.csv"):
        for r in csv.DictReader(open(path)):
            g = _kernel_group(r["Kernel_Name"])
            if g is not None:
                per.setdefault((g, r["Counter_Name"]), []).append(
                    (int(r["Grid_Size"]), float(r["Counter_Value"])))
    total = 0.0
    complete = True
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cal = per.get(("elementwise", c))
        att = per.get(("attn_fwd_kernel", c))
        if not cal or not att or copy_mb <= 0:
            print("# %s: missing calibration or attention dispatches" % c)
            complete = False
            continue
        grid, v = max(cal)
        factor = copy_mb * 1024.0 / v
        avg = sum(x for _, x in att) / len(att)
        print("calibration %s grid=%d read_kib=%.1f known_kib=%d factor=%.4f"
              % (c, grid, v, copy_mb * 1024, factor))
        print("attn_fwd_kernel %s dispatches=%d avg_kib=%.1f scaled_bytes=%.0f"
              % (c, len(att), avg, avg * 1024 * factor))
        total += avg * 1024 * factor
        for (g, cc), vals in sorted(per.items()):
            if cc == c and g not in ("elementwise", "attn_fwd_kernel"):
                xs = [x for _, x in vals]
                print("%s %s dispatches=%d avg_kib=%.1f scaled_bytes=%.0f"
                      % (g, c, len(xs), sum(xs) / len(xs), sum(xs) / len(xs) * 1024 * factor))
    if complete:
        print("attn_source_sha256_16=%s" % source_digest())
        print("traffic_bytes_per_launch=%.0f" % total)


def summarize_counters(paths):
    """Per-kernel averages of every counter in the counter_collection csv
    files (one pass per directory; at most 8 SQ counters fit one pass), then
    ratios for the attention forward and the planner kernels: VALU and LDS
    instructions per MFMA instruction, the share of MFMA-busy cycles in which
    a VALU instruction issued beside it (SQ_VALU_MFMA_COEXEC_CYCLES over
    SQ_VALU_MFMA_BUSY_CYCLES), and the share of wavefront cycles spent
    waiting on a dependency (SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES) or for
    anything (SQ_WAIT_ANY)."""
    import csv
    per = {}
    for path in paths("*counter_collection.csv"):
        for r in csv.DictReader(open(path)):
            g = _kernel_group(r["Kernel_Name"])
            if g is not None:
                per.setdefault(g, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    for g in sorted(per):
        avg = {c: sum(v) / len(v) for c, v in per[g].items()}
        print("# %s" % g)
        for c in sorted(avg):
            print("%-44s %-28s dispatches=%d avg=%.4g" % (g, c, len(per[g][c]), avg[c]))
        ratios = []
        mf = avg.get("SQ_INSTS_MFMA")
        if mf:
            for c, label in (("SQ_INSTS_VALU", "valu_per_mfma"), ("SQ_INSTS_LDS", "lds_per_mfma")):
                if c in avg:
                    ratios.append((label, avg[c] / mf))
        if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
            ratios.append(("coexec_share_of_mfma_busy",
                           avg["SQ_VALU_MFMA_COEXEC_CYCLES"] / avg["SQ_VALU_MFMA_BUSY_CYCLES"]))
        if avg.get("SQ_WAVE_CYCLES"):
            for c, label in (("SQ_WAIT_INST_ANY", "wait_dependency_share"),
                             ("SQ_WAIT_ANY", "wait_any_share")):
                if c in avg:
                    ratios.append((label, avg[c] / avg["SQ_WAVE_CYCLES"]))
        for label, v in ratios:
            print("%-44s %-28s %.4f" % (g, label, v))


def load_traffic(expected_digest):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on another version of the kernel."""
    try:
        kv = dict(line.strip().split("=", 1) for line in open(TRAFFIC_FILE)
                  if "=" in line and not line.startswith("#"))
        if kv.get("attn_source_sha256_16") != expected_digest:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def run_splitk(args, mpb, W, torch, np):
    """Split-K forward on the long-K chunk shape (512 query tokens against a
    32768-token prefix, 32 Q heads on 8 K/V heads): 128 tasks, fewer than the
    GPU's resident workgroups.  HIP events around back-to-back launches of the
    unsplit forward, of the library's split count and of a sweep; effective
    TFLOP/s = 4*d per visible pair."""
    w = W.make("chunk_long_kv")
    d = W.to_device(w)
    stream = torch.cuda.current_stream()
    prob = mpb.make_problem(w.layout, w.dtype, w.batch, w.seqlen_q, w.seqlen_k, w.total_q,
                            w.total_k, w.heads_q, w.heads_k, w.head_dim, w.mask_heads, w.nfunc,
                            0, 0)
    plan = mpb.mask_plan_build(prob, d["mask_func"], None, None, stream=stream)
    st = plan_stats(w, plan)
    eff = 4.0 * w.head_dim * st["visible_pairs"]
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device="cuda")
    auto = mpb.flex_attn_fwd_num_splits(plan)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(sp):
        ws = None
        if sp is not None:
            ws = torch.empty(max(mpb.flex_attn_fwd_splitk_workspace_size(plan, sp), 256),
                             dtype=torch.uint8, device="cuda")
        call = lambda: mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], scale=w.scale, out=out,
                                         lse=lse, workspace=ws, stream=stream, num_splits=sp)
        for _ in range(3):
            call()
        e0.record(stream)
        for _ in range(args.splitk_iters):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.splitk_iters
        return {"us": round(us, 2), "effective_tflops": round(eff / us / 1e6, 2)}

    res = {"workload": "chunk_long_kv", "tasks": st["tasks"], "library_splits": auto,
           "unsplit": timed(None), "library_choice": timed(0),
           "sweep": {str(sp): timed(sp) for sp in (2, 4, 8, 16, 32)},
           "effective_gflop": round(eff / 1e9, 3),
           "basis": "HIP events around %d back-to-back launches (split launch + merge)"
                    % args.splitk_iters}
    res["speedup_library_choice"] = round(res["unsplit"]["us"] / res["library_choice"]["us"], 3)
    plan.close()
    return res


PACKGQA_SHAPES = {
    # 16-token chunks (decoding a few tokens per sample) against 8192 cached
    # keys, 32 Q heads on 8 K/V heads
    "decode16_g4": dict(batch=8, heads_q=32, heads_k=8, seqlen_q=16, seqlen_k=8192),
    # the long-K chunk: 512 queries against a 32768-token prefix
    "chunk512_g4": dict(),
}


def run_packgqa(args, mpb, W, torch, np):
    """PackGQA against one head per tile on GQA shapes (causal chunks at the
    end of a long prefix): HIP events around back-to-back forwards with the
    library's Split-K choice for each plan; effective TFLOP/s = 4*d per
    visible pair, GB/s = algorithmic forward bytes per launch."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for name, shape in PACKGQA_SHAPES.items():
        w = W.chunk_long_kv(**shape)
        d = W.to_device(w)
        prob = mpb.make_problem(w.layout, w.dtype, w.batch, w.seqlen_q, w.seqlen_k, w.total_q,
                                w.total_k, w.heads_q, w.heads_k, w.head_dim, w.mask_heads,
                                w.nfunc, 0, 0)
        o = torch.empty_like(d["q"])
        lse = torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device="cuda")
        row = {"batch": w.batch, "heads_q": w.heads_q, "heads_k": w.heads_k,
               "seqlen_q": w.seqlen_q, "seqlen_k": w.seqlen_k}
        for label, pack in (("unpacked", False), ("packed", True)):
            plan = mpb.mask_plan_build(prob, d["mask_func"], None, None, stream=stream,
                                       pack_gqa=pack)
            st = plan_stats(w, plan)
            eff = 4.0 * w.head_dim * st["visible_pairs"]
            sp = mpb.flex_attn_fwd_num_splits(plan)
            ws = torch.empty(max(mpb.flex_attn_fwd_splitk_workspace_size(plan, 0), 256),
                             dtype=torch.uint8, device="cuda")
            call = lambda: mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], scale=w.scale,
                                             out=o, lse=lse, workspace=ws, stream=stream,
                                             num_splits=0 if sp > 1 else None)
            for _ in range(3):
                call()
            e0.record(stream)
            for _ in range(args.packgqa_iters):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / args.packgqa_iters
            row[label] = {"us": round(us, 2), "tasks": st["tasks"], "splits": sp,
                          "effective_tflops": round(eff / us / 1e6, 2),
                          "gbs": round(attn_bytes(w, plan) / us / 1e3, 1)}
            plan.close()
        row["speedup"] = round(row["unpacked"]["us"] / row["packed"]["us"], 3)
        out[name] = row
    out["basis"] = ("HIP events around %d back-to-back forwards (split launch + merge where "
                    "the library splits)" % args.packgqa_iters)
    return out


def run_paged(args, w, d, plan, kw, mpb, torch, np):
    """Paged K/V overhead: the main workload's K/V scattered into a page pool
    (pages of 2 * tile_k tokens, random page order) and the paged forward
    (remap launch + forward) timed against the contiguous forward on the same
    plan; HIP events around back-to-back launches."""
    p = plan.problem
    ps = 2 * p.tile_k
    g = torch.Generator().manual_seed(0)
    need = [-(-w.sample_bounds(b)[3] // ps) for b in range(w.batch)]
    pps = max(max(need), -(-w.seqlen_k // ps), 1)
    num_pages = sum(need)
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((w.batch, pps), -1, dtype=torch.int32)
    src, dst = [], []
    nxt = 0
    for b in range(w.batch):
        _, _, k_off, k_len = w.sample_bounds(b)
        for lp in range(need[b]):
            table[b, lp] = int(perm[nxt])
            nxt += 1
        kk = torch.arange(k_len)
        src.append(k_off + kk)
        dst.append(table[b, kk // ps].long() * ps + kk % ps)
    src, dst = torch.cat(src).cuda(), torch.cat(dst).cuda()
    kflat = d["k"].reshape(-1, w.heads_k, w.head_dim)
    vflat = d["v"].reshape(-1, w.heads_k, w.head_dim)
    kp = torch.zeros((num_pages * ps, w.heads_k, w.head_dim), dtype=kflat.dtype, device="cuda")
    vp = torch.zeros_like(kp)
    kp[dst] = kflat[src]
    vp[dst] = vflat[src]
    table = table.cuda()
    stream = kw["stream"]
    ws = torch.empty(max(mpb.flex_attn_fwd_paged_workspace_size(plan, 1), 256),
                     dtype=torch.uint8, device="cuda")
    kw_p = {k: v for k, v in kw.items() if k not in ("workspace", "num_splits")}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(call):
        for _ in range(3):
            call()
        e0.record(stream)
        for _ in range(args.fwd_iters):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.fwd_iters

    us_p = timed(lambda: mpb.flex_attn_fwd_paged(plan, d["q"], kp, vp, table, ps, workspace=ws,
                                                 **kw_p))
    us_r = timed(lambda: mpb.flex_attn_fwd_paged(plan, d["q"], kp, vp, table, ps, workspace=ws,
                                                 remap=False, **kw_p))
    us_c = timed(lambda: mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw_p))
    o_p = kw_p["out"].clone()
    mpb.flex_attn_fwd_paged(plan, d["q"], kp, vp, table, ps, workspace=ws, **kw_p)
    torch.cuda.synchronize()
    same = bool(torch.equal(o_p, kw_p["out"]))
    return {"page_size": ps, "num_pages": num_pages, "us_with_remap": round(us_p, 2),
            "us_reusing_remap": round(us_r, 2), "contiguous_us": round(us_c, 2),
            "overhead_pct_with_remap": round(100 * (us_p / us_c - 1), 2),
            "overhead_pct_reusing_remap": round(100 * (us_r / us_c - 1), 2),
            "identical_output": same,
            "basis": "HIP events around %d back-to-back calls (remap launch + forward, or the "
                     "forward alone on lists remapped once)" % args.fwd_iters}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="window_sink")
    ap.add_argument("--tile-q", type=int, default=0)
    ap.add_argument("--tile-k", type=int, default=0)
    ap.add_argument("--fwd-iters", type=int, default=100,
                    help="extra back-to-back forward launches on one plan (steady state)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ablation", action="store_true",
                    help="also time the forward with full tiles forced through the masked path")
    ap.add_argument("--dense-reference", action="store_true",
                    help="also time the all-visible forward at the same shape")
    ap.add_argument("--bwd-iters", type=int, default=20,
                    help="back-to-back backward launches timed on a plan with the K2Q view "
                         "(bf16 workloads; 0 = skip)")
    ap.add_argument("--num-splits", type=int, default=None,
                    help="run the step's forward as the Split-K forward with this many parts "
                         "(0 = the library's choice)")
    ap.add_argument("--splitk-iters", type=int, default=20,
                    help="back-to-back launches per Split-K configuration timed on the long-K "
                         "chunk shape (0 = skip)")
    ap.add_argument("--sync-build", action="store_true",
                    help="time the step with the header read back inside mask_plan_build "
                         "(default: defer_header, the build returns once its launches are "
                         "enqueued)")
    ap.add_argument("--packgqa-iters", type=int, default=20,
                    help="back-to-back forwards per plan in the PackGQA leg (0 = skip)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged K/V overhead leg")
    ap.add_argument("--cold-iters", type=int, default=5,
                    help="forwards timed after writing 512 MiB through HBM (0 = skip)")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the MFMA throughput probe")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="end with plain device copies of this many MiB (counter calibration)")
    ap.add_argument("--config-iters", type=int, default=20,
                    help="launches per workload in the per-config table (0 = skip the table)")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="oracle seconds per workload in the per-config table")
    ap.add_argument("--summarize", nargs=2, metavar=("KIND", "DIRS"),
                    help="print a summary of rocprofv3 csv output under comma-separated DIRS "
                         "(KIND: stats, pmc or counters) and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize[0], args.summarize[1], args.copy_calibration_mb)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mask_planned_block_amd as mpb
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = W.make(args.workload)
    d = W.to_device(w)
    prob = mpb.make_problem(w.layout, w.dtype, w.batch, w.seqlen_q, w.seqlen_k, w.total_q,
                            w.total_k, w.heads_q, w.heads_k, w.head_dim, w.mask_heads, w.nfunc,
                            args.tile_q, args.tile_k)
    stream = torch.cuda.current_stream()
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device="cuda")
    ws = None
    kw = dict(scale=w.scale, softcap=w.softcap if w.softcap > 0 else None,
              alibi_slopes=d["slopes"], alibi_before_softcap=w.alibi_before_softcap,
              out=out, lse=lse, workspace=ws, stream=stream)
    if args.num_splits is not None:
        p0 = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream)
        kw["num_splits"] = args.num_splits
        kw["workspace"] = torch.empty(max(mpb.flex_attn_fwd_splitk_workspace_size(
            p0, args.num_splits), 256), dtype=torch.uint8, device="cuda")
        p0.close()

    defer = not args.sync_build

    def build(deferred=defer):
        return mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream,
                                   defer_header=deferred)

    def step():
        plan = build()
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
        return plan

    # warmup (also compiles nothing: kernels are prebuilt)
    plans = [step() for _ in range(max(args.warmup, 1))]
    torch.cuda.synchronize()
    stats = plan_stats(w, plans[-1])
    tq, tk = plans[-1].problem.tile_q, plans[-1].problem.tile_k
    del plans

    # timed steps: plan build + forward, nothing else on the stream
    keep = []
    host_build = host_fwd = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ta = time.perf_counter()
        plan = build()
        tb = time.perf_counter()
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
        tc = time.perf_counter()
        host_build += tb - ta
        host_fwd += tc - tb
        keep.append(plan)          # released in stream order once no longer needed
        if len(keep) > 2:
            keep.pop(0).close()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / args.steps
    # a deferred plan's GPU checks are read here, after the timed region: the
    # last step's plan must have passed them and its forward's output must be
    # the one a plan built with the header read-back gives
    if defer:
        assert keep[-1].info.build_mode == mpb.BUILD_SINGLE_PASS_DEFERRED
        o_def, l_def = out.clone(), lse.clone()
        p_chk = build(False)
        mpb.flex_attn_fwd(p_chk, d["q"], d["k"], d["v"], **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, o_def) and torch.equal(lse, l_def), "deferred != read-back"
        p_chk.close()

    # the same steps with the header read back inside the build (the host
    # waits for it before it enqueues the forward)
    torch.cuda.synchronize()
    t0s = time.perf_counter()
    for i in range(args.steps):
        plan = build(False)
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
        keep.append(plan)
        if len(keep) > 2:
            keep.pop(0).close()
    torch.cuda.synchronize()
    step_sync_s = (time.perf_counter() - t0s) / args.steps

    # the same steps again, each forward bracketed by HIP events (the event
    # markers perturb the step, so this loop is not the timed one)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        plan = build()
        ev[i][0].record(stream)
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
        ev[i][1].record(stream)
        keep.append(plan)
        if len(keep) > 2:
            keep.pop(0).close()
    torch.cuda.synchronize()
    fwd_in_step_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    fwd_in_step_med_us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3

    # steady-state forward on one plan (back-to-back launches)
    plan = keep[-1]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
    e0.record(stream)
    for _ in range(args.fwd_iters):
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_ss_us = e0.elapsed_time(e1) * 1e3 / args.fwd_iters

    abl = None
    if args.ablation:
        e0.record(stream)
        for _ in range(args.fwd_iters):
            mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], force_partial=True, **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        abl = e0.elapsed_time(e1) * 1e3 / args.fwd_iters

    # plan build alone (host clock around the call, includes its one sync)
    tb = []
    for _ in range(10):
        torch.cuda.synchronize()
        a = time.perf_counter()
        p2 = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream)
        torch.cuda.synchronize()
        tb.append(time.perf_counter() - a)
        p2.close()
    plan_us = float(np.median(tb)) * 1e6

    def build_runs(bwd, timed, n=10):
        """n builds, each alone on the stream: host clock around the call
        (with its one sync), or the GPU stage times from its HIP events."""
        out = []
        for _ in range(n):
            torch.cuda.synchronize()
            a = time.perf_counter()
            p3 = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream,
                                     build_backward=bwd, time_stages=timed)
            torch.cuda.synchronize()
            out.append(p3.stage_times() if timed else time.perf_counter() - a)
            if len(out) < n:
                p3.close()
        return out, p3

    stage_runs, p3 = build_runs(False, True)
    pb = plan_bytes(w, p3)
    p3.close()
    plan_stages = _median_stages(stage_runs)
    gpu_us = sum(v for k, v in plan_stages.items() if k != "span" and v > 0)
    # the backward K2Q view added to the same build
    tbk, p3 = build_runs(True, False)
    p3.close()
    k2q_runs, pk = build_runs(True, True)
    k2q_stages = _median_stages(k2q_runs)
    kb = k2q_bytes(w, pk)
    kmat = k2q_stages["k2q_materialize"]
    kh = pk.info.header
    plan_k2q = {"tile": "%dx%d" % (pk.problem.tile_q, pk.problem.tile_k),
                "build_us_host": round(float(np.median(tbk)) * 1e6, 1), "stages_us": k2q_stages,
                "k_rows": int(kh[4]), "partial": int(kh[5]), "full": int(kh[6]),
                "materialize_algorithmic_bytes": kb,
                "materialize_gbs": round(kb / (kmat * 1e-6) / 1e9, 1) if kmat > 0 else None,
                "materialize_frac_hbm": round(kb / (kmat * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                if kmat > 0 else None}
    pk.close()

    # all-visible forward at the same shape (nfunc = 1, F0 = k_len): the
    # dense attention this mask skips most of
    dense_ref = None
    if args.dense_reference and w.layout == W.LAYOUT_BSHD:
        mf_all = torch.full((1, 1, w.total_q), w.seqlen_k, dtype=torch.int32, device="cuda")
        prob_all = mpb.make_problem(w.layout, w.dtype, w.batch, w.seqlen_q, w.seqlen_k, w.total_q,
                                    w.total_k, w.heads_q, w.heads_k, w.head_dim, 1, 1,
                                    args.tile_q, args.tile_k)
        plan_all = mpb.mask_plan_build(prob_all, mf_all, None, None, stream=stream)
        kw_all = dict(kw, softcap=None, alibi_slopes=None)
        for _ in range(3):
            mpb.flex_attn_fwd(plan_all, d["q"], d["k"], d["v"], **kw_all)
        e0.record(stream)
        for _ in range(args.fwd_iters):
            mpb.flex_attn_fwd(plan_all, d["q"], d["k"], d["v"], **kw_all)
        e1.record(stream)
        torch.cuda.synchronize()
        us_all = e0.elapsed_time(e1) * 1e3 / args.fwd_iters
        fl_all = 4.0 * w.head_dim * w.total_q * w.seqlen_k * w.heads_q
        peak_all = PEAK_BF16_TFLOPS if w.dtype == W.DTYPE_BF16 else PEAK_FP32_MFMA_TFLOPS
        dense_ref = {"us": round(us_all, 2), "tflops": round(fl_all / us_all / 1e6, 2),
                     "pct_peak": round(100 * fl_all / us_all / 1e6 / peak_all, 2)}
        plan_all.close()

    # backward (not part of the step): a plan with the K2Q view, the forward's
    # O and LSE, a seeded dO; HIP events around back-to-back launches
    bwd = None
    if args.bwd_iters > 0 and w.dtype == W.DTYPE_BF16:
        pbw = mpb.mask_plan_build(prob, d["mask_func"], d["cu_q"], d["cu_k"], stream=stream,
                                  build_backward=True)
        ob, lb = mpb.flex_attn_fwd(pbw, d["q"], d["k"], d["v"], **dict(kw, out=None, lse=None))
        dout = torch.from_numpy(W.grad_output(w)).to(torch.bfloat16).reshape(d["q"].shape).cuda()
        dq_b, dk_b, dv_b = (torch.empty_like(d["q"]), torch.empty_like(d["k"]),
                            torch.empty_like(d["v"]))
        ws_b = torch.empty(mpb.flex_attn_bwd_workspace_size(pbw), dtype=torch.uint8, device="cuda")
        kw_b = dict(scale=w.scale, softcap=w.softcap if w.softcap > 0 else None,
                    alibi_slopes=d["slopes"], alibi_before_softcap=w.alibi_before_softcap,
                    dq=dq_b, dk=dk_b, dv=dv_b, workspace=ws_b, stream=stream)
        for _ in range(3):
            mpb.flex_attn_bwd(pbw, d["q"], d["k"], d["v"], ob, lb, dout, **kw_b)
        e0.record(stream)
        for _ in range(args.bwd_iters):
            mpb.flex_attn_bwd(pbw, d["q"], d["k"], d["v"], ob, lb, dout, **kw_b)
        e1.record(stream)
        torch.cuda.synchronize()
        bwd_us = e0.elapsed_time(e1) * 1e3 / args.bwd_iters
        # algorithmic work: five products per visible pair (S, dP, dV, dQ, dK)
        eff_b = 10.0 * w.head_dim * stats["visible_pairs"]
        dense_b = 10.0 * w.head_dim * stats["dense_pairs"]
        bwd = {"tile": "%dx%d" % (pbw.problem.tile_q, pbw.problem.tile_k),
               "us": round(bwd_us, 2), "effective_tflops": round(eff_b / bwd_us / 1e6, 3),
               "dense_equiv_tflops": round(dense_b / bwd_us / 1e6, 3),
               "pct_peak_dense_equiv": round(100 * dense_b / bwd_us / 1e6 / PEAK_BF16_TFLOPS, 2),
               "flops_basis": "10*d per visible pair (S, dP, dV, dQ, dK); the kernels also "
                              "recompute S and dP in both the dQ and the dK/dV launch"}
        pbw.close()

    splitk = run_splitk(args, mpb, W, torch, np) if args.splitk_iters > 0 else None
    packgqa = run_packgqa(args, mpb, W, torch, np) if args.packgqa_iters > 0 else None
    paged = None
    if not args.no_paged and w.dtype == W.DTYPE_BF16 and args.num_splits is None:
        paged = run_paged(args, w, d, plan, kw, mpb, torch, np)

    # cold forward: 512 MiB written through HBM first (more than the 256 MiB
    # MALL), then one forward, HIP events around it; median of 5
    cold = []
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if args.cold_iters else None
    for _ in range(args.cold_iters):
        scratch.fill_(1)
        e0.record(stream)
        mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], **kw)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    fwd_cold_us = float(np.median(cold)) if cold else None
    mfma = None if args.no_mfma_probe else mfma_peak(torch)

    if args.copy_calibration_mb > 0:
        # streaming calibration: reads and writes exactly copy_calibration_mb MiB
        src = torch.ones((args.copy_calibration_mb << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()

    d_ = w.head_dim
    eff = 4.0 * d_ * stats["visible_pairs"]
    exe = 4.0 * d_ * stats["executed_pairs"]
    dense = 4.0 * d_ * stats["dense_pairs"]
    peak = PEAK_BF16_TFLOPS if w.dtype == W.DTYPE_BF16 else PEAK_FP32_MFMA_TFLOPS
    fwd_s = fwd_in_step_us * 1e-6
    # roofline: the kernel's average launch duration from the back-to-back
    # launches on one plan (HIP events on the launch stream); the per-step
    # event spans also hold the host's launch latency
    roof = roofline(eff, attn_bytes(w, plan), fwd_ss_us * 1e-6, peak)
    traffic = load_traffic(source_digest()) if args.workload == "window_sink" else None
    configs = None
    if args.config_iters > 0:
        configs = {name: measure_config(name, args, mpb, W, torch, np)
                   for name in CONFIG_WORKLOADS}

    res = {
        "metric": METRIC,
        "value": round(eff / step_s / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "ms_per_step_header_read_back": round(step_sync_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.DTYPE_BF16 else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, endpoints from the workload definition)",
        "config": {"workload": args.workload, "batch": w.batch, "heads_q": w.heads_q,
                   "heads_k": w.heads_k, "seqlen_q": w.seqlen_q, "seqlen_k": w.seqlen_k,
                   "head_dim": w.head_dim, "mask_heads": w.mask_heads, "nfunc": w.nfunc,
                   "tile": "%dx%d" % (tq, tk),
                   "step": "mask_plan_build (%s) + flex_attn_fwd"
                           % ("header read back in the build" if not defer
                              else "defer_header: the first header read follows the timed "
                                   "steps")},
        "roofline": dict(roof, traffic=traffic, kernel="attn_fwd_kernel",
                         algorithmic_bytes=attn_bytes(w, plan),
                         achieved_basis="algorithmic bytes (hbm) or effective flops (mfma) per "
                         "launch / average launch duration (HIP events around %d back-to-back "
                         "launches on the launch stream); the binding roof is the larger of "
                         "flops / MFMA peak and bytes / 8 TB/s" % args.fwd_iters,
                         measured_mfma_peak=mfma),
        "fwd": {
            "us_in_step": round(fwd_in_step_us, 2),
            "us_steady": round(fwd_ss_us, 2),
            "effective_tflops": round(eff / fwd_s / 1e12, 3),
            "executed_tflops": round(exe / fwd_s / 1e12, 3),
            "dense_equiv_tflops": round(dense / fwd_s / 1e12, 3),
            "pct_peak_dense_equiv": round(100 * dense / fwd_s / 1e12 / peak, 2),
            "pct_peak_executed": round(100 * exe / fwd_s / 1e12 / peak, 2),
            "effective_gflop": round(eff / 1e9, 4), "executed_gflop": round(exe / 1e9, 4),
            "dense_gflop": round(dense / 1e9, 4),
            "force_partial_us": None if abl is None else round(abl, 2),
            "us_in_step_median": round(fwd_in_step_med_us, 2),
            "us_cold": None if fwd_cold_us is None else round(fwd_cold_us, 2),
            "dense_all_visible": dense_ref,
        },
        "plan": {"build_us_host": round(plan_us, 1), "stages_us": plan_stages,
                 "algorithmic_bytes": pb, "gbs_over_stages": round(pb / (gpu_us * 1e-6) / 1e9, 1),
                 **stats},
        "plan_k2q": plan_k2q,
        "bwd": bwd,
        "splitk": splitk,
        "packgqa": packgqa,
        "paged": paged,
        "host": {"build_call_us": round(host_build / args.steps * 1e6, 1),
                 "fwd_call_us": round(host_fwd / args.steps * 1e6, 1)},
        "configs": configs,
    }
    if not args.no_cpu_baseline:
        secs, passes, threads, t_plan, t_attn = cpu_baseline(w, tq, tk, args.cpu_seconds)
        res["cpu_baseline"] = {
            "value": round(eff * passes / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d whole-workload pass(es) of the fp64 oracle (plan + attention, every "
                      "row) in %.1f s" % (passes, secs),
            "plan_s_per_pass": round(t_plan / passes, 4),
            "attention_s_per_pass": round(t_attn / passes, 4)}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
