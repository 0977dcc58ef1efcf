"""Throughput of the block-scaled (grouped) GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--tile ID] [--no-cpu-baseline]

One step = one call of the library entry point for the workload (the whole
hot path: routing discovery, LDS staging, MFMA, per-block rescale, BF16
epilogue) on inputs already resident in HBM.  W untimed steps, then exactly
K timed steps between two synchronisations, timed with HIP events recorded
on the stream the kernels run on.  By default the K steps are captured in
one HIP graph and the timed region is one replay of it (after an untimed
replay), the way a captured MoE layer runs them; --stream times K launches
issued one by one instead.  The line carries the other mode's figure too
(ms_per_step_stream or ms_per_step_graph), timed second in the same
process, and `cold_cache`: the median of single launches, each after a read
of 512 MB that evicts L2 and the last-level cache, beside the median of the
same single launches warm.  Prints one JSON line.

Default workload: grouped FP8 MoE prefill, G=8, M=8192 routed rows in sorted
runs (multinomial counts, unaligned to 128), N=4096, K=7168.

TFLOPS = 2 * (real rows) * N * K / time; padding rows (m_indices = -1) are
excluded.  `value` is whole-job throughput (the timed region over K).
`roofline` prices the kernel against MI355X's published dense MFMA peak for
the arithmetic it uses, at the same average launch duration
(`us_per_launch`).  `cpu_baseline` is the float64 CPU
oracle timed on a bounded row sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS and % of MFMA peak, grouped FP8 / NVFP4 block-scaled GEMM"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK = {"fp8": 5000.0, "fp4": 10100.0, "fp16": 2500.0, "bf16": 2500.0}
HBM_PEAK = 8000.0
TIMING = {"graph": "one HIP graph replay of K captured launches",
          "stream": "K launches issued one by one on the stream"}
OTHER = {"graph": "stream", "stream": "graph"}

WORKLOADS = {
    "c2_moe_fp8": dict(kind="fp8", desc="grouped FP8 MoE prefill, G=8, M=8192, N=4096, K=7168"),
    "c3_skewed_fp8": dict(kind="fp8", desc="skewed grouped FP8, G=32 Zipf(1.2), M=16384 incl. "
                          "padding, N=2048, K=7168; runs padded to 128 rows",
                          run_align=128),
    "c4_dense_nvfp4": dict(kind="fp4", desc="dense NVFP4, M=2048, N=36864, K=4608"),
    "c5_moe_nvfp4": dict(kind="fp4", desc="grouped NVFP4 W4A4 MoE prefill, G=8x8192 rows, "
                         "N=8192, K=8192"),
    "c1_tiny_fp8": dict(kind="fp8", desc="tiny grouped FP8, G=2, M=256, N=256, K=512"),
    "d5_decode_w4a16": dict(kind="w4a16",
                            desc="W4A16 decode on c5's experts: 64 tokens x top-2 of G=8 (128 "
                                 "rows), BF16 activations x NVFP4 B [8, 8192, 8192]"),
    "p4_problems_nvfp4": dict(kind="fp4_problems",
                              desc="8 NVFP4 problems of different shapes in one launch: "
                                   "multinomial(16384) rows, (N, K) alternately (4096, 7168) and "
                                   "(7168, 2048)"),
    "p8_problems_fp8": dict(kind="fp8_problems",
                            desc="8 block-scaled FP8 problems of different shapes in one launch: "
                                 "multinomial(16384) rows, (N, K) alternately (4096, 7168) and "
                                 "(7168, 2048)"),
    # Latency shapes of the flashinfer#7877 page's timing table: launch-bound,
    # the interesting figure is ms_per_step.
    "p2_unaligned": dict(kind="fp8", desc="small grouped FP8, G=2, M=65, N=128, K=128"),
    "p2_m777_g8": dict(kind="fp8", desc="small grouped FP8, G=8, M=777, N=256, K=512"),
    # The activation quantisers (the step before the GEMM), on the A-operand
    # shapes of c2 and c5: HBM-bound, reported in GB/s.
    "q_fp8_c2": dict(kind="quant_fp8", M=8192, K=7168,
                     desc="BF16 -> FP8 1x128 activations of c2, M=8192, K=7168"),
    "q_nvfp4_c5": dict(kind="quant_nvfp4", M=65536, K=8192,
                       desc="BF16 -> NVFP4 activations of c5, M=65536, K=8192"),
    "q_nvfp4_static_c5": dict(kind="quant_nvfp4_static", M=65536, K=8192,
                              desc="BF16 -> NVFP4 activations of c5 with a calibrated global "
                                   "scale (amax of the first 64 rows / 2688), M=65536, K=8192"),
    # The quantiser fused with the MoE row expansion: c2's A operand built
    # from 4096 tokens routed top-2 of 8 experts (8192 expanded rows).
    "q_fp8_expand_c2": dict(kind="quant_fp8_expand", M=8192, K=7168, T=4096, G=8, top_k=2,
                            desc="token rows -> expert-ordered FP8 1x128 A operand of c2: "
                                 "4096 BF16 tokens x top-2 of 8 experts (8192 rows), K=7168"),
}
QUANT_METRIC = "GB/s (algorithmic bytes / time) and % of HBM peak, activation quantiser"


# Source files each workload's kernels are built from: a committed traffic
# profile stays valid while these are unchanged.
KERNEL_SOURCES = {
    "fp8": ("fp8_grouped.hip", "common.h", "offsets.h"),
    "fp4": ("fp4.hip", "common.h", "offsets.h"),
    "fp4_problems": ("fp4.hip", "common.h", "offsets.h"),
    "fp8_problems": ("fp8_grouped.hip", "common.h", "offsets.h"),
    "quant_fp8": ("quant.hip", "common.h"),
    "quant_nvfp4": ("quant.hip", "common.h"),
    "quant_nvfp4_static": ("quant.hip", "common.h"),
    "quant_fp8_expand": ("quant.hip", "common.h"),
    "w4a16": ("w4a16.hip", "common.h", "offsets.h"),
}


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp4_grouped_gemm_amd", "csrc")
    for f in KERNEL_SOURCES[WORKLOADS[workload]["kind"]]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != src_hash:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(p: dict) -> float:
    """Bytes a launch must move at least once: A rows and scales of real
    rows, B and its scales of non-empty experts, all of C."""
    M, N, K, G = p["M"], p["N"], p["K"], p["G"]
    ids = p.get("m_indices")
    if p["kind"] == "fp8":
        real = M if ids is None else int(np.count_nonzero((ids >= 0) & (ids < G)))
        used = G if ids is None else len(set(ids[(ids >= 0) & (ids < G)].tolist()))
        return real * K + real * (K // 128) * 4 + used * N * K + used * (N // 128) * (K // 128) * 4 \
            + M * 4 + M * N * 2
    real = M if ids is None else int(np.count_nonzero((ids >= 0) & (ids < G)))
    used = 1 if ids is None else len(set(ids[(ids >= 0) & (ids < G)].tolist()))
    return real * (K // 2 + K // 16) + used * N * (K // 2 + K // 16) + M * N * 2 + \
        (0 if ids is None else M * 4)


def host_threads():
    """(cores this process may run on, BLAS threads the oracle's matrix
    products use)."""
    from threadpoolctl import threadpool_info
    blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return len(os.sched_getaffinity(0)), int(blas)


def cpu_baseline(p: dict, C_gpu, seconds: float):
    """Time the oracle on a bounded row sample of the workload (chunks of
    rows in a seeded random order until ``seconds`` of CPU work or all rows),
    and check those rows of the GPU output against it."""
    import oracle
    from threadpoolctl import threadpool_info

    from fp4_grouped_gemm_amd.util import c_to_f64, row_ids
    M = p["M"]
    order = np.random.default_rng(1).permutation(M)
    ids_all = row_ids(p)
    done, refs = [], []
    t0 = time.perf_counter()
    for c0 in range(0, M, 256):
        rows = np.sort(order[c0:c0 + 256])
        if p["kind"] == "fp8":
            r = oracle.grouped_fp8_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], ids_all,
                                        rows=rows)
        elif p.get("m_indices") is None:
            r = oracle.fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], p["alpha"], rows=rows)
        else:
            r = oracle.grouped_fp4_gemm(p["A"], p["B"], p["a_scale"], p["b_scale"], ids_all,
                                        p["alpha"], rows=rows)
        done.append(rows)
        refs.append(r)
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    rows = np.concatenate(done)
    ref = np.concatenate(refs)
    ids = None if ids_all is None else ids_all[rows]
    real = int(rows.size if ids is None else np.count_nonzero(ids >= 0))
    flops = 2.0 * real * p["N"] * p["K"]
    cores, blas = host_threads()
    res = oracle.check_tolerance(c_to_f64(C_gpu)[rows], ref, ids)
    base = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOPS", "cores": cores,
            "blas_threads": blas,
            "kind": "oracle",
            "sample": f"{rows.size} of {M} rows ({real} non-padding) x all {p['N']} columns of "
                      f"the same workload, float64 NumPy/BLAS, {dt:.1f} s"}
    parity = {"rows": int(rows.size), "ok": bool(res["ok"]),
              "worst_ratio": round(res["worst_ratio"], 4)}
    return base, parity


def _csv_rows(path_glob):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(path_glob)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def rocprof_summary(root: str, workload: str, kernel: str, command: str) -> str:
    """Summarise rocprofv3 CSV output under `root` (subdirectories trace/,
    fetch/, write/, cfetch/, cwrite/ as written by the profiling commands in
    the returned text) for kernels whose name contains `kernel`.  Returns the
    text summary and writes profiles/traffic_<workload>.txt."""
    def mean(xs):
        return sum(xs) / len(xs) if xs else float("nan")
    trace = [r for r in _csv_rows(f"{root}/trace/*kernel_trace.csv") if kernel in r["Kernel_Name"]]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    stats = [r for r in _csv_rows(f"{root}/trace/*kernel_stats.csv") if kernel in r["Name"]]

    def counter(sub, name, kname):
        rows = [r for r in _csv_rows(f"{root}/{sub}/*counter_collection.csv")
                if r["Counter_Name"] == name and kname in r["Kernel_Name"]]
        return [float(r["Counter_Value"]) for r in rows]
    fetch = counter("fetch", "FETCH_SIZE", kernel)
    write = counter("write", "WRITE_SIZE", kernel)
    cf = counter("cfetch", "FETCH_SIZE", "copyBuffer")
    cw = counter("cwrite", "WRITE_SIZE", "copyBuffer")
    gib_kib = float(1 << 20)
    f_scale = gib_kib / mean(cf) if cf else float("nan")
    w_scale = gib_kib / mean(cw) if cw else float("nan")
    hbm = mean(fetch) * 1024 * f_scale + mean(write) * 1024 * w_scale
    lines = [
        f"# rocprofv3 summary: {kernel} on {workload}",
        "",
        f"command: {command}",
        f"kernel_source_sha={kernel_source_hash(workload)}",
        f"dispatches traced: {len(durs)}; mean duration {mean(durs):.2f} us; "
        f"min {min(durs) if durs else float('nan'):.2f} us; max {max(durs) if durs else float('nan'):.2f} us",
    ]
    # The profiled run's own result line (its stdout, saved beside the CSVs):
    # its timed region is the last `steps` dispatches of the kernel.
    run = None
    log = os.path.join(root, "trace.log")
    if os.path.exists(log):
        with open(log) as fh:
            for line in fh:
                if line.startswith('{"metric"'):
                    run = json.loads(line)
    if run and durs:
        k = min(int(run["steps"]), len(durs))
        lines.append(f"timed region of that run (its last {k} dispatches): mean "
                     f"{mean(durs[-k:]):.2f} us; the run's own line: "
                     f"{run['roofline']['us_per_launch']} us per step")
    for r in stats:
        lines.append("kernel_stats: " + ", ".join(f"{k}={v}" for k, v in r.items()))
    lines += [
        f"FETCH_SIZE per dispatch (KiB): mean {mean(fetch):.1f} over {len(fetch)}",
        f"WRITE_SIZE per dispatch (KiB): mean {mean(write):.1f} over {len(write)}",
        f"copy calibration (1 GiB read + 1 GiB written): FETCH_SIZE {mean(cf):.1f} KiB, "
        f"WRITE_SIZE {mean(cw):.1f} KiB -> scale fetch x{f_scale:.4f}, write x{w_scale:.4f}",
        f"hbm_bytes_per_launch={hbm:.0f}",
    ]
    text = "\n".join(lines) + "\n"
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.txt"), "w") as fh:
        fh.write(f"# HBM traffic of {kernel} on {workload}, from rocprofv3 FETCH_SIZE/WRITE_SIZE\n")
        fh.write(f"# scaled by a 1 GiB copy calibration (fetch x{f_scale:.4f}, write x{w_scale:.4f})\n")
        fh.write(f"# command: {command}\n")
        fh.write(f"kernel_source_sha={kernel_source_hash(workload)}\n")
        fh.write(f"mean_duration_us={mean(durs):.3f}\n")
        fh.write(f"hbm_bytes_per_launch={hbm:.0f}\n")
    return text


def quant_bytes(kind: str, M: int, K: int) -> int:
    """Bytes a quantiser launch must move at least once: read X (BF16), write
    the codes and the scales.  The dynamic NVFP4 path reads X twice (the
    global amax comes before any code); the second read is not counted.  The
    static one (a given global scale) reads X once and writes no scale."""
    if kind == "quant_fp8":
        return M * K * 2 + M * K + M * (K // 128) * 4
    if kind == "quant_fp8_expand":  # every expanded row reads its token row
        return M * K * 2 + M * K + M * (K // 128) * 4 + M * 4
    if kind == "quant_nvfp4_static":
        return M * K * 2 + M * K // 2 + M * (K // 16)
    return M * K * 2 + M * K // 2 + M * (K // 16) + 4


def time_modes(torch, call, steps: int, timing: str, single: bool = False):
    """(ms per step in the `timing` mode, ms per step in the other mode, or
    None with `single`)."""
    ms, _ = time_launches(torch, call, steps, timing == "graph")
    other = None if single else time_launches(torch, call, steps, timing != "graph")[0]
    return ms, other


FLUSH_BYTES = 512 << 20  # twice the 256 MB last-level cache


def cold_cache_timing(torch, call, launches: int):
    """Per-launch times with cold caches: before each launch a 512 MB buffer
    is read (a sum), which leaves L2 and the last-level cache holding other,
    clean lines -- an overwrite instead would leave dirty lines whose
    write-back lands in the timed launch -- then HIP events on the current
    stream bracket that one launch.  Returns (median ms cold, median ms of
    the same loop without the flush).  Each launch stands alone here, so even
    the warm figure includes the launch ramp that the back-to-back timing of
    `time_launches` spreads over many launches."""
    stream = torch.cuda.current_stream()
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(launches)]

    def median_ms(do_flush: bool) -> float:
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            if do_flush:
                flush.sum()
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in ev)

    cold = median_ms(True)
    warm = median_ms(False)
    del flush
    return cold, warm


def cold_cache_entry(torch, call, args, work: float, unit: str, scale: float):
    """The `cold_cache` object of a result line: `work` units per launch,
    reported as work / seconds * scale in `unit` (None when switched off)."""
    if args.cold_launches <= 0 or args.single_timing:
        return None
    print("[bench] cold-cache launches", file=sys.stderr, flush=True)
    cold, warm = cold_cache_timing(torch, call, args.cold_launches)
    return {"launches": args.cold_launches, "flush_bytes": FLUSH_BYTES,
            "ms_median": round(cold, 5), "value": round(work / (cold * 1e-3) * scale, 2),
            "warm_ms_median": round(warm, 5),
            "warm_value": round(work / (warm * 1e-3) * scale, 2), "unit": unit}


def time_launches(torch, call, steps: int, graph: bool = False):
    """Time `steps` calls of `call` (each one kernel launch) on the current
    stream, with HIP events recorded on that stream around the timed region
    (or around one graph replay of `steps` captured launches).  Returns
    (ms_per_step, ms_per_launch), both the region over `steps`: the average
    launch duration in steady state.  Launches are not bracketed one by one:
    an event between two launches is a barrier, which for the short kernels
    adds the launch ramp to every duration and for the grouped GEMMs removes
    the overlap of one launch's tail with the next launch's head."""
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(steps):
                call()
        g.replay()  # untimed first replay
        torch.cuda.synchronize()
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / steps
        return ms, ms
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    return ms, ms


def bench_quant(args, torch):
    import fp4_grouped_gemm_amd as fgg
    w = WORKLOADS[args.workload]
    kind, M, K = w["kind"], w["M"], w["K"]
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    rng = np.random.default_rng(0)
    rows_np = None
    if kind == "quant_fp8_expand":
        from workloads import decode_routing, moe_expand
        T = w["T"]
        routing = decode_routing(T, w["top_k"], w["G"], rng).reshape(T, w["top_k"])
        rows_np, _ = moe_expand(routing, w["G"])
        assert rows_np.size == M
        X = torch.from_numpy(rng.standard_normal((T, K), dtype=np.float32)).to(torch.bfloat16)
        rows_d = torch.from_numpy(rows_np).cuda()
    else:
        X = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(torch.bfloat16)
    Xd = X.cuda()
    g_static = float(X[:64].float().abs().max()) / 2688.0  # a calibration on the first rows
    if kind == "quant_fp8":
        run = lambda: fgg.quantize_fp8_1x128(Xd)
    elif kind == "quant_fp8_expand":
        run = lambda: fgg.quantize_fp8_1x128(Xd, rows=rows_d)
    elif kind == "quant_nvfp4_static":
        run = lambda: fgg.quantize_nvfp4(Xd, global_scale=g_static)
    else:
        run = lambda: fgg.quantize_nvfp4(Xd)
    for _ in range(args.warmup):
        out = run()
    ms, ms_other = time_modes(torch, run, args.steps, args.timing, args.single_timing)
    ms_launch = ms
    cold = cold_cache_entry(torch, run, args, quant_bytes(kind, M, K), "GB/s", 1e-9)
    out = run()
    torch.cuda.synchronize()
    nbytes = quant_bytes(kind, M, K)
    gbps = nbytes / (ms * 1e-3) / 1e9
    gbps_launch = nbytes / (ms_launch * 1e-3) / 1e9
    res = {
        "metric": QUANT_METRIC, "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded NumPy N(0,1), BF16, resident in HBM)",
        "config": {"workload": args.workload, "desc": w["desc"], "M": M, "K": K,
                   "timing": TIMING[args.timing], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbps_launch, 1), "peak": HBM_PEAK,
                     "unit": "GB/s", "frac": round(gbps_launch / HBM_PEAK, 4),
                     "traffic": measured_traffic(args.workload, kernel_source_hash(args.workload)),
                     "algorithmic_bytes": nbytes, "us_per_launch": round(ms_launch * 1e3, 2)},
        "kernel_source_sha": kernel_source_hash(args.workload),
    }
    res["ms_per_step_" + OTHER[args.timing]] = (None if ms_other is None
                                                   else round(ms_other, 5))
    res["cold_cache"] = cold
    if not args.no_cpu_baseline:
        import oracle.quant as oq
        from threadpoolctl import threadpool_info
        print("[bench] cpu baseline (oracle on a row sample)", file=sys.stderr, flush=True)
        Xf = X.float().numpy()
        if rows_np is not None:
            Xf = Xf[rows_np]  # every row maps to a token (no padding rows here)
        Q = [t.cpu().numpy() for t in out]
        done, ok = 0, True
        t0 = time.perf_counter()
        for r0 in range(0, M, 64):
            rows = Xf[r0:r0 + 64]
            if kind in ("quant_fp8", "quant_fp8_expand"):
                q, sc = oq.quantize_fp8_1x128(rows)
                ok &= bool(np.array_equal(q, Q[0][r0:r0 + 64]) and
                           np.array_equal(sc, Q[1][r0:r0 + 64]))
            else:
                q, sc, _ = oq.quantize_nvfp4(rows, np.float32(Q[2][0]))
                ok &= bool(np.array_equal(q, Q[0][r0:r0 + 64]) and np.array_equal(sc, Q[1][r0:r0 + 64]))
            done += rows.shape[0]
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cores, blas = host_threads()
        res["cpu_baseline"] = {
            "value": round(quant_bytes(kind, done, K) / dt / 1e9, 4), "unit": "GB/s",
            "cores": cores, "blas_threads": blas, "kind": "oracle",
            "sample": f"{done} of {M} rows of the same workload (NumPy float32 decisions, "
                      f"table-search encoders), {dt:.1f} s; the global scale from the GPU run"}
        res["parity_sample"] = {"rows": done, "ok": ok, "bitwise": True}
    print(json.dumps(res), flush=True)


def w4a16_bytes(p: dict) -> int:
    """Bytes a W4A16 launch must move at least once: the weights and scales
    of every expert that has a row, the activations, the routing, C."""
    M, N, K = p["M"], p["N"], p["K"]
    ids = p["m_indices"]
    used = int(np.unique(ids[(ids >= 0) & (ids < p["G"])]).size)
    return used * N * (K // 2 + K // 16) + M * K * 2 + M * 4 + M * N * 2


def bench_w4a16(args, torch):
    """Grouped W4A16 decode: HBM-bound on the weights; GB/s and µs."""
    import fp4_grouped_gemm_amd as fgg
    import oracle
    from fp4_grouped_gemm_amd.util import c_to_f64
    from workloads import make

    if not os.path.exists(fgg.library_path()):
        from fp4_grouped_gemm_amd.build import build
        build()
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    p = make(args.workload)
    A = torch.from_numpy(p["A_bits"].view(np.int16)).cuda().view(torch.bfloat16)
    B, sb = torch.from_numpy(p["B"]).cuda(), torch.from_numpy(p["b_scale"]).cuda()
    ids = torch.from_numpy(p["m_indices"]).cuda()
    C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")

    def call():
        fgg.grouped_w4a16_gemm(A, B, sb, ids, p["b_global"], out=C)

    for _ in range(args.warmup):
        call()
    ms, ms_other = time_modes(torch, call, args.steps, args.timing, args.single_timing)
    ms_launch = ms
    nbytes = w4a16_bytes(p)
    cold = cold_cache_entry(torch, call, args, nbytes, "GB/s", 1e-9)
    gbps = nbytes / (ms * 1e-3) / 1e9
    gbps_launch = nbytes / (ms_launch * 1e-3) / 1e9
    res = {
        "metric": "GB/s (algorithmic bytes / time) and % of HBM peak, grouped W4A16 decode",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 x nvfp4_e2m1",
        "data": "synthetic (seeded NumPy; weights quantised on the host, resident in HBM)",
        "config": {"workload": args.workload, "desc": WORKLOADS[args.workload]["desc"],
                   "M": p["M"], "N": p["N"], "K": p["K"], "G": p["G"],
                   "timing": TIMING[args.timing], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbps_launch, 1), "peak": HBM_PEAK,
                     "unit": "GB/s", "frac": round(gbps_launch / HBM_PEAK, 4),
                     "traffic": measured_traffic(args.workload, kernel_source_hash(args.workload)),
                     "algorithmic_bytes": nbytes, "us_per_launch": round(ms_launch * 1e3, 2)},
        "kernel_source_sha": kernel_source_hash(args.workload),
    }
    res["ms_per_step_" + OTHER[args.timing]] = (None if ms_other is None
                                                   else round(ms_other, 5))
    res["cold_cache"] = cold
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        print("[bench] cpu baseline (oracle, every row)", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        ref = oracle.grouped_w4a16_gemm(p["A"], p["B"], p["b_scale"], p["m_indices"],
                                        p["b_global"])
        dt = time.perf_counter() - t0
        ok = oracle.check_tolerance(c_to_f64(C), ref, p["m_indices"])["ok"]
        cores, blas = host_threads()
        res["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": cores, "blas_threads": blas, "kind": "oracle",
                               "sample": f"the whole workload ({p['M']} rows), float64 "
                                         f"NumPy/BLAS, {dt:.1f} s"}
        res["parity_sample"] = {"rows": p["M"], "ok": bool(ok)}
    print(json.dumps(res), flush=True)


def bench_problems(args, torch):
    """A batch of dense NVFP4 (fp4_gemm_problems) or block-scaled FP8
    (fp8_gemm_problems) problems of different shapes, one launch per step."""
    import fp4_grouped_gemm_amd as fgg
    import oracle
    from fp4_grouped_gemm_amd.util import c_to_f64, to_device as to_dev
    from workloads import make

    if not os.path.exists(fgg.library_path()):
        from fp4_grouped_gemm_amd.build import build
        build()
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    p = make(args.workload)
    probs = p["problems"]
    ds = [to_dev(q) for q in probs]
    outs = [torch.empty((q["M"], q["N"]), dtype=torch.bfloat16, device="cuda") for q in probs]
    fp8 = p["kind"] == "fp8_problems"
    if fp8:
        batch = [(d["A"], d["B"][0], d["a_scale"], d["b_scale"][0]) for d in ds]
        run_batch = fgg.fp8_gemm_problems
    else:
        batch = [(d["A"], d["B"], d["a_scale"], d["b_scale"], q["alpha"])
                 for d, q in zip(ds, probs)]
        run_batch = fgg.fp4_gemm_problems
    kw = {} if args.tile is None else {"tile_id": args.tile}
    for _ in range(args.warmup):
        run_batch(batch, outs, **kw)
    ms, ms_other = time_modes(torch, lambda: run_batch(batch, outs, **kw),
                              args.steps, args.timing, args.single_timing)
    ms_launch = ms
    flops = sum(2.0 * q["M"] * q["N"] * q["K"] for q in probs)
    cold = cold_cache_entry(torch, lambda: run_batch(batch, outs, **kw), args, flops,
                            "TFLOPS", 1e-12)
    tflops = flops / (ms * 1e-3) / 1e12
    tflops_launch = flops / (ms_launch * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if fp8 else "nvfp4_e2m1",
        "data": "synthetic (seeded NumPy; quantised on the host, resident in HBM)",
        "config": {"workload": args.workload, "desc": WORKLOADS[args.workload]["desc"],
                   "problems": [[q["M"], q["N"], q["K"]] for q in probs],
                   "tile": args.tile, "timing": TIMING[args.timing],
                   "parallelism": "single GPU"},
        "kernel_source_sha": kernel_source_hash(args.workload),
    }
    peak = "fp8" if fp8 else "fp4"
    out["roofline"] = {"bound": "mfma", "achieved": round(tflops_launch, 2), "peak": PEAK[peak],
                       "peak_dtype": peak, "unit": "TFLOP/s",
                       "frac": round(tflops_launch / PEAK[peak], 4),
                       "traffic": measured_traffic(args.workload, kernel_source_hash(args.workload)),
                       "mfma_dtype": peak if fp8 else "fp16",
                       "us_per_launch": round(ms_launch * 1e3, 2)}
    if not fp8:
        out["roofline"]["frac_of_fp16_peak"] = round(tflops_launch / PEAK["fp16"], 4)
    out["ms_per_step_" + OTHER[args.timing]] = (None if ms_other is None
                                                   else round(ms_other, 5))
    out["cold_cache"] = cold
    if not args.no_cpu_baseline:
        # the oracle on the first rows of every problem, in turn, until the budget
        print("[bench] cpu baseline (oracle on a row sample)", file=sys.stderr, flush=True)
        from threadpoolctl import threadpool_info
        t0, fl, ok, nrows = time.perf_counter(), 0.0, True, 0
        for c0 in range(0, max(q["M"] for q in probs), 128):
            for q, C in zip(probs, outs):
                rows = np.arange(c0, min(c0 + 128, q["M"]))
                if rows.size == 0:
                    continue
                if fp8:
                    r = oracle.grouped_fp8_gemm(q["A"], q["B"], q["a_scale"], q["b_scale"],
                                                q["m_indices"], rows=rows)
                else:
                    r = oracle.fp4_gemm(q["A"], q["B"], q["a_scale"], q["b_scale"], q["alpha"],
                                        rows=rows)
                ok &= oracle.check_tolerance(c_to_f64(C)[rows], r)["ok"]
                fl += 2.0 * rows.size * q["N"] * q["K"]
                nrows += rows.size
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        cores, blas = host_threads()
        out["cpu_baseline"] = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOPS",
                               "cores": cores, "blas_threads": blas, "kind": "oracle",
                               "sample": f"first {nrows} rows over the 8 problems x all columns, "
                                         f"float64 NumPy/BLAS, {dt:.1f} s"}
        out["parity_sample"] = {"rows": nrows, "ok": bool(ok)}
    print(json.dumps(out), flush=True)


def tune_report(args, torch):
    """Heuristic top-1 against the best of the ranker's top-k on every GEMM
    workload (the measurement the flashinfer#3948 page reports: the top-1
    pick's loss and the geomean loss of tuning only the top candidates)."""
    import fp4_grouped_gemm_amd as fgg
    from fp4_grouped_gemm_amd.util import to_device as to_dev
    from workloads import make

    if not os.path.exists(fgg.library_path()):
        from fp4_grouped_gemm_amd.build import build
        build()
    rows, ratios, lit_ratios = [], [], []
    for name, w in WORKLOADS.items():
        if w["kind"] not in ("fp8", "fp4"):
            continue  # the quantisers, W4A16 and the problem batch have no tile choice to tune
        print(f"[bench] tune {name}", file=sys.stderr, flush=True)
        p = make(name)
        d = to_dev(p)
        big = p["M"] * p["N"] * p["K"] > 1 << 34
        kw = dict(top_k=args.top_k, reps=10 if big else 100)
        if w.get("run_align"):
            kw["run_align"] = w["run_align"]
        fgg.tune_clear()
        if p["kind"] == "fp8":
            _, rep = fgg.grouped_fp8_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"],
                                               d["m_indices"], **kw)
        elif p.get("m_indices") is None:
            _, rep = fgg.fp4_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"], p["alpha"], **kw)
        else:
            _, rep = fgg.grouped_fp4_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"],
                                               d["m_indices"], p["alpha"], **kw)
        heur, best = rep["ms"][0], rep["ms"][rep["best"]]
        ratios.append(heur / best)
        rows.append(dict(workload=name, candidates=rep["tile_id"],
                         us=[round(1e3 * t, 2) for t in rep["ms"]], heuristic=rep["tile_id"][0],
                         best=rep["chosen"], heuristic_loss=round(heur / best - 1.0, 4)))
        # the page's literal score form, ranked on the same shape: its top-1's
        # time among the timed candidates (all configs when top_k covers them)
        lit = fgg.rank_tiles(fgg.FP8 if p["kind"] == "fp8" else fgg.FP4, p["M"], p["N"], p["K"],
                             p["G"], num_cus=fgg.device_info()["num_cus"],
                             run_align=w.get("run_align", 0), variant=fgg.SCORE_LITERAL)[0]["id"]
        if lit in rep["tile_id"]:
            t_lit = rep["ms"][rep["tile_id"].index(lit)]
            lit_ratios.append(t_lit / best)
            rows[-1].update(literal=lit, literal_loss=round(t_lit / best - 1.0, 4))
        align = w.get("run_align", 0)
        if align:
            # the ranker's pick under the workload's run-alignment promise
            top = fgg.rank_tiles(fgg.FP8 if p["kind"] == "fp8" else fgg.FP4, p["M"], p["N"],
                                 p["K"], p["G"], num_cus=fgg.device_info()["num_cus"],
                                 run_align=align)[0]["id"]
            if top in rep["tile_id"]:
                t = rep["ms"][rep["tile_id"].index(top)]
                rows[-1].update(run_align=align, heuristic_aligned=top,
                                heuristic_aligned_loss=round(t / best - 1.0, 4))
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del d, p
        torch.cuda.empty_cache()
    geo = float(np.exp(np.mean(np.log(ratios))))
    res = {"metric": "bounded autotune: heuristic top-1 time / best-of-top-k time",
           "top_k": args.top_k, "workloads": rows,
           "geomean_heuristic_over_best": round(geo, 4),
           "geomean_loss": round(geo - 1.0, 4)}
    if len(lit_ratios) == len(ratios):
        geo_l = float(np.exp(np.mean(np.log(lit_ratios))))
        res.update(geomean_literal_over_best=round(geo_l, 4),
                   geomean_literal_loss=round(geo_l - 1.0, 4))
    print(json.dumps(res), flush=True)


def bench_gemm(args, torch, workload: str, cold_launches: int, cpu_seconds: float,
               primary: bool = True) -> dict:
    """One GEMM workload: warm-up, the timed region, the cold-cache figure
    (cold_launches > 0), the oracle baseline on a row sample (cpu_seconds >
    0); returns the result record.  The launch options of the command line
    (--tile, --run-split, --max-workgroups, --autotune) apply to the primary
    workload only."""
    import fp4_grouped_gemm_amd as fgg
    from fp4_grouped_gemm_amd.util import run, to_device as to_dev
    from workloads import make
    from workloads.gen import real_rows

    if not os.path.exists(fgg.library_path()):
        from fp4_grouped_gemm_amd.build import build
        build()
    print(f"[bench] generating {workload}", file=sys.stderr, flush=True)
    p = make(workload)
    d = to_dev(p)
    kind = WORKLOADS[workload]["kind"]
    M, N, K, G = p["M"], p["N"], p["K"], p["G"]
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tile = args.tile if primary else None
    kw = {} if tile is None else {"tile_id": tile}
    if primary and args.run_split and p.get("m_indices") is not None:
        kw["run_split"] = args.run_split
    if primary and args.max_workgroups:
        kw["max_workgroups"] = args.max_workgroups
    # the workload's routing promise (its runs start on multiples of this)
    run_align = WORKLOADS[workload].get("run_align", 0) if not args.no_run_align else 0
    if run_align and p.get("m_indices") is not None:
        kw["run_align"] = run_align
    tuned = None
    if primary and args.autotune and tile is None:
        # the library's bounded autotune, once, untimed: later calls of this
        # shape launch the config it recorded
        print("[bench] autotune", file=sys.stderr, flush=True)
        fgg.tune_clear()
        tk = dict(top_k=args.top_k, reps=5)
        if kind == "fp8":
            _, tuned = fgg.grouped_fp8_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"],
                                                 d["m_indices"], out=C, **tk)
        elif p.get("m_indices") is None:
            _, tuned = fgg.fp4_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"], p["alpha"],
                                         out=C, **tk)
        else:
            _, tuned = fgg.grouped_fp4_gemm_tune(d["A"], d["B"], d["a_scale"], d["b_scale"],
                                                 d["m_indices"], p["alpha"], out=C, **tk)
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run(p, d, out=C, **kw)
    ms, ms_other = time_modes(torch, lambda: run(p, d, out=C, **kw), args.steps, args.timing,
                             args.single_timing)
    ms_launch = ms
    rr = real_rows(p)
    flops = 2.0 * rr * N * K
    cold = (cold_cache_entry(torch, lambda: run(p, d, out=C, **kw), args, flops, "TFLOPS", 1e-12)
            if cold_launches > 0 else None)
    tflops = flops / (ms * 1e-3) / 1e12
    tflops_launch = flops / (ms_launch * 1e-3) / 1e12
    # the MFMA the kernel issues (the exact NVFP4 path runs FP16 MFMAs), and
    # the peak the fraction is priced against: the input format's own dense
    # peak (FP8 for FP8, FP4 for NVFP4), with the FP16 fraction kept beside
    # it for NVFP4 -- the exact path cannot exceed 2.5 / 10.1 of the FP4 peak
    mma = "fp8" if kind == "fp8" else "fp16"
    peak_kind = "fp8" if kind == "fp8" else "fp4"
    src = kernel_source_hash(workload)
    traffic = measured_traffic(workload, src)
    tiles = fgg.rank_tiles(fgg.FP8 if kind == "fp8" else fgg.FP4, M, N, K, G,
                           num_cus=fgg.device_info()["num_cus"], run_align=kw.get("run_align", 0))
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if kind == "fp8" else "nvfp4_e2m1",
        "data": "synthetic (seeded NumPy; quantised on the host, resident in HBM)",
        "config": {"workload": workload, "desc": WORKLOADS[workload]["desc"],
                   "M": M, "N": N, "K": K, "G": G, "real_rows": rr,
                   "tile": (tile if tile is not None
                            else tuned["chosen"] if tuned else tiles[0]["id"]),
                   "tile_choice": ("given" if tile is not None
                                   else "bounded autotune" if tuned else "ranker"),
                   "run_split": kw.get("run_split", 0),
                   "max_workgroups": kw.get("max_workgroups", 0),
                   "run_align": kw.get("run_align", 0),
                   "timing": TIMING[args.timing], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops_launch, 2),
                     "peak": PEAK[peak_kind], "peak_dtype": peak_kind,
                     "unit": "TFLOP/s", "frac": round(tflops_launch / PEAK[peak_kind], 4),
                     "traffic": traffic, "mfma_dtype": mma,
                     "algorithmic_bytes": algorithmic_bytes(p),
                     "hbm_gbps_algorithmic": round(algorithmic_bytes(p) / (ms_launch * 1e-3) / 1e9, 1),
                     "us_per_launch": round(ms_launch * 1e3, 2)},
        "kernel_source_sha": src,
    }
    out["ms_per_step_" + OTHER[args.timing]] = (None if ms_other is None
                                                   else round(ms_other, 5))
    out["cold_cache"] = cold
    if kind == "fp4":
        out["roofline"]["frac_of_fp16_peak"] = round(tflops_launch / PEAK["fp16"], 4)
    if cpu_seconds > 0:
        print(f"[bench] cpu baseline (oracle on a row sample of {workload})", file=sys.stderr,
              flush=True)
        base, parity = cpu_baseline(p, C, cpu_seconds)
        out["cpu_baseline"] = base
        out["parity_sample"] = parity
    del d, C
    torch.cuda.empty_cache()
    return out


def tput_sweep(args, torch):
    """Per-CU throughput of every tile config on problems that every config
    tiles into whole waves of the device (so the ranker's other terms are
    1), relative to the best config: the measurement behind the ranker's
    `throughput` constants."""
    import fp4_grouped_gemm_amd as fgg
    from fp4_grouped_gemm_amd.util import run, to_device as to_dev
    from workloads import fp8_problem, nvfp4_problem
    rng = np.random.default_rng(0)
    out = {"metric": "tile config throughput, relative to the best config", "kinds": {}}
    for kind, name in ((fgg.FP8, "fp8"), (fgg.FP4, "fp4")):
        print(f"[bench] tput sweep {name}", file=sys.stderr, flush=True)
        if kind == fgg.FP8:
            # 8192 x 8192 x 7168, one expert: 1024 / 2048 / 2048 / 4096 tiles
            p = fp8_problem(np.zeros(8192, np.int32), 8192, 7168, 1, rng)
        else:
            p = nvfp4_problem(None, 8192, 8192, 4096, 1, rng)
        d = to_dev(p)
        C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
        flops = 2.0 * p["M"] * p["N"] * p["K"]
        tiles = fgg.rank_tiles(kind, p["M"], p["N"], p["K"], p["G"],
                               num_cus=fgg.device_info()["num_cus"])
        res = {}
        for t in sorted(tiles, key=lambda t: t["id"]):
            call = lambda: run(p, d, out=C, tile_id=t["id"])  # noqa: E731
            for _ in range(3):
                call()
            ms = min(time_launches(torch, call, 10, True)[0] for _ in range(3))
            res[t["id"]] = dict(block_m=t["block_m"], block_n=t["block_n"], waves=t["waves"],
                                wg_per_cu=t["wg_per_cu"], us=round(ms * 1e3, 1),
                                tflops=round(flops / (ms * 1e-3) / 1e12, 1),
                                tput_constant=round(t["tput"], 3))
        best = max(r["tflops"] for r in res.values())
        for r in res.values():
            r["tput_measured"] = round(r["tflops"] / best, 3)
        out["kinds"][name] = dict(M=p["M"], N=p["N"], K=p["K"], tiles=res)
        del d, C, p
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def round_sweep(args, torch):
    """Launch time against the number of tile rounds (tiles / workgroup
    slots) on dense problems whose column count grows one round in eight at
    a time: what a partly filled last round of tiles costs, for the ranker's
    round term.  256x256 tiles, M = 2048 (8 row windows), N = 256 nt."""
    import fp4_grouped_gemm_amd as fgg
    from fp4_grouped_gemm_amd.util import run, to_device as to_dev
    from workloads import fp8_problem, nvfp4_problem
    cus = fgg.device_info()["num_cus"]
    out = {"metric": "launch time against tile rounds, 256x256 tiles", "num_cus": cus,
           "kinds": {}}
    for kind, name, K in ((fgg.FP8, "fp8", 7168), (fgg.FP4, "fp4", 4608)):
        rows = []
        for nt in range(cus // 8, 2 * cus // 8 + 1, cus // 64):
            rng = np.random.default_rng(nt)
            N = 256 * nt
            print(f"[bench] round sweep {name} N={N}", file=sys.stderr, flush=True)
            if kind == fgg.FP8:
                p = fp8_problem(np.zeros(2048, np.int32), N, K, 1, rng)
            else:
                p = nvfp4_problem(None, 2048, N, K, 1, rng)
            d = to_dev(p)
            C = torch.empty((p["M"], p["N"]), dtype=torch.bfloat16, device="cuda")
            call = lambda: run(p, d, out=C, tile_id=0)  # noqa: E731
            for _ in range(3):
                call()
            ms = min(time_launches(torch, call, 10, True)[0] for _ in range(3))
            rows.append(dict(N=N, tiles=8 * nt, rounds=8 * nt / cus, us=round(ms * 1e3, 1)))
            del d, C, p
            torch.cuda.empty_cache()
        out["kinds"][name] = dict(M=2048, K=K, rows=rows)
    print(json.dumps(out), flush=True)


def routing_sweep(args, torch):
    """Grouped FP8 launch time of one 8192 x 4096 x 7168 problem under
    different row routings, per tile config: what windows holding an expert
    boundary cost.  Dense (one expert), runs of 2048/1024/256 rows aligned
    to the 256-row windows, and two-expert runs of 128, 64 and 32 rows
    alternating (every 256-row window then takes two passes, each filling
    half of the window's rows, spread evenly (128) or not (64, 32) over the
    wave rows), and c2's shape of boundary: 8 runs of 1024 shifted by 100
    rows, so 7 of the 32 windows hold a boundary."""
    import fp4_grouped_gemm_amd as fgg
    from fp4_grouped_gemm_amd.util import to_device as to_dev
    from workloads import fp8_problem
    M, N, K = 8192, 4096, 7168
    rows = np.arange(M)
    routings = {
        "dense": np.zeros(M, np.int32),
        "runs1024_aligned": (rows // 1024).astype(np.int32),
        "alt256": ((rows // 256) % 2).astype(np.int32),
        "alt128": ((rows // 128) % 2).astype(np.int32),
        "alt64": ((rows // 64) % 2).astype(np.int32),
        "alt32": ((rows // 32) % 2).astype(np.int32),
        "runs1024_shift100": np.minimum((rows + 100) // 1024, 7).astype(np.int32),
    }
    p = fp8_problem(np.zeros(M, np.int32), N, K, 8, np.random.default_rng(0))
    d = to_dev(p)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    out = {"metric": "grouped FP8 launch time against the row routing", "M": M, "N": N, "K": K,
           "tiles": {}}
    for tile in range(fgg.num_tiles(fgg.FP8)):
        row = {}
        for name, ids in routings.items():
            print(f"[bench] routing sweep tile {tile} {name}", file=sys.stderr, flush=True)
            mi = torch.from_numpy(ids).cuda()
            call = lambda: fgg.grouped_fp8_gemm(d["A"], d["B"], d["a_scale"], d["b_scale"], mi,  # noqa: E731
                                                out=C, tile_id=tile)
            for _ in range(3):
                call()
            ms = min(time_launches(torch, call, 10, True)[0] for _ in range(3))
            row[name] = round(ms * 1e3, 1)
        out["tiles"][str(tile)] = row
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2_moe_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--tile", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timing", choices=("graph", "stream"), default="graph",
                    help="graph (default): capture the K timed launches in one HIP graph and "
                         "time one replay, as a captured MoE layer runs them; stream: time K "
                         "launches issued one by one on the stream.  The line reports the "
                         "other mode's ms per step too.")
    ap.add_argument("--graph", dest="timing", action="store_const", const="graph",
                    help="same as --timing graph")
    ap.add_argument("--stream", dest="timing", action="store_const", const="stream",
                    help="same as --timing stream")
    ap.add_argument("--cold-launches", type=int, default=50,
                    help="also time this many single launches with the caches flushed before "
                         "each (a 512 MB read) and report their median as cold_cache (0: skip)")
    ap.add_argument("--no-run-align", action="store_true",
                    help="do not pass the workload's run-alignment promise to the ranker")
    ap.add_argument("--single-timing", action="store_true",
                    help="time only the chosen mode, with no cold-cache launches (profiling "
                         "runs: every traced dispatch then comes from the mode the line reports)")
    ap.add_argument("--tune-report", action="store_true",
                    help="bounded autotune of every GEMM workload: time the ranker's top-k tile "
                         "configs (the library's *_tune calls), report heuristic top-1 against "
                         "the best of the k, and the geomean loss; one JSON line")
    ap.add_argument("--top-k", type=int, default=4)
    ap.add_argument("--round-sweep", action="store_true",
                    help="time dense 256x256-tiled problems from one to two rounds of tiles in "
                         "eighths (what a partly filled last round costs); one JSON line")
    ap.add_argument("--routing-sweep", action="store_true",
                    help="time grouped FP8 on one shape under routings with and without expert "
                         "boundaries inside the row windows, per tile config; one JSON line")
    ap.add_argument("--tput-sweep", action="store_true",
                    help="time every tile config on problems that fill whole waves for all of "
                         "them and print each config's throughput relative to the best (the "
                         "ranker's throughput constants); one JSON line")
    ap.add_argument("--autotune", action="store_true",
                    help="GEMM workloads: run the library's bounded autotune of the ranker's "
                         "top-k configs once (untimed) and time the config it records")
    ap.add_argument("--max-workgroups", type=int, default=0,
                    help="fgg_options.max_workgroups (0: one workgroup per tile)")
    ap.add_argument("--run-split", type=int, default=0,
                    help="fgg_options.run_split (0 automatic, -1 never, 1 always)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--no-nvfp4", action="store_true",
                    help="default workload only: skip the NVFP4 sub-records (c4, c5)")
    ap.add_argument("--nvfp4-cpu-seconds", type=float, default=8.0,
                    help="CPU time budget of each NVFP4 sub-record's oracle sample")
    ap.add_argument("--rocprof-summary", default=None, metavar="DIR",
                    help="summarise rocprofv3 CSV output in DIR (see rocprof_summary) and exit")
    ap.add_argument("--kernel", default="fp8_grouped_kernel",
                    help="kernel-name substring for --rocprof-summary")
    ap.add_argument("--command", default="", help="profiling command recorded by --rocprof-summary")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="instead of the GEMM, time a plain 1 GiB device-to-device copy; its "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE per dispatch calibrate the HBM "
                         "traffic counters (1 GiB read + 1 GiB written per launch)")
    args = ap.parse_args()
    if args.rocprof_summary:
        print(rocprof_summary(args.rocprof_summary, args.workload, args.kernel, args.command))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                          "gbps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
        return

    if args.tune_report:
        tune_report(args, torch)
        return

    if args.tput_sweep:
        tput_sweep(args, torch)
        return

    if args.round_sweep:
        round_sweep(args, torch)
        return

    if args.routing_sweep:
        routing_sweep(args, torch)
        return

    if WORKLOADS[args.workload]["kind"] == "w4a16":
        bench_w4a16(args, torch)
        return

    if WORKLOADS[args.workload]["kind"] in ("fp4_problems", "fp8_problems"):
        bench_problems(args, torch)
        return

    if WORKLOADS[args.workload]["kind"].startswith("quant"):
        if not os.path.exists(os.path.join(ROOT, "fp4_grouped_gemm_amd", "libfgg.so")):
            from fp4_grouped_gemm_amd.build import build
            build()
        bench_quant(args, torch)
        return

    out = bench_gemm(args, torch, args.workload, args.cold_launches,
                     0.0 if args.no_cpu_baseline else args.cpu_seconds)
    if args.workload == "c2_moe_fp8" and not args.no_nvfp4:
        # the NVFP4 half of the metric: the dense (flashinfer#3948 page's
        # mm_fp4 review shape) and grouped W4A4 (onnxruntime#29824 page)
        # workloads, each timed the same way, as sub-records of the one line
        out["nvfp4"] = {}
        for w in ("c4_dense_nvfp4", "c5_moe_nvfp4"):
            sub = bench_gemm(args, torch, w, 0,
                             0.0 if args.no_cpu_baseline else args.nvfp4_cpu_seconds,
                             primary=False)
            for k in ("metric", "n_gpus", "higher_is_better", "scaling", "vs_baseline", "data"):
                sub.pop(k, None)
            out["nvfp4"][w] = sub
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
