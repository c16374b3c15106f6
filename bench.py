"""Throughput of the LLM.int8() linear layer on one MI355X.

A step is one full forward call (outlier scan, activation quantization, int8
GEMM with fused dequantization and fp16 outlier product) over one batch of the
prefill workload: X fp16 [2048, 4096] with 6 injected outlier feature columns,
W [11008, 4096] stored as int8 + per-row fp32 scale, threshold 6.0. The weight
is quantized once before timing (load time). Inputs are synthetic and seeded
and already resident in HBM when the timed region starts.

Prints one JSON line. Besides the headline TOPS it carries the roofline of the
dominant kernel (the int8 GEMM, timed with HIP events on the launch stream),
the decode-shaped workload (T=8, K=N=4096) as GB/s against HBM bandwidth, the
input gradient through the frozen layer at the prefill shape (fp16 TFLOP/s
against the fp16 MFMA peak), the blockwise 8-bit codec (GB/s against HBM
bandwidth) and the CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LLM.int8() linear TOPS + % int8 MFMA peak (T=2048) / % HBM BW (T<=8)"
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 MFMA, tera-ops/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "kb_gemm_prefill_counters.txt")
PROFILE_BWD_COUNTERS = os.path.join(ROOT, "profiles", "kg_backward_prefill_counters.txt")
BWD_SOURCES = ("bwd.hip", "gemm_common.h", "device_util.h", "internal.h", "ranges.h")
PROFILE_DECODE_COUNTERS = os.path.join(ROOT, "profiles", "kd_gemv_decode_counters.txt")
DECODE_SOURCES = ("gemv.hip", "device_util.h", "internal.h", "ranges.h")
PROFILE_NEXT_COUNTERS = os.path.join(ROOT, "profiles", "bf16_codec_nf4_counters.txt")
NEXT_SOURCES = ("gemm.hip", "gemm_common.h", "blockwise.hip", "fourbit.hip", "device_util.h",
                "internal.h", "ranges.h")


def roofline(bound, kernel, achieved, peak, unit, traffic, **extra):
    """The roofline object of one kernel: achieved / peak, with the counter traffic."""
    return {"bound": bound, "kernel": kernel, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic, **extra}


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10,
                   help="untimed calls before timing; at least this many, and at least "
                        "--warmup-ms of back-to-back calls (the clock ramps up under load)")
    p.add_argument("--warmup-ms", type=float, default=30.0)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-backward", action="store_true", help="skip the input-gradient workload")
    p.add_argument("--no-codec", action="store_true", help="skip the blockwise codec workload")
    p.add_argument("--no-bf16", action="store_true", help="skip the bf16 + bias workload")
    p.add_argument("--no-fourbit", action="store_true", help="skip the 4-bit weight workload")
    p.add_argument("--no-probe", action="store_true", help="skip the matrix-core rate probe")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the tiny, large and outlier-sweep workloads")
    p.add_argument("--config-steps", type=int, default=20,
                   help="timed calls per tiny / large / sweep point")
    p.add_argument("--decode-copies", type=int, default=24,
                   help="distinct weight copies cycled in the decode timing (> last-level cache)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the measurement, run 5 plain device copies of MIB MiB (untimed), "
                        "a known-size reference for HBM byte counters")
    return p.parse_args()


def kernel_source_hash(files=None) -> str:
    h = hashlib.sha256()
    for f in files or ("gemm.hip", "gemm_common.h", "device_util.h", "internal.h", "ranges.h"):
        with open(os.path.join(ROOT, "mixed_precision_int8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(path=None, files=None, key="hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when absent or taken on different kernel source."""
    path = path or PROFILE_COUNTERS
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash(files):
        return None
    m = re.search(key + r":\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def committed_mfma_activity():
    """(MFMA busy %, effective shader clock in GHz) of the prefill GEMM from the
    committed counter summary, or (None, None) when absent or stale."""
    if committed_traffic() is None:
        return None, None
    text = open(PROFILE_COUNTERS).read()
    busy = re.search(r"=\s*([0-9.]+)% MFMA busy", text)
    clock = re.search(r"=\s*([0-9.]+) GHz", text)
    return (float(busy.group(1)) if busy else None, float(clock.group(1)) if clock else None)


_PROBE = None


def _probe_lib():
    """libllmint8_probe.so: measurement helpers built beside the product library."""
    import ctypes
    global _PROBE
    if _PROBE is None:
        lib = ctypes.CDLL(os.path.join(ROOT, "mixed_precision_int8_amd", "libllmint8_probe.so"))
        vp, i = ctypes.c_void_p, ctypes.c_int
        for name, args in (("llmint8_bench_probe_mfma_i8", [i, i, vp, vp]),
                           ("llmint8_bench_probe_mfma_i8_lds_random", [i, i, vp, vp]),
                           ("llmint8_bench_probe_stream", [vp, ctypes.c_size_t, vp, vp]),
                           ("llmint8_bench_probe_empty", [vp, vp])):
            getattr(lib, name).argtypes = args
            getattr(lib, name).restype = i
        _PROBE = lib
    return _PROBE


def _probe_check(st, name):
    if st != 0:
        raise RuntimeError(f"{name} failed ({st})")


def probe_mfma_i8(blocks, iters, out, stream):
    """The matrix-core rate probe: blocks x 4 wavefronts, each iters x 4
    v_mfma_i32_32x32x32_i8 from registers. Returns the int8 operation count."""
    import ctypes
    _probe_check(_probe_lib().llmint8_bench_probe_mfma_i8(int(blocks), int(iters), ctypes.c_void_p(out.data_ptr()),
                                                          ctypes.c_void_p(stream.cuda_stream)), "probe")
    return blocks * 4 * iters * 4 * 2 * 32 * 32 * 32


def probe_mfma_i8_lds_random(blocks, iters, out, stream):
    """The same MFMA, 8 wavefronts of 4 x 2 blocks with fragments re-read from LDS full
    of pseudo-random bytes every k-step. Returns the int8 operation count."""
    import ctypes
    _probe_check(_probe_lib().llmint8_bench_probe_mfma_i8_lds_random(
        int(blocks), int(iters), ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream)),
        "probe_lds_random")
    return blocks * 8 * iters * 4 * 8 * 2 * 32 * 32 * 32


def probe_stream(buf, n16, out, stream):
    import ctypes
    _probe_check(_probe_lib().llmint8_bench_probe_stream(ctypes.c_void_p(buf.data_ptr()), int(n16),
                                                         ctypes.c_void_p(out.data_ptr()),
                                                         ctypes.c_void_p(stream.cuda_stream)), "probe_stream")


def probe_empty(out, stream):
    import ctypes
    _probe_check(_probe_lib().llmint8_bench_probe_empty(ctypes.c_void_p(out.data_ptr()),
                                                        ctypes.c_void_p(stream.cuda_stream)), "probe_empty")


def graph_us_per_call(fn, n_calls, replays, stream):
    """fn(0) .. fn(n_calls - 1) captured once in a HIP graph and replayed: microseconds
    per call without the per-call host (Python) submission cost. The calls must
    launch kernels only (no memsets, no allocations)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (replays * n_calls) * 1e3
    del g
    return us


# targets of the whole call at >= 60% of the int8 peak (us), per workload
CALL_TARGET_US = {"large": 639.0, "sweep": 289.0}


def time_linear(m8, torch, Xd, Wq, sW, thr, Y, ws, steps, warmup, stream):
    """Whole calls between two events after a warm-up (at least 30 ms of calls), then
    per-kernel times from events recorded between the kernels of the same call."""
    import numpy as np
    w0 = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - w0) < 0.03:
        m8.llmint8_linear(Xd, Wq, sW, thr, Y=Y, workspace=ws)
        n += 1
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        m8.llmint8_linear(Xd, Wq, sW, thr, Y=Y, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for row in evs:          # a torch event exists once it has been recorded
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    nk = 0
    for row in evs:
        nk = m8.llmint8_linear_timed(Xd, Wq, sW, thr, Y, ws, row)
    torch.cuda.synchronize()
    per = [float(np.mean([row[i].elapsed_time(row[i + 1]) for row in evs])) for i in range(nk)]
    names = ["ka_scan", "ka_prepare", "kb_gemm"] if nk == 3 else ["kd_gemv"]
    return call_ms, dict(zip(names, per))


def graph_call_us(m8, torch, Xd, Wq, sW, thr, Y, ws, stream, calls=20, replays=10):
    """Per-call time of `calls` calls captured in one HIP graph, replayed."""
    return graph_us_per_call(lambda i: m8.llmint8_linear(Xd, Wq, sW, thr, Y=Y, workspace=ws),
                             calls, replays, stream)


def bench_configs(args, dev, stream):
    """Tiny (CFG1), large (CFG4) and the outlier-fraction sweep (CFG5: n_out x threshold):
    TOPS and % int8 peak of the whole call, per-kernel times, the GEMM's roofline, and
    (sweep) the accuracy of Y against the fp32 product at both thresholds."""
    import numpy as np
    import torch

    import mixed_precision_int8_amd as m8
    import workloads

    out = {}

    def one(name, w, W_dev, Wq, sW, X, thr, target_us=None, accuracy=False):
        T, K, N = X.shape[0], X.shape[1], Wq.shape[0]
        Xd = torch.from_numpy(X).to(dev)
        Y = torch.empty((T, N), dtype=torch.float16, device=dev)
        need = m8.llmint8_workspace_bytes(T, K, N)
        ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None
        dbg = m8.llmint8_linear_debug(Xd, Wq, sW, thr, workspace=ws, want_C=False)
        count = int(dbg["count"].cpu()[0])
        del dbg
        call_ms, kern = time_linear(m8, torch, Xd, Wq, sW, thr, Y, ws, args.config_steps,
                                    args.warmup, stream)
        ops = 2.0 * T * N * K
        tops = ops / (call_ms * 1e-3) / 1e12
        rec = {"T": T, "K": K, "N": N, "threshold": thr, "outliers": count,
               "us_per_call": round(call_ms * 1e3, 2), "TOPS": round(tops, 1),
               "pct_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
               "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()}}
        if "kb_gemm" in kern:
            g = ops / (kern["kb_gemm"] * 1e-3) / 1e12
            rec["gemm_tile"] = m8.llmint8_gemm_tile(T, N)
            rec["roofline"] = roofline("mfma", "kb_gemm", g, PEAK_INT8_TOPS, "TFLOP/s", None,
                                       unit_note="int8 tera-ops/s")
        else:
            rec["graph_us_per_call"] = round(graph_call_us(m8, torch, Xd, Wq, sW, thr, Y, ws, stream), 2)
        if target_us:
            rec["target_us"] = target_us
            rec["meets_target"] = bool(rec["us_per_call"] <= target_us)
        if accuracy:
            # accuracy context (not parity): Y against the fp32 product X . W^T
            Xf = Xd.float()
            torch.backends.cuda.matmul.allow_tf32 = False
            ref = Xf @ W_dev.float().t()
            rec["rel_err_vs_fp32_product"] = float((Y.float() - ref).abs().max() / ref.abs().max())
            del Xf, ref
        del Xd, Y, ws
        return rec

    w1 = workloads.CONFIGS["tiny"]
    W, X, _, _ = workloads.make(w1)
    Wdv = torch.from_numpy(W).to(dev)
    Wq, sW = m8.llmint8_quantize_weight(Wdv)
    out["tiny"] = one("tiny", w1, Wdv, Wq, sW, X, w1.threshold)
    out["tiny"]["workload"] = "tiny T=16 K=1024 N=1024, 4 outlier columns (latency-bound)"

    w4 = workloads.CONFIGS["large"]
    W, X, _, _ = workloads.make(w4)
    Wdv = torch.from_numpy(W).to(dev)
    Wq, sW = m8.llmint8_quantize_weight(Wdv)
    del W
    out["large"] = one("large", w4, Wdv, Wq, sW, X, w4.threshold, CALL_TARGET_US["large"])
    out["large"]["workload"] = "large T=4096 K=8192 N=28672, 25 outlier columns, 41 rows zeroed"
    del Wdv, Wq, sW

    w5 = workloads.CONFIGS["sweep"]
    W = workloads.make_weight(workloads.rng_for(w5.seed, 0), w5.N, w5.K, w5.sigma)
    Wdv = torch.from_numpy(W).to(dev)
    Wq, sW = m8.llmint8_quantize_weight(Wdv)
    del W
    sweep = {}
    for n_out in workloads.SWEEP_N_OUT:
        X = workloads.make(w5.with_(n_out=n_out), with_weight=False)[1]
        for thr in workloads.SWEEP_THRESHOLDS:
            key = f"n_out={n_out},thr={'inf' if thr == float('inf') else thr}"
            sweep[key] = one(key, w5, Wdv, Wq, sW, X, thr, CALL_TARGET_US["sweep"], accuracy=True)
    out["sweep"] = {"workload": "sweep T=2048 K=N=14336, n_out in {0, 8, 64, 512}, "
                                "threshold in {6, inf}", "points": sweep}
    del Wdv, Wq, sW
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixed_precision_int8_amd as m8
    import workloads

    m8.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    w = workloads.CONFIGS["prefill"]
    W, X, cols, _ = workloads.make(w)
    T, K, N = w.T, w.K, w.N
    Wd = torch.from_numpy(W).to(dev)
    Wq, sW = m8.llmint8_quantize_weight(Wd)
    Xd = torch.from_numpy(X).to(dev)
    Y = torch.empty((T, N), dtype=torch.float16, device=dev)
    ws = torch.empty((m8.llmint8_workspace_bytes(T, K, N),), dtype=torch.uint8, device=dev)
    thr = w.threshold
    torch.cuda.synchronize()

    def step():
        m8.llmint8_linear(Xd, Wq, sW, thr, Y=Y, workspace=ws)

    warm = 0
    w0 = time.perf_counter()
    while warm < args.warmup or (time.perf_counter() - w0) * 1e3 < args.warmup_ms:
        step()
        warm += 1
        if warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    ops = 2.0 * T * N * K
    tops = ops / (ms_per_step * 1e-3) / 1e12

    # per-kernel durations of the same call, events recorded between its kernels
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    nk = 0
    for row in evs:
        nk = m8.llmint8_linear_timed(Xd, Wq, sW, thr, Y, ws, row, path=m8.LLMINT8_PATH_AUTO)
    torch.cuda.synchronize()
    per_kernel = [float(np.mean([row[i].elapsed_time(row[i + 1]) for row in evs])) for i in range(nk)]
    names = ["ka_scan", "ka_prepare", "kb_gemm"] if nk == 3 else ["kd_gemv"]
    gemm_ms = per_kernel[-1]
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    traffic = committed_traffic()
    mfma_busy, sclk = committed_mfma_activity()

    result = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "prefill_mlp_up", "T": T, "K": K, "N": N, "threshold": thr,
                   "injected_outlier_columns": int(len(cols)), "seed": w.seed,
                   "pct_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2)},
        "roofline": {"bound": "mfma", "kernel": "int8 GEMM (kb_gemm_split for the 352x256 tile, "
                                                 "kb_gemm for the others)",
                     "gemm_tile": m8.llmint8_gemm_tile(T, N), "achieved": round(achieved, 2),
                     "counters": {"mfma_busy_pct": mfma_busy, "effective_sclk_ghz": sclk,
                                  "source": "profiles/kb_gemm_prefill_counters.txt"},
                     "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "unit_note": "int8 tera-ops/s, 2 ops per multiply-add",
                     "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": traffic,
                     "algorithmic_ops_per_launch": ops, "avg_launch_ms": round(gemm_ms, 5)},
        "kernels_ms": {n: round(v, 5) for n, v in zip(names, per_kernel)},
        "wall_s_timed_region": round(wall, 4),
    }

    # ---- the other workloads of the layer: tiny (latency), large hidden size and
    # the outlier-fraction sweep (n_out x threshold), each timed like the headline
    if not args.no_configs:
        result["configs"] = bench_configs(args, dev, stream)

    # ---- the GEMM's MFMA instruction on its own (register operands, no memory
    # traffic): what the chip delivers at its running clock
    if not args.no_probe:
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        pblocks, piters = 4 * cus, 2000
        pout = torch.empty((pblocks * 256,), dtype=torch.int32, device=dev)
        for _ in range(3):
            pops = probe_mfma_i8(pblocks, piters, pout, stream)
        torch.cuda.synchronize()
        pms = []
        for _ in range(5):
            p0 = torch.cuda.Event(enable_timing=True)
            p1 = torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            probe_mfma_i8(pblocks, piters, pout, stream)
            p1.record(stream)
            torch.cuda.synchronize()
            pms.append(p0.elapsed_time(p1))
        ptops = pops / (sorted(pms)[len(pms) // 2] * 1e-3) / 1e12
        gemm_tops = result["roofline"]["achieved"] if result.get("roofline") else None
        result["mfma_probe"] = {
            "instruction": "v_mfma_i32_32x32x32_i8", "workgroups": pblocks, "ops_per_call": pops,
            "TOPS": round(ptops, 1), "pct_int8_peak": round(100.0 * ptops / PEAK_INT8_TOPS, 2),
            "gemm_fraction_of_probe": round(gemm_tops / ptops, 4) if gemm_tops else None}
        del pout
        # the same instruction on operands that change every instruction (fragments
        # re-read from LDS full of pseudo-random bytes): int8 MFMA power grows with the
        # operand bits that switch, and the chip lowers its clock
        rout = torch.empty((cus * 512,), dtype=torch.int32, device=dev)
        for _ in range(3):
            rops = probe_mfma_i8_lds_random(cus, 400, rout, stream)
        torch.cuda.synchronize()
        rms = []
        for _ in range(5):
            p0 = torch.cuda.Event(enable_timing=True)
            p1 = torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            probe_mfma_i8_lds_random(cus, 400, rout, stream)
            p1.record(stream)
            torch.cuda.synchronize()
            rms.append(p0.elapsed_time(p1))
        rtops = rops / (sorted(rms)[2] * 1e-3) / 1e12
        del rout
        # the prefill GEMM itself on all-zero int8 codes (nothing switches) against
        # the workload's codes, same kernel and shapes
        Xz = torch.zeros((T, K), dtype=torch.float16, device=dev)
        Xz[:, 0] = 1.0
        Wz = torch.zeros((N, K), dtype=torch.float16, device=dev)
        Wz[:, 0] = 0.02
        Wqz, sWz = m8.llmint8_quantize_weight(Wz)
        del Wz
        Yz = torch.empty_like(Y)   # the headline's Y stays for the parity check
        zkern = time_linear(m8, torch, Xz, Wqz, sWz, thr, Yz, ws, args.steps, args.warmup, stream)[1]
        del Xz, Wqz, sWz, Yz
        result["mfma_probe"]["random_operands"] = {
            "kernel": "8 wavefronts x (4 x 2) 32x32 blocks, fragments re-read from LDS (random bytes) "
                      "every k-step, no global memory", "TOPS": round(rtops, 1),
            "pct_int8_peak": round(100.0 * rtops / PEAK_INT8_TOPS, 2),
            "gemm_fraction": round(gemm_tops / rtops, 4) if gemm_tops else None}
        if result.get("roofline"):
            # context for the GEMM's fraction: what the same instruction sustains on
            # operands that switch like real ones, with no memory traffic at all
            result["roofline"]["random_operand_mfma_TOPS"] = round(rtops, 1)
            result["roofline"]["frac_of_random_operand_mfma"] = round(gemm_tops / rtops, 4)
        result["mfma_probe"]["gemm_on_zero_codes"] = {
            "kb_gemm_us": round(zkern["kb_gemm"] * 1e3, 2),
            "kb_gemm_us_workload": round(gemm_ms * 1e3, 2),
            "TOPS": round(ops / (zkern["kb_gemm"] * 1e-3) / 1e12, 1)}

    # ---- decode-shaped workload: HBM-bound weight streaming
    if not args.no_decode:
        wd = workloads.CONFIGS["decode"]
        Wd2, X2, _, _ = workloads.make(wd)
        Wq2, sW2 = m8.llmint8_quantize_weight(torch.from_numpy(Wd2).to(dev))
        copies = [(Wq2.clone(), sW2.clone()) for _ in range(args.decode_copies)]
        dec = {}
        for Td in (1, 4, 8):
            Xt = torch.from_numpy(np.ascontiguousarray(X2[:Td])).to(dev)
            Yt = torch.empty((Td, wd.N), dtype=torch.float16, device=dev)
            wst = torch.empty((m8.llmint8_workspace_bytes(Td, wd.K, wd.N),), dtype=torch.uint8, device=dev)
            for i in range(args.warmup):
                q, s = copies[i % len(copies)]
                m8.llmint8_linear(Xt, q, s, wd.threshold, Y=Yt, workspace=wst)
            torch.cuda.synchronize()
            reps = max(args.steps, 2 * len(copies))
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for i in range(reps):
                q, s = copies[i % len(copies)]
                m8.llmint8_linear(Xt, q, s, wd.threshold, Y=Yt, workspace=wst)
            a1.record(stream)
            torch.cuda.synchronize()
            us = a0.elapsed_time(a1) / reps * 1e3
            # the same loop captured in a HIP graph: back-to-back calls without
            # the per-call host (Python) submission cost
            gus = graph_us_per_call(
                lambda i: m8.llmint8_linear(Xt, copies[i][0], copies[i][1], wd.threshold, Y=Yt,
                                            workspace=wst),
                len(copies), max(1, reps // len(copies)), stream)
            nbytes = wd.N * wd.K + 4 * wd.N + 2 * Td * wd.K + 2 * Td * wd.N
            gbs = nbytes / (us * 1e-6) / 1e9
            ggbs = nbytes / (gus * 1e-6) / 1e9
            # the kernel alone: events recorded on the launch stream right around it
            kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for row in kev:
                for e in row:
                    e.record(stream)
            torch.cuda.synchronize()
            for i, row in enumerate(kev):
                q, s = copies[i % len(copies)]
                m8.llmint8_linear_timed(Xt, q, s, wd.threshold, Yt, wst, row)
            torch.cuda.synchronize()
            kus = float(np.mean([row[0].elapsed_time(row[1]) for row in kev])) * 1e3
            dec[f"T{Td}"] = {"us_per_call": round(us, 3), "GB_per_s": round(gbs, 1),
                             "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
                             "graph_us_per_call": round(gus, 3), "graph_GB_per_s": round(ggbs, 1),
                             "graph_pct_hbm": round(100.0 * ggbs / PEAK_HBM_GBS, 2),
                             "kernel_us": round(kus, 3), "algorithmic_bytes": nbytes}
        dtraffic = committed_traffic(PROFILE_DECODE_COUNTERS, DECODE_SOURCES)
        k1 = dec["T1"]
        result["decode"] = {
            "workload": "decode_gemv K=4096 N=4096", "kernel": "kd_gemv",
            "weight_copies_cycled": len(copies), **dec,
            # per launch: the HIP-graph replay of back-to-back calls (events around the
            # replays, on the launch stream) divided by the calls; events around a single
            # kernel ("kernel_us") add their own ~2 us at this size
            "roofline": roofline("hbm", "kd_gemv<1> (T = 1)",
                                 k1["algorithmic_bytes"] / (k1["graph_us_per_call"] * 1e-6) / 1e9,
                                 PEAK_HBM_GBS, "GB/s", dtraffic,
                                 algorithmic_bytes_per_launch=k1["algorithmic_bytes"],
                                 avg_launch_us=k1["graph_us_per_call"])}
        if not args.no_probe:
            # what one launch can do at this size: an empty kernel, and a plain read of
            # the same weight bytes, both per call in a HIP graph, copies cycled the same way
            out1 = torch.zeros(1, dtype=torch.int32, device=dev)
            assert copies[0][0].numel() == wd.N * wd.K and (wd.N * wd.K) % 16 == 0
            n16 = wd.N * wd.K // 16          # exactly the int8 weight's bytes
            e_us = graph_us_per_call(lambda i: probe_empty(out1, torch.cuda.current_stream()),
                                     len(copies), 10, stream)
            s_us = graph_us_per_call(
                lambda i: probe_stream(copies[i][0], n16, out1, torch.cuda.current_stream()),
                len(copies), 10, stream)
            result["decode"]["floor"] = {
                "empty_kernel_graph_us_per_call": round(e_us, 3),
                "plain_read_graph_us_per_call": round(s_us, 3),
                "plain_read_GB_per_s": round(n16 * 16 / (s_us * 1e-6) / 1e9, 1),
                "plain_read_pct_hbm": round(100.0 * n16 * 16 / (s_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
                "note": "a plain read of the int8 decode weight (16.78 MB), 256-thread workgroups, one "
                        "16-byte load per thread, the fastest launch shape measured for this size"}
        del copies

    # ---- bf16 activations with a fused bias: the prefill and decode shapes again
    if not args.no_bf16:
        Wb_np = workloads.as_bf16_input(W)
        Xb_np = workloads.as_bf16_input(X)
        bias_np = workloads.make_bias(w.seed, N, bf16=True)

        def _bf(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        Wqb, sWb = m8.llmint8_quantize_weight_ex(_bf(Wb_np))
        Xb, biasb = _bf(Xb_np), _bf(bias_np)
        Yb = torch.empty((T, N), dtype=torch.bfloat16, device=dev)

        def timed_calls(fn, reps, warm):
            # warm by count and by time, as for the headline: clocks ramp up
            i = 0
            t_w = time.perf_counter()
            while i < warm or (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
                fn(i)
                i += 1
                if i % 16 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            q0 = torch.cuda.Event(enable_timing=True)
            q1 = torch.cuda.Event(enable_timing=True)
            q0.record(stream)
            for i in range(reps):
                fn(i)
            q1.record(stream)
            torch.cuda.synchronize()
            return q0.elapsed_time(q1) / reps

        pms = timed_calls(lambda i: m8.llmint8_linear_ex(Xb, Wqb, sWb, thr, bias=biasb, Y=Yb,
                                                         workspace=ws),
                          args.steps, max(args.warmup, 20))
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for row in bev:          # torch creates the HIP event on its first record
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        nkb = 0
        for row in bev:
            nkb = m8.llmint8_linear_timed_ex(Xb, Wqb, sWb, thr, Yb, ws, row, bias=biasb)
        torch.cuda.synchronize()
        kms = [float(np.mean([r[i].elapsed_time(r[i + 1]) for r in bev])) for i in range(nkb)]
        bgemm = kms[-1]
        bf = {"prefill": {"T": T, "K": K, "N": N, "ms_per_call": round(pms, 5),
                          "TOPS": round(ops / (pms * 1e-3) / 1e12, 2),
                          "pct_int8_peak": round(100.0 * ops / (pms * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                          "fp16_no_bias_ms_per_call": round(ms_per_step, 5),
                          "kernels_ms": {n_: round(v, 5) for n_, v in
                                         zip(["ka_scan", "ka_prepare", "kb_gemm"], kms)},
                          "roofline": roofline("mfma", "kb_gemm (bf16 activations, bias)",
                                               ops / (bgemm * 1e-3) / 1e12, PEAK_INT8_TOPS,
                                               "TFLOP/s",
                                               committed_traffic(PROFILE_NEXT_COUNTERS, NEXT_SOURCES,
                                                                 "bf16_gemm_hbm_bytes_per_launch"),
                                               unit_note="int8 tera-ops/s, 2 ops per multiply-add",
                                               algorithmic_ops_per_launch=ops,
                                               avg_launch_ms=round(bgemm, 5))}}
        if not args.no_decode:
            wd = workloads.CONFIGS["decode"]
            Wd3, X3, _, _ = workloads.make(wd, T=1)
            Wq3, sW3 = m8.llmint8_quantize_weight_ex(_bf(workloads.as_bf16_input(Wd3)))
            cps = [(Wq3.clone(), sW3.clone()) for _ in range(args.decode_copies)]
            X3b = _bf(workloads.as_bf16_input(X3))
            b3 = _bf(workloads.make_bias(wd.seed, wd.N, bf16=True))
            Y3 = torch.empty((1, wd.N), dtype=torch.bfloat16, device=dev)
            ws3 = torch.empty((m8.llmint8_workspace_bytes(1, wd.K, wd.N),), dtype=torch.uint8,
                              device=dev)
            reps = max(args.steps, 2 * len(cps))
            dms = timed_calls(lambda i: m8.llmint8_linear_ex(X3b, cps[i % len(cps)][0],
                                                             cps[i % len(cps)][1], wd.threshold,
                                                             bias=b3, Y=Y3, workspace=ws3),
                              reps, args.warmup)
            gus = graph_us_per_call(
                lambda i: m8.llmint8_linear_ex(X3b, cps[i][0], cps[i][1], wd.threshold, bias=b3,
                                               Y=Y3, workspace=ws3),
                len(cps), max(1, reps // len(cps)), stream)
            nbytes = wd.N * wd.K + 4 * wd.N + 2 * wd.K + 2 * wd.N + 2 * wd.N
            bf["decode_T1"] = {"K": wd.K, "N": wd.N, "us_per_call": round(dms * 1e3, 3),
                               "GB_per_s": round(nbytes / (dms * 1e-3) / 1e9, 1),
                               "pct_hbm": round(100.0 * nbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                               "graph_us_per_call": round(gus, 3),
                               "graph_pct_hbm": round(100.0 * nbytes / (gus * 1e-6) / 1e9
                                                      / PEAK_HBM_GBS, 2),
                               "algorithmic_bytes": nbytes, "weight_copies_cycled": len(cps)}
            del cps
        result["bf16_bias"] = {"workload": "bf16 X, bias and Y; the prefill and decode layers",
                               "timing": "whole calls between two events", **bf}

    # ---- 4-bit (NF4) weights: the decode-shaped linear that streams the codes,
    # at the decode layer (K = N = 4096) and the large layer (K = 8192, N = 28672)
    if not args.no_fourbit:
        fb = {}
        block = 64
        for lname, cfg, Ts, ncopies in (("decode_layer", workloads.CONFIGS["decode"], (1, 8), 32),
                                        ("large_layer", workloads.CONFIGS["large"], (1, 8), 3)):
            K4, N4 = cfg.K, cfg.N
            W4 = torch.from_numpy(workloads.make_weight(workloads.rng_for(cfg.seed, 0), N4, K4,
                                                        cfg.sigma)).to(dev)
            pk, am = m8.llmint8_quantize_4bit(W4, block, "nf4")
            del W4
            cps = [(pk.clone(), am.clone()) for _ in range(ncopies)]
            X4all = workloads.make(cfg, T=max(Ts), with_weight=False)[1]
            for T4 in Ts:
                X4 = torch.from_numpy(np.ascontiguousarray(X4all[:T4])).to(dev)
                Y4 = torch.empty((T4, N4), dtype=torch.float16, device=dev)

                def call(i, X4=X4, Y4=Y4, N4=N4):
                    p_, a_ = cps[i % len(cps)]
                    m8.llmint8_linear_4bit(X4, p_, a_, N4, block, "nf4", Y=Y4)

                i = 0
                t_w = time.perf_counter()
                while i < max(args.warmup, 2 * len(cps)) or (time.perf_counter() - t_w) * 1e3 < args.warmup_ms:
                    call(i)
                    i += 1
                    if i % 16 == 0:
                        torch.cuda.synchronize()
                torch.cuda.synchronize()
                reps = max(args.steps, 2 * len(cps)) // len(cps) * len(cps)
                q0 = torch.cuda.Event(enable_timing=True)
                q1 = torch.cuda.Event(enable_timing=True)
                q0.record(stream)
                for i in range(reps):
                    call(i)
                q1.record(stream)
                torch.cuda.synchronize()
                us = q0.elapsed_time(q1) / reps * 1e3
                gus = graph_us_per_call(lambda i: call(i), len(cps), max(2, reps // len(cps)),
                                        stream)
                nbytes = N4 * K4 // 2 + 4 * (N4 * K4 // block) + 2 * T4 * K4 + 2 * T4 * N4
                gbs = nbytes / (us * 1e-6) / 1e9
                fb[f"{lname}_T{T4}"] = {"K": K4, "N": N4, "T": T4, "us_per_call": round(us, 3),
                                        "GB_per_s": round(gbs, 1),
                                        "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
                                        "graph_us_per_call": round(gus, 3),
                                        "graph_pct_hbm": round(100.0 * nbytes / (gus * 1e-6) / 1e9
                                                               / PEAK_HBM_GBS, 2),
                                        "algorithmic_bytes": nbytes, "weight_copies_cycled": len(cps)}
            if lname == "large_layer":
                # the standalone dequantization of the same weight (fp16 out)
                outs = [torch.empty((N4 * K4,), dtype=torch.float16, device=dev) for _ in range(2)]
                for i in range(4):
                    m8.llmint8_dequantize_4bit(cps[i % 2][0], cps[i % 2][1], block, "nf4",
                                               out=outs[i % 2])
                torch.cuda.synchronize()
                q0 = torch.cuda.Event(enable_timing=True)
                q1 = torch.cuda.Event(enable_timing=True)
                q0.record(stream)
                for i in range(10):
                    m8.llmint8_dequantize_4bit(cps[i % 2][0], cps[i % 2][1], block, "nf4",
                                               out=outs[i % 2])
                q1.record(stream)
                torch.cuda.synchronize()
                us = q0.elapsed_time(q1) / 10 * 1e3
                nbytes = N4 * K4 // 2 + 4 * (N4 * K4 // block) + 2 * N4 * K4
                fb["large_layer_dequantize"] = {"us_per_call": round(us, 2),
                                                "GB_per_s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                                "pct_hbm": round(100.0 * nbytes / (us * 1e-6) / 1e9
                                                                 / PEAK_HBM_GBS, 2),
                                                "algorithmic_bytes": nbytes}
                del outs
            del cps, pk, am
        big = fb.get("large_layer_T1")
        rl = None
        if big:
            rl = roofline("hbm", "kn_gemv_x (large layer, T = 1; X rows in LDS)", big["GB_per_s"], PEAK_HBM_GBS, "GB/s",
                          committed_traffic(PROFILE_NEXT_COUNTERS, NEXT_SOURCES,
                                            "nf4_large_hbm_bytes_per_launch"),
                          algorithmic_bytes_per_launch=big["algorithmic_bytes"],
                          avg_launch_us=big["us_per_call"])
        result["fourbit_nf4"] = {"workload": "NF4 weights, block 64, fp16 activations; the decode "
                                             "and large layers", "kernel": "kn_gemv_x (X rows staged in LDS by chunks of K)",
                                 "bound": "hbm", "peak_GB_per_s": PEAK_HBM_GBS,
                                 "timing": "whole calls (one kernel each) between two events",
                                 "roofline": rl, **fb}

    # ---- input gradient through the frozen layer, at the prefill layer's shape:
    # one kernel, the weight dequantized on the fly
    if not args.no_backward:
        dY_np = workloads.make_output_grad(w.seed, T, N)
        dY = torch.from_numpy(dY_np).to(dev)
        dX = torch.empty((T, K), dtype=torch.float16, device=dev)

        def bstep():
            m8.llmint8_linear_backward_input(dY, Wq, sW, dX=dX)

        bw = 0
        w0 = time.perf_counter()
        while bw < args.warmup or (time.perf_counter() - w0) * 1e3 < args.warmup_ms:
            bstep()
            bw += 1
            if bw % 16 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(args.steps):
            bstep()
        b1.record(stream)
        torch.cuda.synchronize()
        bms = b0.elapsed_time(b1) / args.steps
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for row in bev:          # torch creates the HIP event on its first record
            for e in row:
                e.record(stream)
        torch.cuda.synchronize()
        for row in bev:
            m8.llmint8_linear_backward_input_timed(dY, Wq, sW, row, dX=dX)
        torch.cuda.synchronize()
        gf_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in bev]))
        flops = 2.0 * T * N * K
        # the separate transposed dequantization (llmint8_dequantize_weight_t), for reference
        WdT = torch.empty((K, N), dtype=torch.float16, device=dev)
        for _ in range(3):
            m8.llmint8_dequantize_weight_t(Wq, sW, WdT=WdT)
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record(stream)
        for _ in range(10):
            m8.llmint8_dequantize_weight_t(Wq, sW, WdT=WdT)
        d1.record(stream)
        torch.cuda.synchronize()
        dq_ms = d0.elapsed_time(d1) / 10
        del WdT
        dq_bytes = N * K + 4 * N + 2 * N * K
        result["backward_input"] = {
            "workload": "input gradient of the prefill layer: dY fp16 [2048, 11008] -> dX [2048, 4096]",
            "T": T, "K": K, "N": N, "dtype": "f16 operands, f32 accumulation",
            "warmup_steps_run": bw, "ms_per_call": round(bms, 5),
            "TFLOPS": round(flops / (bms * 1e-3) / 1e12, 2),
            "pct_fp16_peak": round(100.0 * flops / (bms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 2),
            "kernels_ms": {"kg_backward_dq": round(gf_ms, 5)},
            "roofline": {"bound": "mfma", "kernel": "kg_backward_dq (Wq dequantized on the fly)",
                         "achieved": round(flops / (gf_ms * 1e-3) / 1e12, 2),
                         "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(flops / (gf_ms * 1e-3) / 1e12 / PEAK_FP16_TFLOPS, 4),
                         "traffic": committed_traffic(PROFILE_BWD_COUNTERS, BWD_SOURCES,
                                                      "backward_hbm_bytes_per_launch"),
                         "algorithmic_ops_per_launch": flops,
                         "algorithmic_bytes_per_launch": N * K + 4 * N + 2 * T * N + 2 * T * K,
                         "avg_launch_ms": round(gf_ms, 5)},
            "dequantize_weight_t": {"kernel": "kg_dequant_t (llmint8_dequantize_weight_t, not on the "
                                              "backward path)", "ms_per_call": round(dq_ms, 5),
                                    "GB_per_s": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 1),
                                    "pct_hbm": round(100.0 * dq_bytes / (dq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)},
        }

    # ---- blockwise 8-bit codec: the prefill weight (fp16) and an optimizer-state
    # sized fp32 tensor, at the smallest and largest supported block
    if not args.no_codec:
        codec = {}
        tensors = {"f16_weight": Wd.reshape(-1),
                   "f32_state": torch.from_numpy(workloads.make_state(w.seed, N * K)).to(dev)}
        copies = 3   # three of everything: the working set exceeds the 256 MB MALL
        for name, t in tensors.items():
            n = t.numel()
            el = t.element_size()
            ins = [t.clone() for _ in range(copies)]
            for block in (64, 4096):
                nb = -(-n // block)
                qs = [torch.empty((n,), dtype=torch.int8, device=dev) for _ in range(copies)]
                ams = [torch.empty((nb,), dtype=torch.float32, device=dev) for _ in range(copies)]
                outs = [torch.empty_like(t) for _ in range(copies)]
                fns = {"quantize": lambda i: m8.llmint8_quantize_blockwise(ins[i], block, q=qs[i],
                                                                            absmax=ams[i]),
                       "dequantize": lambda i: m8.llmint8_dequantize_blockwise(qs[i], ams[i], block,
                                                                              out=outs[i])}
                nbytes = {"quantize": n * el + n + 4 * nb, "dequantize": n + 4 * nb + n * el}
                for op, fn in fns.items():
                    for i in range(max(args.warmup, 10)):
                        fn(i % copies)
                    torch.cuda.synchronize()
                    c0e = torch.cuda.Event(enable_timing=True)
                    c1e = torch.cuda.Event(enable_timing=True)
                    reps = max(args.steps // 2, 10) // copies * copies
                    c0e.record(stream)
                    for i in range(reps):
                        fn(i % copies)
                    c1e.record(stream)
                    torch.cuda.synchronize()
                    us = c0e.elapsed_time(c1e) / reps * 1e3
                    gbs = nbytes[op] / (us * 1e-6) / 1e9
                    codec[f"{name}_block{block}_{op}"] = {
                        "us_per_call": round(us, 2), "GB_per_s": round(gbs, 1),
                        "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2), "bytes": nbytes[op]}
            del ins, qs, ams, outs
        q64 = codec["f16_weight_block64_quantize"]
        result["blockwise_codec"] = {"workload": f"{N * K} elements (the prefill weight, and an fp32 "
                                                 "state of the same size)", "bound": "hbm",
                                     "copies_cycled": copies, "peak_GB_per_s": PEAK_HBM_GBS,
                                     "roofline": roofline(
                                         "hbm", "kq_blockwise (fp16, block 64)", q64["GB_per_s"],
                                         PEAK_HBM_GBS, "GB/s",
                                         committed_traffic(PROFILE_NEXT_COUNTERS, NEXT_SOURCES,
                                                           "codec_quantize_hbm_bytes_per_launch"),
                                         algorithmic_bytes_per_launch=q64["bytes"],
                                         avg_launch_us=q64["us_per_call"]),
                                     **codec}
        del tensors

    # ---- CPU oracle baseline on this host (bounded: the full prefill call once)
    if not args.no_cpu:
        import oracle
        threads = oracle_threads()
        Yg = Y.cpu().numpy()
        c0 = time.perf_counter()
        Wq_ref, sW_ref = oracle.quantize_weight(W)
        c1 = time.perf_counter()
        st = oracle.linear(X, Wq_ref, sW_ref, thr)
        c2 = time.perf_counter()
        cpu_tops = ops / (c2 - c1) / 1e12
        # the same call stage by stage, with the oracle's own step functions
        s0 = time.perf_counter()
        mask = oracle.outlier_columns(X, thr)
        Xq_o, aX_o = oracle.quantize_activations(X, mask)
        s1 = time.perf_counter()
        C_o = oracle.int8_matmul(Xq_o, Wq_ref)
        s2 = time.perf_counter()
        idx_o = np.flatnonzero(mask).astype(np.int32)
        Xo_o, Wd_o = oracle.outlier_operands(X, Wq_ref, sW_ref, idx_o)
        oracle.output(C_o, aX_o, sW_ref, Xo_o, Wd_o)
        s3 = time.perf_counter()
        del C_o, Xq_o
        result["cpu_baseline"] = {"value": round(cpu_tops, 5), "unit": "TOPS", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"one full prefill call (T={T},K={K},N={N}); "
                                            f"{c2 - c1:.2f} s, weight quantization "
                                            f"{c1 - c0:.2f} s not counted",
                                  "stages_s": {"outlier_scan_and_quantize": round(s1 - s0, 4),
                                               "int8_product_dgemm": round(s2 - s1, 4),
                                               "outlier_product_and_epilogue": round(s3 - s2, 4),
                                               "weight_quantize": round(c1 - c0, 4)}}
        result["parity"] = {"Y_max_abs_rel_err": oracle.parity_error(Yg, st.Y),
                            "outliers": st.count}
        if "bf16_bias" in result:
            rows = np.sort(np.random.default_rng(w.seed + 1).choice(T, size=16, replace=False))
            Wqb_ref, sWb_ref = oracle.quantize_weight(Wb_np, "bf16")
            c5 = time.perf_counter()
            stb = oracle.linear(Xb_np, Wqb_ref, sWb_ref, thr, rows=rows, dtype="bf16", bias=bias_np)
            c6 = time.perf_counter()
            result["bf16_bias"]["cpu_oracle"] = {
                "value": round(2.0 * len(rows) * N * K / (c6 - c5) / 1e12, 5), "unit": "TOPS",
                "cores": threads, "kind": "oracle",
                "sample": f"{len(rows)} output rows of the bf16 prefill call (the outlier scan and "
                          f"activation quantization cover all {T} rows), {c6 - c5:.2f} s"}
            Ybg = Yb.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
            result["bf16_bias"]["parity"] = {
                "Y_max_abs_rel_err_sampled_rows": oracle.parity_error(
                    oracle.bf16_bits_to_f32(Ybg), oracle.bf16_bits_to_f32(stb.Y)),
                "Y_bit_identical_fraction": float(np.mean(Ybg == stb.Y)), "rows": len(rows),
                "weight_codes_identical": bool(np.array_equal(Wqb.cpu().numpy(), Wqb_ref))}
        if "blockwise_codec" in result:
            sl = W[: (1 << 24) // K]                 # 16 M elements of the fp16 weight
            c7 = time.perf_counter()
            qc, ac = oracle.quantize_blockwise(sl, 64)
            c8 = time.perf_counter()
            oracle.dequantize_blockwise(qc, ac, 64)
            c9 = time.perf_counter()
            nq = sl.size
            result["blockwise_codec"]["cpu_oracle"] = {
                "value": round((3 * nq + 4 * nq // 64) / (c8 - c7) / 1e9, 3), "unit": "GB/s",
                "dequantize_GB_per_s": round((3 * nq + 4 * nq // 64) / (c9 - c8) / 1e9, 3),
                "cores": threads, "kind": "oracle",
                "sample": f"quantize then dequantize {nq} fp16 elements, block 64"}
        if "fourbit_nf4" in result:
            wd4 = workloads.CONFIGS["decode"]
            W4 = workloads.make_weight(workloads.rng_for(wd4.seed, 0), wd4.N, wd4.K, wd4.sigma)
            X4 = workloads.make(wd4, T=1, with_weight=False)[1]
            p4, a4 = oracle.quantize_4bit(W4, 64, "nf4")
            c10 = time.perf_counter()
            oracle.linear_4bit(X4, p4, a4, 64, "nf4", wd4.N)
            c11 = time.perf_counter()
            nb4 = wd4.N * wd4.K // 2 + 4 * wd4.N * wd4.K // 64 + 2 * wd4.K + 2 * wd4.N
            result["fourbit_nf4"]["cpu_oracle"] = {
                "value": round(nb4 / (c11 - c10) / 1e9, 4), "unit": "GB/s", "cores": threads,
                "kind": "oracle",
                "sample": f"one NF4 linear of the decode layer (T=1, K=N={wd4.K}), {c11 - c10:.2f} s"}
        if "backward_input" in result:
            # oracle input gradient on a seeded sample of rows: parity, and its CPU rate
            rows = np.sort(np.random.default_rng(w.seed).choice(T, size=64, replace=False))
            c3 = time.perf_counter()
            dX_ref = oracle.linear_backward_input(dY_np[rows], Wq_ref, sW_ref)
            c4 = time.perf_counter()
            dXg = dX.cpu().numpy()[rows]
            result["backward_input"]["parity"] = {
                "dX_max_abs_rel_err_sampled_rows": oracle.parity_error(dXg, dX_ref), "rows": len(rows)}
            result["backward_input"]["cpu_oracle"] = {
                "value": round(2.0 * len(rows) * N * K / (c4 - c3) / 1e12, 5), "unit": "TFLOPS",
                "cores": threads, "sample": f"{len(rows)} rows of dX, {c4 - c3:.2f} s "
                                            "(weight dequantization included)"}

    print(json.dumps(result), flush=True)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.empty((n,), dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
