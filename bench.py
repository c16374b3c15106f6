"""Throughput of the LLM.int8() linear layer on one MI355X.

A step is one full forward call (outlier scan, activation quantization, int8
GEMM with fused dequantization and fp16 outlier product) over one batch of the
prefill workload: X fp16 [2048, 4096] with 6 injected outlier feature columns,
W [11008, 4096] stored as int8 + per-row fp32 scale, threshold 6.0. The weight
is quantized once before timing (load time). Inputs are synthetic and seeded
and already resident in HBM when the timed region starts.

Prints one JSON line. Besides the headline TOPS it carries the roofline of the
dominant kernel (the int8 GEMM, timed with HIP events on the launch stream),
the decode-shaped workload (T=8, K=N=4096) as GB/s against HBM bandwidth, and
the CPU oracle timed on this host.
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
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "kb_gemm_prefill_counters.txt")


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
    p.add_argument("--decode-copies", type=int, default=24,
                   help="distinct weight copies cycled in the decode timing (> last-level cache)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the measurement, run 5 plain device copies of MIB MiB (untimed), "
                        "a known-size reference for HBM byte counters")
    return p.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("gemm.hip", "device_util.h", "internal.h"):
        with open(os.path.join(ROOT, "mixed_precision_int8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(units_per_launch_bytes):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary, or
    None when absent or taken on different kernel source."""
    if not os.path.exists(PROFILE_COUNTERS):
        return None
    text = open(PROFILE_COUNTERS).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash():
        return None
    m = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
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
    traffic = committed_traffic(None)

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
        "roofline": {"bound": "mfma", "kernel": "kb_gemm", "achieved": round(achieved, 2),
                     "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                     "unit_note": "int8 tera-ops/s, 2 ops per multiply-add",
                     "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": traffic,
                     "algorithmic_ops_per_launch": ops, "avg_launch_ms": round(gemm_ms, 5)},
        "kernels_ms": {n: round(v, 5) for n, v in zip(names, per_kernel)},
        "wall_s_timed_region": round(wall, 4),
    }

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
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(len(copies)):
                    q, s = copies[i % len(copies)]
                    m8.llmint8_linear(Xt, q, s, wd.threshold, Y=Yt, workspace=wst)
            g.replay()
            torch.cuda.synchronize()
            greps = max(1, reps // len(copies))
            a0.record(stream)
            for _ in range(greps):
                g.replay()
            a1.record(stream)
            torch.cuda.synchronize()
            gus = a0.elapsed_time(a1) / (greps * len(copies)) * 1e3
            nbytes = wd.N * wd.K + 4 * wd.N + 2 * Td * wd.K + 2 * Td * wd.N
            gbs = nbytes / (us * 1e-6) / 1e9
            ggbs = nbytes / (gus * 1e-6) / 1e9
            dec[f"T{Td}"] = {"us_per_call": round(us, 3), "GB_per_s": round(gbs, 1),
                             "pct_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
                             "graph_us_per_call": round(gus, 3), "graph_GB_per_s": round(ggbs, 1),
                             "graph_pct_hbm": round(100.0 * ggbs / PEAK_HBM_GBS, 2),
                             "algorithmic_bytes": nbytes}
            del g
        result["decode"] = {"workload": "decode_gemv K=4096 N=4096", "kernel": "kd_gemv",
                            "weight_copies_cycled": len(copies), **dec}
        del copies

    # ---- CPU oracle baseline on this host (bounded: the full prefill call once)
    if not args.no_cpu:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # noqa: BLE001
            threads = os.cpu_count() or 1
        Yg = Y.cpu().numpy()
        c0 = time.perf_counter()
        Wq_ref, sW_ref = oracle.quantize_weight(W)
        c1 = time.perf_counter()
        st = oracle.linear(X, Wq_ref, sW_ref, thr)
        c2 = time.perf_counter()
        cpu_tops = ops / (c2 - c1) / 1e12
        result["cpu_baseline"] = {"value": round(cpu_tops, 5), "unit": "TOPS", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"one full prefill call (T={T},K={K},N={N}); "
                                            f"{c2 - c1:.2f} s, weight quantization "
                                            f"{c1 - c0:.2f} s not counted"}
        result["parity"] = {"Y_max_abs_rel_err": oracle.parity_error(Yg, st.Y),
                            "outliers": st.count}

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
