#!/usr/bin/env python3
"""Benchmark of the FP16 -> FP32 block-tiled product on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20]

One step is one call C <- A.B + C at M = N = K = 8192 (FP16 A, B ~ N(0,1); FP32 C ~ N(0,1);
FP32 accumulation), inputs already resident in HBM.  Prints ONE JSON line with the throughput
(2*M*N*K FLOP per step), the roofline of the kernel against the FP16 dense MFMA peak, the
4096^3 pair (grouped vs row-major launch order) as secondary numbers, and the FP64 CPU oracle
timed on a bounded sample of the same workload.

Other modes (used for the rocprofv3 summaries under profiles/):
    --no-cpu-baseline --no-secondary     GPU steps only
    --copy-calibration                   a device-to-device copy of known size, for scaling the
                                         FETCH_SIZE / WRITE_SIZE counters
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12     # 256 CUs x 4096 FP16 FLOP/clk/CU x 2.4 GHz = 2516.6
METRIC = "FP16->FP32 GEMM TFLOP/s at 4096^3/8192^3 + fraction of MFMA FP16 peak"
KERNEL_SOURCES = [os.path.join(ROOT, "dense_tiled_gemm_f16_amd", "csrc", f)
                  for f in ("gemm_f16_f32.hip", "tile_order.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_gemm_accum8192.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(flops_per_launch: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if the summary
    is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    vals = dict(re.findall(r"^- (\w+): ([0-9a-fA-F.eE+-]+)\s*$", text, flags=re.M))
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_gemm(lib, dA, dB, dC, beta, opts, steps, warmup):
    """(seconds per call from HIP events on the launch stream, wall seconds for the K calls)."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        lib.gemm(dA, dB, dC, beta=beta, opts=opts)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        lib.gemm(dA, dB, dC, beta=beta, opts=opts)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3 / steps, wall


def cpu_baseline(A, B, C, beta, budget_s: float):
    """The FP64 oracle on whole rows of the same problem, as many as fit the time budget.

    A first batch (one row per thread) warms the oracle up; a second, timed batch measures the rate;
    a third fills the rest of the budget.  Only the second and third batches are reported."""
    import oracle
    M, K = A.shape
    N = B.shape[1]
    threads = oracle.max_threads()

    def run(r0, n):
        t0 = time.perf_counter()
        oracle.gemm(A[r0:r0 + n], B, beta=beta, C=(C[r0:r0 + n] if C is not None else None))
        return time.perf_counter() - t0

    r = min(threads, M)
    run(0, r)
    n2 = min(4 * threads, M - r)
    spent = run(r, n2) if n2 > 0 else 0.0
    done = n2
    if n2 > 0 and spent < budget_s:
        n3 = min(int(n2 * (budget_s - spent) / max(spent, 1e-9)), M - r - n2)
        if n3 > 0:
            spent += run(r + n2, n3)
            done += n3
    tflops = 2.0 * done * N * K / spent / 1e12 if done else 0.0
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows of the %dx%dx%d product (FP64 triple loop), %.1f s" % (done, M, M, N, K, spent)}


def copy_calibration(nbytes: int, reps: int):
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=-1)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus %d asked)" % args.gpus,
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import dense_tiled_gemm_f16_amd as lib
    from gemm_inputs import PROBLEMS, problem_arrays

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    lib.load()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return 0

    opts = {"tile": args.tile, "group_m": args.group_m, "xcd_remap": args.xcd_remap}
    p = PROBLEMS["accum8192"]
    print("bench: generating %s inputs" % p.name, file=sys.stderr, flush=True)
    A, B, C = problem_arrays(p)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.from_numpy(C).cuda()
    plan = lib.plan(dA, dB, dC, opts)
    flops = 2.0 * p.M * p.N * p.K

    print("bench: timing %d steps after %d warmup" % (args.steps, args.warmup), file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    sec, wall = time_gemm(lib, dA, dB, dC, p.beta, opts, args.steps, args.warmup)
    tflops = flops / sec / 1e12

    out = {
        "metric": METRIC,
        "value": round(flops * args.steps / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "D = A.B + C, M=N=K=8192, A,B fp16 N(0,1), C fp32 N(0,1), fp32 accumulate",
                   "M": p.M, "N": p.N, "K": p.K, "beta": p.beta, "seed": p.seed, "accumulate": "f32",
                   "tile": "%dx%d" % (plan["bm"], plan["bn"]), "bk": plan["bk"], "group_m": plan["group_m"],
                   "xcd_remap": plan["xcd_remap"], "grid": plan["grid"], "parallelism": "single GPU"},
    }
    traffic = read_traffic(flops)
    out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(PEAK_TFLOPS, 1),
                       "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4),
                       "traffic": traffic, "kernel_ms": round(sec * 1e3, 4),
                       "kernel": "gemm_f16_f32_kernel<Tile<%d,%d,...>>" % (plan["bm"], plan["bn"]),
                       "kernel_source_sha256": kernel_source_hash()}

    if not args.no_secondary:
        del dA, dB, dC
        torch.cuda.empty_cache()
        q = PROBLEMS["square4096"]
        A4, B4, _ = problem_arrays(q)
        dA4, dB4 = torch.from_numpy(A4).cuda(), torch.from_numpy(B4).cuda()
        dC4 = torch.empty((q.M, q.N), dtype=torch.float32, device="cuda")
        sec_g, _ = time_gemm(lib, dA4, dB4, dC4, 0.0, {"group_m": 8}, 50, 10)
        sec_r, _ = time_gemm(lib, dA4, dB4, dC4, 0.0, {"group_m": 1, "xcd_remap": 0}, 50, 10)
        f4 = 2.0 * q.M * q.N * q.K
        out["secondary"] = {
            "square4096_group_m8_tflops": round(f4 / sec_g / 1e12, 2),
            "square4096_row_major_tflops": round(f4 / sec_r / 1e12, 2),
            "square4096_tile": "%dx%d" % tuple(lib.plan(dA4, dB4, dC4)[k] for k in ("bm", "bn")),
        }
        del dA4, dB4, dC4

    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host cores", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(A, B, C, p.beta, args.cpu_budget)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
