#!/usr/bin/env python3
"""Benchmark of the FP16 -> FP32 block-tiled product on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 200]

Warm-up: at least --warmup untimed calls, and more until the board has settled -- at least
--warmup-seconds (1.0 s) of calls and two consecutive batches within 1 % of each other (at most
8 s).  The board's clock climbs for a fraction of a second once the product starts: a run with
5 warm-up calls and 20 timed ones measured 0.98 ms per call where the settled board takes 0.87 ms.
The JSON line reports the warm-up calls actually run ("warmup_calls_run").

One step is one call C <- A.B + C at M = N = K = 8192 (FP16 A, B ~ N(0,1); FP32 C ~ N(0,1);
FP32 accumulation), inputs already resident in HBM.  Prints ONE JSON line with the throughput
(2*M*N*K FLOP per step), the roofline of the kernel against the FP16 dense MFMA peak, the
4096^3 pair (grouped vs row-major launch order) as secondary numbers, and the FP64 CPU oracle
timed on a bounded sample of the same workload.

The line also carries the board's sustained matrix-core ceiling ("mfma_ceiling"): back-to-back
v_mfma_f32_32x32x16_f16 with changing N(0,1)-like operands on every SIMD, from a separate
measurement-only library.  Under the board's power limit this sets the clock, so it bounds what
any FP16 GEMM sustains on the same board; the GEMM's fraction of it is reported next to the
fraction of the published peak.  It is measured right before the warm-up and again right after
the timed window.  "clock_ghz_timed" is the GEMM's own effective clock in the timed window: its
GPU-active cycles per dispatch (GRBM_GUI_ACTIVE per XCD, from the committed counter summary of the
same kernel source) over the timed per-call duration.

Other modes (used for the summaries under profiles/):
    --no-cpu-baseline --no-secondary     GPU steps only
    --workload NAME [--tile/--group-m/--xcd-remap]
                                         GPU steps only, on another workload of gemm_inputs
    --copy-calibration                   a device-to-device copy of known size, for scaling the
                                         FETCH_SIZE / WRITE_SIZE counters
    --configs                            every workload: kernel time (back-to-back calls),
                                         TFLOP/s, tile grid, and the oracle's time on the host
                                         cores; prints a markdown table
    --splitk                             deep-K problems with few output tiles: plain call against
                                         split-K with the library's split count (markdown table)
    --skinny                             skinny problems (a few rows or columns, long K): plain call
                                         against the library's call (split-K where its cost model
                                         prefers it), GB/s against HBM (markdown table)
    --mfma-ceiling                       the matrix-core ceiling alone
    --power                              rocm-smi power and clock readings while 8192^3 runs
    --softmax                            the fused row softmax (second workload): GPU time, GB/s
                                         against the 8 TB/s HBM roofline, the oracle's time
                                         (--softmax-shapes MxN ...: only those shapes)
    --unaligned                          odd squares (rows not 16-byte aligned, register-staged
                                         path): every tile, the default, torch.matmul
    --ksweep                             8192 x 8192 x K for K = 2048..32768: the per-call cost that
                                         does not grow with K, and the main loop's rate
    --variant noswizzle                  GPU steps only, through the measurement build without the
                                         LDS swizzle (for the bank-conflict counter comparison)
    --lds-probe                          LDS fragment-read rate of the product's read patterns under
                                         each swizzle key (measurement library)
    --latency-probe                      latency of one direct-to-LDS load served by L2 or by HBM
    --lds-mix-probe                      LDS traffic of a main-loop slice without the matrix instructions:
                                         direct-to-LDS loads and fragment reads alone and together
    --vmem-probe                         load-path cost of MFMA fragments read straight into registers
    --phases [--workload/--shape/--ld]   per-phase shader cycles of one call (prologue, main loop,
                                         K tail, epilogue, gaps between tiles on a CU), from the
                                         measurement build whose kernels stamp their phases
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12     # 256 CUs x 4096 FP16 FLOP/clk/CU x 2.4 GHz = 2516.6
METRIC = "FP16\u2192FP32 GEMM TFLOP/s at 4096\u00b3/8192\u00b3 + fraction of MFMA FP16 peak"
KERNEL_SOURCES = [os.path.join(ROOT, "dense_tiled_gemm_f16_amd", "csrc", f)
                  for f in ("gemm_f16_f32.hip", "tile_order.h", "gemm_launch.h")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_gemm_accum8192.md")
COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "counters_gemm_accum8192.md")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_summary_value(path: str, key: str):
    """A number from a committed rocprofv3 summary's "- key: value" lines, or None if the summary
    is missing, lacks the key, or was taken on a different kernel source."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    vals = dict(re.findall(r"^- (\w+): ([0-9a-fA-F.eE+-]+)\s*$", text, flags=re.M))
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def read_traffic(flops_per_launch: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary (None if stale or missing)."""
    return read_summary_value(TRAFFIC_SUMMARY, "hbm_bytes_per_launch")


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


def time_calls(fn, steps):
    """(seconds per call from HIP events on the launch stream, wall seconds for the `steps` calls)."""
    import torch
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / 1e3 / steps, wall


def settle(fn, min_calls: int, min_seconds: float, max_seconds: float = 8.0, batch: int = 20, tol: float = 0.01):
    """Untimed warm-up: at least min_calls calls and min_seconds of wall time, then until two
    consecutive batches of `batch` calls take per-call times within `tol` of each other (or
    max_seconds have passed).  Returns (calls run, seconds, per-call seconds of the last batch)."""
    import torch
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    calls = 0
    for _ in range(min_calls):
        fn()
        calls += 1
    torch.cuda.synchronize()
    prev = last = None
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        calls += batch
        prev, last = last, e0.elapsed_time(e1) / 1e3 / batch
        spent = time.perf_counter() - t0
        if spent >= max_seconds:
            break
        if spent >= min_seconds and prev is not None and abs(last - prev) <= tol * prev:
            break
    return calls, time.perf_counter() - t0, last


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


def mfma_ceiling(seconds: float = 1.0, grid: int = 256):
    """Sustained FP16 matrix-core throughput and shader clock of this board (see the module doc)."""
    import ctypes
    import numpy as np
    import torch
    from dense_tiled_gemm_f16_amd import build as hb
    lib = ctypes.CDLL(hb.MEASURE_LIB_PATH)
    lib.gemm_f16_mfma_ceiling.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.gemm_f16_mfma_ceiling.restype = ctypes.c_int
    rng = np.random.default_rng(11)
    src = torch.from_numpy(rng.standard_normal(1024 * 8).astype(np.float16)).cuda()
    out = torch.zeros(grid * 4, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    iters = 4000                                     # 256k MFMAs per wave, ~5 ms per launch
    t0 = time.perf_counter()
    while True:
        rc = lib.gemm_f16_mfma_ceiling(src.data_ptr(), out.data_ptr(), grid, iters, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("mfma ceiling launch failed (%d)" % rc)
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    d = out.cpu().numpy().reshape(grid, 4).astype(np.float64)
    sec = d[:, 1] / 100e6                             # s_memrealtime ticks at 100 MHz
    mfmas = d[:, 2]
    waves = grid * 4
    flops = waves * mfmas.mean() * 2 * 32 * 32 * 16
    return {"tflops": round(flops / sec.max() / 1e12, 1), "clock_ghz": round(float((d[:, 0] / sec).mean()) / 1e9, 3),
            "ticks_per_mfma": round(float((d[:, 0] / mfmas).mean()), 2), "seconds": round(seconds, 1)}


def graph_seconds(fn, calls: int = 50, replays: int = 20) -> float:
    """Seconds per call of `fn` from `calls` calls captured in one graph and replayed: back-to-back
    calls of a few tens of microseconds are bound by the host's launch rate, not the kernels (the
    library launches only kernels on the stream, so the graph holds exactly its work)."""
    import torch
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fn()
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / (replays * calls)


def eager_seconds(fn, target_s: float = 0.05) -> float:
    """Seconds per call of `fn` from HIP events around back-to-back calls (about target_s of work)."""
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    reps = int(min(2000, max(10, target_s / max(time.perf_counter() - t0, 1e-6))))
    for _ in range(max(3, reps // 10)):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def vendor_seconds(dA, dB, dC, beta: float, rounds: int = 5, calls: int = 20):
    """Seconds per call of the same product through torch -- FP16 operands, FP32 result:
    torch.addmm(C, A, B, out_dtype=float32) for beta = 1, torch.mm(A, B, out_dtype=float32) for
    beta = 0 -- after a one-second settle, median of `rounds` batches; None where this torch has no
    FP32-output product for FP16 operands."""
    import torch
    try:
        if beta == 1.0:
            fn = lambda: torch.addmm(dC, dA, dB, out_dtype=torch.float32)
        elif beta == 0.0:
            fn = lambda: torch.mm(dA, dB, out_dtype=torch.float32)
        else:
            return None
        fn()
        torch.cuda.synchronize()
    except (RuntimeError, TypeError):
        return None
    t_end = time.perf_counter() + 1.0
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()
    res = []
    for _ in range(rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / 1e3 / calls)
    return statistics.median(res)


def same_op_seconds(A, B):
    """Seconds per call of torch's product of the same FP16 operands with an FP32 result
    (torch.mm with out_dtype), the operation this library computes; None where this torch lacks it."""
    import torch
    fn = lambda: torch.mm(A, B, out_dtype=torch.float32)
    try:
        fn()
        torch.cuda.synchronize()
    except (RuntimeError, TypeError):
        return None
    return call_seconds(fn)


def call_seconds(fn) -> float:
    sec = eager_seconds(fn)
    return graph_seconds(fn) if sec < 100e-6 else sec


SPLITK_SHAPES = [(128, 128, 131072), (256, 256, 65536), (512, 512, 65536), (1024, 1024, 32768),
                 (256, 4096, 16384), (1536, 1536, 24576), (2048, 2048, 16384), (4096, 4096, 4096)]


def run_splitk(args):
    """Deep-K problems with few output tiles: the plain call, split-K with the library's split count,
    and torch.matmul (hipBLASLt) on the same FP16 operands for context; checks the split result
    against the plain one on sampled outputs."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    gen = torch.Generator(device="cuda").manual_seed(7)
    print("| M x N x K | plain: tiles | plain | split count | split-K | gain | torch.matmul FP16 "
          "| torch, same operation (FP32 result) |")
    print("|---|---|---|---|---|---|---|---|")
    for M, N, K in SPLITK_SHAPES:
        A = torch.randn((M, K), device="cuda", generator=gen).half()
        B = torch.randn((K, N), device="cuda", generator=gen).half()
        C0 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        C1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        s = lib.gemm_f16_f32_splitk_choose(M, N, K)
        W = torch.empty(max(lib.gemm_f16_f32_splitk_workspace(M, N, s) // 4, 1), dtype=torch.float32, device="cuda")
        flops = 2.0 * M * N * K
        t_plain = call_seconds(lambda: lib.gemm(A, B, C0, splits=1))
        t_split = call_seconds(lambda: lib.gemm_splitk(A, B, C1, splits=s, workspace=W))
        t_torch = call_seconds(lambda: torch.matmul(A, B))
        t_same = same_op_seconds(A, B)
        torch.cuda.synchronize()
        diff = float((C0 - C1).abs().max())
        assert diff <= 1e-4 * K ** 0.5, diff
        pl = lib.plan(A, B, C0)
        grid_s = "%d of %dx%d" % (pl["grid"], pl["bm"], pl["bn"])
        same = "%.1f us (%.0f TF)" % (t_same * 1e6, flops / t_same / 1e12) if t_same else "--"
        print("| %dx%dx%d | %s | %.1f us (%.0f TF) | %d | %.1f us (%.0f TF) | %.2fx | %.1f us (%.0f TF) | %s |" % (
            M, N, K, grid_s, t_plain * 1e6, flops / t_plain / 1e12, s, t_split * 1e6, flops / t_split / 1e12,
            t_plain / t_split, t_torch * 1e6, flops / t_torch / 1e12, same), flush=True)
        del A, B, C0, C1, W
        torch.cuda.empty_cache()
    return 0


SKINNY_SHAPES = [(1, 4096, 4096), (1, 8192, 8192), (16, 8192, 8192), (16, 8192, 28672), (16, 28672, 8192),
                 (8, 5120, 13824), (64, 4096, 16384), (128, 8192, 8192), (256, 8192, 28672), (1, 2048, 8192),
                 (64, 1024, 32768), (8192, 64, 8192), (1, 16384, 4096)]


def run_skinny(args):
    """Skinny problems (a few rows or columns, long K): memory-bound, so they are timed against HBM.
    The plain call (splits=1) against the library's own call (gemm(): split-K when its cost model
    predicts it faster), and torch.matmul on the same operands for context; algorithmic bytes are
    A, B and C once, 2(MK + KN) + 4MN.  Checks the library's result against the plain one."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    gen = torch.Generator(device="cuda").manual_seed(13)
    print("| M x N x K | plain: tiles | plain | split count | library's call | GB/s (A, B, C once) | of 8 TB/s | "
          "gain | torch.matmul FP16 | torch, same operation (FP32 result) |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    shapes = SKINNY_SHAPES
    if args.skinny_shapes:
        shapes = [tuple(int(v) for v in t.lower().split("x")) for t in args.skinny_shapes]
    for M, N, K in shapes:
        A = torch.randn((M, K), device="cuda", generator=gen).half()
        B = torch.randn((K, N), device="cuda", generator=gen).half()
        C0 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        C1 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        s = lib.gemm_f16_f32_splitk_choose(M, N, K)
        W = torch.empty(max(lib.gemm_f16_f32_splitk_workspace(M, N, s) // 4, 1), dtype=torch.float32, device="cuda")
        t_plain = call_seconds(lambda: lib.gemm(A, B, C0, splits=1))
        t_lib = call_seconds(lambda: lib.gemm(A, B, C1, workspace=W))
        t_torch = call_seconds(lambda: torch.matmul(A, B))
        t_same = same_op_seconds(A, B)
        torch.cuda.synchronize()
        diff = float((C0 - C1).abs().max())
        assert diff <= 1e-4 * K ** 0.5, diff
        pl = lib.plan(A, B, C0)
        byt = 2.0 * (M * K + K * N) + 4.0 * M * N
        print("| %dx%dx%d | %d of %dx%d | %.1f us | %d | %.1f us | %.0f | %.2f | %.2fx | %.1f us | %s |" % (
            M, N, K, pl["grid"], pl["bm"], pl["bn"], t_plain * 1e6, s, t_lib * 1e6, byt / t_lib / 1e9,
            byt / t_lib / 8e12, t_plain / t_lib, t_torch * 1e6, "%.1f us" % (t_same * 1e6) if t_same else "--"),
            flush=True)
        del A, B, C0, C1, W
        torch.cuda.empty_cache()
    return 0


KSWEEP = (2048, 4096, 8192, 16384, 32768)


def run_ksweep(args):
    """8192 x 8192 x K for growing K, beta = 1 and 0: the fit time = a + b*K separates the per-call
    cost that does not grow with K (the lockstep prologue and epilogue of each round of tiles) from
    the main loop's rate."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M = N = 8192
    gen = torch.Generator(device="cuda").manual_seed(12)
    C = torch.randn((M, N), device="cuda", generator=gen)
    times = {0: [], 1: []}
    print("| K | beta = 1 | beta = 0 |")
    print("|---|---|---|")
    for K in KSWEEP:
        A = torch.randn((M, K), device="cuda", generator=gen).half()
        B = torch.randn((K, N), device="cuda", generator=gen).half()
        f = 2.0 * M * N * K
        call_seconds(lambda: lib.gemm(A, B, C, beta=1.0))   # untimed: the first reading of a size runs low
        t1 = call_seconds(lambda: lib.gemm(A, B, C, beta=1.0))
        t0 = call_seconds(lambda: lib.gemm(A, B, C, beta=0.0))
        times[1].append(t1)
        times[0].append(t0)
        print("| %d | %.1f us (%.0f TF) | %.1f us (%.0f TF) |" % (K, t1 * 1e6, f / t1 / 1e12, t0 * 1e6, f / t0 / 1e12),
              flush=True)
        del A, B
    for beta in (1, 0):
        # least squares over the K values
        n = len(KSWEEP)
        mk = sum(KSWEEP) / n
        mt = sum(times[beta]) / n
        b = sum((k - mk) * (t - mt) for k, t in zip(KSWEEP, times[beta])) / sum((k - mk) ** 2 for k in KSWEEP)
        a = mt - b * mk
        print("\nbeta = %d: fixed %.1f us per call, main loop %.0f TFLOP/s" % (beta, a * 1e6, 2.0 * M * N / b / 1e12))
    return 0


UNALIGNED_SIZES = (1025, 1793, 2049, 2561, 3073, 4097, 6143, 8191)


def run_unaligned(args):
    """Odd squares n^3 with dense rows (n elements, not a multiple of 8): both operands take the
    register-staged path.  Each tile forced, the library's default, and torch.matmul (hipBLASLt,
    FP16 output) on the same operands for context; the default's result is checked against the
    K-split-free 128x128 tile's on sampled rows."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    gen = torch.Generator(device="cuda").manual_seed(11)
    tiles = (1, 2, 3, 4, 5)
    print("| n | default tile | default | " + " | ".join("tile %d" % t for t in tiles)
          + " | torch.matmul FP16 | torch, same operation (FP32 result) |")
    print("|---|---|---|" + "---|" * len(tiles) + "---|---|")
    for n in UNALIGNED_SIZES:
        A = torch.randn((n, n), device="cuda", generator=gen).half()
        B = torch.randn((n, n), device="cuda", generator=gen).half()
        C0 = torch.empty((n, n), dtype=torch.float32, device="cuda")
        C1 = torch.empty((n, n), dtype=torch.float32, device="cuda")
        pl = lib.plan(A, B, C0)
        assert not pl["vec_a"] and not pl["vec_b"]
        tf = lambda sec: 2.0 * n ** 3 / sec / 1e12
        call_seconds(lambda: lib.gemm(A, B, C0))   # untimed: the first reading of a size runs low
        t_def = call_seconds(lambda: lib.gemm(A, B, C0))
        per_tile = [call_seconds(lambda: lib.gemm(A, B, C1, opts={"tile": t})) for t in tiles]
        lib.gemm(A, B, C1, opts={"tile": 2})
        t_torch = call_seconds(lambda: torch.matmul(A, B))
        t_same = same_op_seconds(A, B)
        torch.cuda.synchronize()
        rows = torch.arange(0, n, max(1, n // 64), device="cuda")
        diff = float((C0[rows] - C1[rows]).abs().max())
        assert diff <= 2e-4 * n ** 0.5, diff
        dflt = "%d" % pl["tile"] if not pl["tile2"] else "%d, %s from %d: %d" % (
            pl["tile"], "columns" if pl["split_dim"] else "rows", pl["split_at"], pl["tile2"])
        print("| %d | %s | %.0f TF | %s | %.0f TF | %s |" % (n, dflt, tf(t_def), " | ".join("%.0f" % tf(x) for x in per_tile),
                                                          tf(t_torch), "%.0f TF" % tf(t_same) if t_same else "--"),
              flush=True)
        del A, B, C0, C1
        torch.cuda.empty_cache()
    return 0


def run_power(args):
    """Board power and clocks while 8192^3 D = A.B + C runs back to back: rocm-smi is read while a queue
    of calls keeps the GPU busy; prints a table of its readings (sclk level, temperatures, power when
    reported)."""
    import subprocess
    import torch
    import dense_tiled_gemm_f16_amd as lib
    from gemm_inputs import PROBLEMS, problem_arrays
    p = PROBLEMS["accum8192"]
    A, B, C = problem_arrays(p)
    dA, dB, dC = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(), torch.from_numpy(C).cuda()
    for _ in range(20):
        lib.gemm(dA, dB, dC, beta=1.0)
    torch.cuda.synchronize()
    def smi():
        out = subprocess.run(["rocm-smi", "--showpower", "--showclocks", "--showtemp"], capture_output=True,
                             text=True, timeout=60)
        return "\n".join(l for l in (out.stdout + out.stderr).splitlines()
                         if l.strip() and not set(l.strip()) <= set("=") and "ROCm System" not in l)
    def parse(text):
        sclk = re.search(r"sclk clock level: \d+: \((\d+)Mhz\)", text)
        tj = re.search(r"Sensor junction\) \(C\): ([\d.]+)", text)
        tm = re.search(r"Sensor memory\) \(C\): ([\d.]+)", text)
        pw = re.search(r"Power \(W\): ([\d.]+)", text)
        return [m.group(1) if m else "-" for m in (sclk, tj, tm, pw)]
    readings = [("idle (after warm-up)", parse(smi()))]
    for i in range(6):
        for _ in range(1000):              # about a second of queued work per reading
            lib.gemm(dA, dB, dC, beta=1.0)
        readings.append(("GEMM queue running, reading %d" % i, parse(smi())))
    torch.cuda.synchronize()
    print("| reading | sclk level reported (MHz) | junction temperature (C) | memory temperature (C) | power (W) |")
    print("|---|---|---|---|---|")
    for name, vals in readings:
        print("| %s | %s |" % (name, " | ".join(vals)))
    return 0


def run_configs(args):
    """Every workload: GPU kernel time from HIP events around back-to-back calls, and the oracle."""
    import numpy as np
    import torch
    import dense_tiled_gemm_f16_amd as lib
    import oracle
    from dense_tiled_gemm_f16_amd import model
    from gemm_inputs import PROBLEMS, problem_arrays
    rows = []
    cases = [(n, {}, None) for n in ("square256", "ragged300x200x150", "ragged129x65x33", "skinny1x1000x64",
                                     "square1792", "square1793")]
    cases += [("square1793", {}, 1800), ("square4096", {"group_m": 8}, None),
              ("square4096", {"group_m": 1, "xcd_remap": 0}, None), ("accum8192", {}, None)]
    threads = oracle.max_threads()
    for name, opts, ld in cases:
        p = PROBLEMS[name]
        A, B, C = problem_arrays(p)
        lda, ldb, ldc = (ld, ld, ld) if ld else (p.K, p.N, p.N)
        dA = torch.zeros((p.M, lda), dtype=torch.float16, device="cuda")[:, :p.K]
        dB = torch.zeros((p.K, ldb), dtype=torch.float16, device="cuda")[:, :p.N]
        dC = torch.zeros((p.M, ldc), dtype=torch.float32, device="cuda")[:, :p.N]
        dA.copy_(torch.from_numpy(A)); dB.copy_(torch.from_numpy(B))
        if C is not None:
            dC.copy_(torch.from_numpy(C))
        flops = 2.0 * p.M * p.N * p.K
        lib.gemm(dA, dB, dC, beta=p.beta, opts=opts)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lib.gemm(dA, dB, dC, beta=p.beta, opts=opts)
        torch.cuda.synchronize()
        one = time.perf_counter() - t0
        reps = int(min(2000, max(20, 0.05 / max(one, 1e-6))))
        # the board idles while the oracle runs between cases: bring its clock back first
        settle(lambda: lib.gemm(dA, dB, dC, beta=p.beta, opts=opts), 5, 1.0)
        sec, _ = time_gemm(lib, dA, dB, dC, p.beta, opts, reps, max(5, reps // 10))
        eager_sec = sec
        if sec < 100e-6:
            sec = graph_seconds(lambda: lib.gemm(dA, dB, dC, beta=p.beta, opts=opts))
        pl = lib.plan(dA, dB, dC, opts)
        # the same operation through torch (FP16 operands, FP32 result), for context
        t_vendor = None
        if p.beta in (0.0, 1.0):
            vfn = ((lambda: torch.addmm(dC, dA, dB, out_dtype=torch.float32)) if p.beta
                   else (lambda: torch.mm(dA, dB, out_dtype=torch.float32)))
            try:
                settle(vfn, 5, 0.5)
                t_vendor = call_seconds(vfn)
            except (RuntimeError, TypeError):
                t_vendor = None
        waves, util = model.wave_utilization(model.tile_count(p.M, p.N, pl["bm"], pl["bn"]), 256)
        # oracle: whole problem when it takes under ~20 s on the host cores, else whole rows
        nrows = p.M if p.M * p.N * p.K <= 4096 ** 3 else max(threads, 512)
        t0 = time.perf_counter()
        oracle.gemm(A[:nrows], B, beta=p.beta, C=(C[:nrows] if C is not None else None))
        osec = (time.perf_counter() - t0) * p.M / nrows
        # one host thread: whole rows up to about 2e9 multiply-adds, scaled to all rows
        nrows1 = int(max(1, min(p.M, 2e9 // max(p.N * p.K, 1))))
        oracle.set_threads(1)
        t0 = time.perf_counter()
        oracle.gemm(A[:nrows1], B, beta=p.beta, C=(C[:nrows1] if C is not None else None))
        osec1 = (time.perf_counter() - t0) * p.M / nrows1
        oracle.set_threads(threads)
        rows.append({"workload": name + ("" if ld is None else " (lda=ldb=ldc=%d)" % ld)
                     + ("" if not opts else " " + ",".join("%s=%s" % kv for kv in opts.items())),
                     "M": p.M, "N": p.N, "K": p.K, "beta": p.beta, "gpu_us": sec * 1e6, "eager_us": eager_sec * 1e6,
                     "graph": eager_sec != sec, "reps": reps,
                     "tflops": flops / sec / 1e12, "frac_peak": flops / sec / 1e12 / PEAK_TFLOPS,
                     "tile": "%dx%dx%d" % (pl["bm"], pl["bn"], pl["bk"]), "grid": pl["grid"], "waves": waves, "util": util,
                     "direct_to_lds": bool(pl["vec_a"] and pl["vec_b"]),
                     "oracle_s": osec, "oracle_rows": int(nrows), "oracle1_s": osec1, "oracle1_rows": nrows1,
                     "speedup": osec / sec, "vendor_us": t_vendor * 1e6 if t_vendor else None})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del dA, dB, dC
        torch.cuda.empty_cache()
    print("| workload | M x N x K | beta | tile | tiles / waves on 256 CUs (util) | direct-to-LDS | GPU time per call "
          "| eager back-to-back | TFLOP/s | of 2516.6 | torch, same operation | oracle on %d host threads "
          "| oracle on 1 thread | GPU / oracle |" % threads)
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        osrc = "%.3g s%s" % (r["oracle_s"], "" if r["oracle_rows"] == r["M"] else " (from %d rows)" % r["oracle_rows"])
        osrc1 = "%.3g s%s" % (r["oracle1_s"], "" if r["oracle1_rows"] == r["M"] else " (from %d rows)" % r["oracle1_rows"])
        vend = "%.1f us (%.1f TF)" % (r["vendor_us"], 2.0 * r["M"] * r["N"] * r["K"] / r["vendor_us"] / 1e6) \
            if r["vendor_us"] else "--"
        print("| %s | %dx%dx%d | %g | %s | %d / %d (%.0f%%) | %s | %.1f us%s | %.1f us | %.1f | %.3f | %s | %s | %s | %.3g |"
              % (r["workload"], r["M"], r["N"], r["K"], r["beta"], r["tile"], r["grid"], r["waves"], 100 * r["util"],
                 "yes" if r["direct_to_lds"] else "no", r["gpu_us"], " (graph)" if r["graph"] else "", r["eager_us"],
                 r["tflops"], r["frac_peak"], vend, osrc, osrc1, r["speedup"]))
    return 0


def run_softmax(args):
    """The fused row softmax: the page's configuration and larger ones, against the HBM roofline.

    Each shape is timed twice: on one X/Y pair, called back to back (X, re-read every call, can stay in
    the GPU's 256 MB memory-attached cache while X and Y fit it), and cycling through enough pairs
    that the calls' footprint exceeds 1 GB, so every read comes from HBM (the roofline figure)."""
    import numpy as np
    import torch
    import dense_tiled_gemm_f16_amd as lib
    import oracle
    threads = oracle.max_threads()
    rows = []
    shapes = ((4096, 1024), (16384, 1024), (65536, 1024), (16384, 4096), (8192, 8192), (2048, 20000),
              (1024, 32768), (1024, 49152), (512, 65536), (256, 131072), (128, 262144),
              (16384, 8192),                                 # an input larger than the 256 MB cache
              (8192, 8191), (2048, 50257), (256, 131071))   # the last three: rows not 16-byte aligned
    if args.softmax_shapes:
        shapes = [tuple(int(v) for v in s.split("x")) for s in args.softmax_shapes]

    def time_calls(pairs, calls=20, reps=10, op=lib.softmax_rows):
        """Seconds per call: `calls` calls captured in a graph cycling through `pairs`, replayed."""
        for X, Y in pairs:
            op(X, Y)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in range(calls):
                X, Y = pairs[c % len(pairs)]
                op(X, Y)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (reps * calls)

    for M, N in shapes:
        rng = np.random.default_rng(2)              # the page's generator and seed for its 4096 x 1024 case
        x = rng.standard_normal((M, N)).astype(np.float32)
        X = torch.from_numpy(x).cuda()
        Y = torch.empty_like(X)
        sec = time_calls([(X, Y)])
        # more pairs (copies of X) until the footprint passes 1 GB; the graph cycles through them
        npair = max(2, -(-(1 << 30) // (2 * M * N * 4)))
        calls = max(20, npair)
        pairs = [(X, Y)] + [(X.clone(), torch.empty_like(X)) for _ in range(npair - 1)]
        sec_cold = time_calls(pairs, calls=calls, reps=max(1, 200 // calls))
        # the same bytes moved by a plain device copy (torch's copy kernel), same pairs: what HBM gives
        # a stream of one read and one write per element
        sec_copy = time_calls(pairs, calls=calls, reps=max(1, 200 // calls), op=lambda a, b: b.copy_(a))
        del pairs
        lib.softmax_rows(X, Y)
        torch.cuda.synchronize()
        out = Y.cpu().numpy()
        nr = min(M, 512)
        t0 = time.perf_counter()
        ref = oracle.softmax_rows(x[:nr])
        osec = (time.perf_counter() - t0) * M / nr
        err = float(np.max(np.abs(out[:nr] - ref)))
        alg = 2.0 * M * N * 4
        # up to 65536 elements stay in registers (81920 for 81921-138752 elements); beyond, 40448
        # more stay in LDS when the rows are 16-byte aligned (N % 4 == 0 here) and the rest is
        # read twice
        regs = 81920 if 81920 < N <= 138752 else 65536
        passes = 2 + max(0, N - regs - (40448 if N % 4 == 0 else 0)) / N
        rows.append((M, N, sec, sec_cold, sec_copy, npair, alg, passes, osec, nr, err))
        print(json.dumps({"softmax": [M, N], "us": sec * 1e6, "us_from_hbm": sec_cold * 1e6,
                          "GBps_from_hbm": alg / sec_cold / 1e9}), file=sys.stderr, flush=True)
        del X, Y
        torch.cuda.empty_cache()
    print("| M x N (FP32) | one X/Y pair: time per call | of 8 TB/s | X/Y pairs past 1 GB: time per call "
          "| algorithmic GB/s (2MN x 4 B) | of 8 TB/s | device copy of the same bytes | softmax / copy rate "
          "| passes over HBM | oracle on %d host threads | max abs error vs oracle |" % threads)
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for M, N, sec, sec_cold, sec_copy, npair, alg, passes, osec, nr, err in rows:
        print("| %d x %d | %.1f us | %.3f | %.1f us (%d pairs) | %.0f | %.3f | %.1f us (%.3f) | %.2f | %.2f | %.3g s%s "
              "| %.2e |" % (M, N, sec * 1e6, alg / sec / 8e12, sec_cold * 1e6, npair, alg / sec_cold / 1e9,
                            alg / sec_cold / 8e12, sec_copy * 1e6, alg / sec_copy / 8e12, sec_copy / sec_cold, passes,
                            osec, "" if nr == M else " (from %d rows)" % nr, err))
    return 0


LDS_PROBE_MODES = [
    (0, "A fragment, 64-byte rows", "none"), (1, "A fragment, 64-byte rows", "(r>>1)&3"),
    (2, "A fragment, 64-byte rows", "(r^r>>2)&3 (product, single-slice panels)"),
    (3, "A fragment, 128-byte rows (paired)", "none"), (4, "A fragment, 128-byte rows (paired)", "(r^r>>3)&7 (product)"),
    (5, "contiguous 1 KiB ds_read_b128 (reference)", "-"),
    (6, "B transposing read, 512-byte k rows", "none"), (7, "B transposing read, 512-byte k rows", "2(r&3) (product)"),
    (8, "contiguous 512 B ds_read_b64_tr_b16 (reference)", "-")]


def run_lds_probe(args):
    """LDS fragment-read rate of the product's read patterns under each swizzle (measurement library):
    256 workgroups of four waves, 16 reads per round, 4096 rounds; shader cycles per read per wave."""
    import ctypes
    import numpy as np
    import torch
    from dense_tiled_gemm_f16_amd import build as hb
    m = ctypes.CDLL(hb.MEASURE_LIB_PATH)
    m.gemm_f16_lds_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    m.gemm_f16_lds_read_probe.restype = ctypes.c_int
    grid, rounds = 256, 4096
    out = torch.zeros(grid * 4 * 2, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print("| access | swizzle key | cycles per read per wave (4 waves contending) | bytes per read |")
    print("|---|---|---|---|")
    for mode, what, key in LDS_PROBE_MODES:
        for _ in range(2):                          # the first launch warms the board; the second is kept
            rc = m.gemm_f16_lds_read_probe(out.data_ptr(), grid, mode, rounds, stream)
            if rc != 0:
                raise RuntimeError("lds probe launch failed (%d)" % rc)
            torch.cuda.synchronize()
        d = out.cpu().numpy().reshape(grid * 4, 2)
        cyc = float(np.median(d[:, 0])) / (rounds * 16)
        print("| %s | %s | %.1f | %d |" % (what, key, cyc, 512 if mode >= 6 else 1024), flush=True)
    return 0


# (KiB written into LDS per round, how, read set, what it stands for) of bench.py --lds-mix-probe; how:
# 0 direct-to-LDS loads, 1 ds_write_b128 from registers (no memory traffic), 2 global loads staged
# through registers, 3 half direct-to-LDS and half staged through registers
LDS_MIX_CASES = [
    (0, 0, 1, "16 KiB of ds_read_b128 only"),
    (0, 0, 2, "the 256x256 tile's NN fragment reads for one slice only (8 KiB b128 + 8 KiB transposing)"),
    (0, 0, 3, "the K-split tile's fragment reads for one slice only (4 KiB b128 + 4 KiB transposing)"),
    (8, 0, 0, "8 KiB of direct-to-LDS loads only"),
    (16, 0, 0, "16 KiB of direct-to-LDS loads only"),
    (8, 1, 0, "8 KiB of ds_write_b128 from registers only"),
    (8, 2, 0, "8 KiB staged through registers only (global loads, then ds_write_b128)"),
    (8, 0, 1, "8 KiB of direct-to-LDS loads + 16 KiB of ds_read_b128"),
    (8, 0, 2, "one slice of the 256x256 tile (NN): 8 KiB of direct-to-LDS loads + its 16 KiB of fragment reads"),
    (4, 0, 2, "4 KiB of direct-to-LDS loads + the 256x256 tile's 16 KiB of fragment reads"),
    (8, 1, 2, "8 KiB of ds_write_b128 from registers + the 256x256 tile's fragment reads"),
    (8, 2, 2, "8 KiB staged through registers + the 256x256 tile's fragment reads"),
    (8, 3, 2, "4 KiB direct-to-LDS + 4 KiB staged through registers + the 256x256 tile's fragment reads"),
    (8, 0, 3, "one slice of the K-split tile: 8 KiB of direct-to-LDS loads + its 8 KiB of fragment reads"),
    (8, 2, 3, "8 KiB staged through registers + the K-split tile's fragment reads"),
]
LDS_MIX_READ_BYTES = {0: 0, 1: 16384, 2: 16384, 3: 8192}


def run_lds_mix_probe(args):
    """LDS traffic of a main-loop slice without the matrix instructions (measurement library): 256
    workgroups of four waves, every wave running 2048 rounds of D KiB written into LDS (direct-to-LDS
    loads of 1 KiB, or staged through registers, from 64 KiB per workgroup: inside its XCD's L2, above
    the vector L1) and a set of fragment reads in the product's patterns; shader cycles per round per
    wave and the LDS bytes per cycle per CU."""
    import ctypes
    import numpy as np
    import torch
    from dense_tiled_gemm_f16_amd import build as hb
    m = ctypes.CDLL(hb.MEASURE_LIB_PATH)
    m.gemm_f16_lds_mix_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p]
    m.gemm_f16_lds_mix_probe.restype = ctypes.c_int
    grid, rounds, region = 256, 2048, 64 << 10
    src = torch.zeros(grid * region, dtype=torch.uint8, device="cuda")
    out = torch.zeros(grid * 4 * 2, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print("| per wave per round | written (KiB) | fragment reads (KiB) | cycles per round per wave "
          "| written bytes per cycle per CU | read bytes per cycle per CU | LDS bytes per cycle per CU |")
    print("|---|---|---|---|---|---|---|")
    for d, writer, kind, what in LDS_MIX_CASES:
        for _ in range(2):                          # the first launch warms the board; the second is kept
            rc = m.gemm_f16_lds_mix_probe(src.data_ptr(), src.numel(), region, out.data_ptr(), grid, d, writer,
                                          kind, rounds, stream)
            if rc != 0:
                raise RuntimeError("lds mix probe launch failed (%d)" % rc)
            torch.cuda.synchronize()
        cyc = float(np.median(out.cpu().numpy().reshape(grid * 4, 2)[:, 0])) / rounds
        ld, rd = 4 * d * 1024 / cyc, 4 * LDS_MIX_READ_BYTES[kind] / cyc
        print("| %s | %d | %d | %.0f | %.1f | %.1f | %.1f |" % (what, d, LDS_MIX_READ_BYTES[kind] // 1024, cyc, ld, rd,
                                                             ld + rd), flush=True)
    return 0


VMEM_PATTERNS = [(0, "contiguous 1 KiB (8 whole cache lines per load)"),
                 (1, "16x16x32 A fragment: 16 rows x 64 B per load"),
                 (2, "32x32x16 A fragment: 32 rows x 32 B per load"),
                 (3, "contiguous 1 KiB starting 2 bytes past a 16-byte boundary"),
                 (4, "contiguous 1 KiB starting 4 bytes past a 16-byte boundary"),
                 (5, "one 2-byte load per lane, 16 bytes apart"),
                 (6, "realigned chunks (2 bytes past a boundary): 16 bytes from the 4-byte boundary + the last element")]


def run_vmem_probe(args):
    """What the load path charges for MFMA fragments read straight from memory into registers
    (measurement library): 256 workgroups of four waves, each wave issuing 4095 rounds of 8
    global_load_dwordx4 over 64 KiB per workgroup (inside its XCD's L2, above the vector L1)."""
    import ctypes
    import numpy as np
    import torch
    from dense_tiled_gemm_f16_amd import build as hb
    m = ctypes.CDLL(hb.MEASURE_LIB_PATH)
    m.gemm_f16_vmem_pattern_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    m.gemm_f16_vmem_pattern_probe.restype = ctypes.c_int
    grid, rounds = 256, 4095
    src = torch.zeros(grid * (64 << 10) + 4096, dtype=torch.uint8, device="cuda")   # slack for the misaligned patterns
    out = torch.zeros(grid * 4 * 2, dtype=torch.int64, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print("| load pattern | cycles per load per wave (4 waves) | bytes per cycle per CU |")
    print("|---|---|---|")
    for pat, what in VMEM_PATTERNS:
        for _ in range(2):                          # the first launch warms the board; the second is kept
            rc = m.gemm_f16_vmem_pattern_probe(src.data_ptr(), src.numel(), out.data_ptr(), grid, pat, rounds, stream)
            if rc != 0:
                raise RuntimeError("vmem probe launch failed (%d)" % rc)
            torch.cuda.synchronize()
        cyc = float(np.median(out.cpu().numpy().reshape(grid * 4, 2)[:, 0])) / ((rounds - 1) * 8)
        print("| %s | %.1f | %.1f |" % (what, cyc, 4 * 1024 / cyc), flush=True)
    return 0


def run_latency_probe(args):
    """Latency of one 1 KiB direct-to-LDS load (global_load_lds_dwordx4, 64 lanes x 16 B), waited for
    before the next: L2 hits (a region per workgroup re-read after a warming pass: 1 MiB with 8
    workgroups, 64 KiB with 256 -- 2 MiB per XCD either way, inside its 4 MB L2 and above the 32 KiB
    vector L1) and HBM (a fresh window 64 KiB apart each time in a 1 GiB buffer).  8 one-wave
    workgroups (one per XCD) and 256 (one per CU)."""
    import ctypes
    import numpy as np
    import torch
    from dense_tiled_gemm_f16_amd import build as hb
    m = ctypes.CDLL(hb.MEASURE_LIB_PATH)
    m.gemm_f16_dma_latency_probe.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                             ctypes.c_void_p]
    m.gemm_f16_dma_latency_probe.restype = ctypes.c_int
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    print("| where the load is served | workgroups | loads timed per wave | cycles per load | ns per load "
          "| clock while probing |")
    print("|---|---|---|---|---|---|")
    for grid in (8, 256):
        region = (1 << 20) if grid == 8 else (64 << 10)
        cases = [("L2 (%d KiB per workgroup, after a warming pass)" % (region >> 10), 2048, region // 1024, 1024,
                  region, 1)]
        iters = 2048 if grid == 8 else 64
        cases.append(("HBM (fresh 1 KiB windows, 64 KiB apart)", iters, iters, 65536, iters * 65536, 0))
        for what, it, windows, stride, gstride, warm in cases:
            if (grid - 1) * gstride + (windows - 1) * stride + 1024 > nbytes:
                raise ValueError("probe would read past its buffer")
            out = torch.zeros(grid * 3, dtype=torch.int64, device="cuda")
            rc = m.gemm_f16_dma_latency_probe(src.data_ptr(), nbytes, out.data_ptr(), grid, it, windows, stride,
                                              gstride, warm, stream)
            if rc != 0:
                raise RuntimeError("latency probe launch failed (%d)" % rc)
            torch.cuda.synchronize()
            d = out.cpu().numpy().reshape(grid, 3).astype(np.float64)
            cyc = float(np.median(d[:, 0] / d[:, 2]))
            ns = float(np.median(d[:, 1] / d[:, 2])) * 10.0
            ghz = float(np.median(d[:, 0] / (d[:, 1] / 100e6))) / 1e9
            print("| %s | %d | %d | %.0f | %.0f | %.2f GHz |" % (what, grid, it, cyc, ns, ghz), flush=True)
    return 0


def run_phases(args, lib, gemm_call, pl, p):
    """Per-phase shader cycles of one call, from the measurement build whose kernels stamp s_memtime
    at their phase boundaries (libgemm_f16_phases.so; the product library has no stamps): entry to
    the end of the main loop's prologue, the main loop, the masked K tail, the epilogue; the shader
    clock of each workgroup; and, per CU, the gap between one tile's end and the next tile's start."""
    import ctypes
    import numpy as np
    import torch
    from dense_tiled_gemm_f16_amd import build as hb
    if pl["tile2"]:
        raise SystemExit("--phases takes single-launch calls only (this shape splits into two launches)")
    ph = ctypes.CDLL(hb.PHASES_LIB_PATH)
    setter = getattr(ph, "gemm_f16_phase_buffer_" + args.layout.lower())
    setter.argtypes = [ctypes.c_void_p]
    setter.restype = ctypes.c_int
    settle(gemm_call, 20, 0.5)
    buf = torch.zeros(pl["grid"] * 8, dtype=torch.int64, device="cuda")
    if setter(buf.data_ptr()) != 0:
        raise RuntimeError("gemm_f16_phase_buffer failed")
    gemm_call()
    torch.cuda.synchronize()
    setter(None)
    d = buf.cpu().numpy().reshape(pl["grid"], 8).astype(np.int64)
    assert np.all(d[:, 4] > d[:, 0]), "missing phase stamps"
    cyc = {"entry to the end of the prologue": d[:, 1] - d[:, 0], "main loop": d[:, 2] - d[:, 1],
           "masked K tail": d[:, 3] - d[:, 2], "epilogue": d[:, 4] - d[:, 3], "whole tile": d[:, 4] - d[:, 0]}
    secs = (d[:, 6] - d[:, 5]) / 100e6
    clock = (d[:, 4] - d[:, 0]) / secs / 1e9
    cu = (d[:, 7] >> 32) * 256 + ((d[:, 7] >> 8) & 0xFF)
    gaps = []
    for c in np.unique(cu):
        w = d[cu == c]
        w = w[np.argsort(w[:, 5])]
        gaps += list((w[1:, 5] - w[:-1, 6]) / 100e6 * float(np.median(clock)) * 1e9)
    span = (d[:, 6].max() - d[:, 5].min()) / 100e6
    total = float(np.median(cyc["whole tile"]))
    print("%s (%s), tile %dx%dx%d, %d workgroups on %d CUs; one call: %.1f us from the first entry to the last end, "
          "shader clock %.2f GHz (median over workgroups)\n" % (
              p.name, args.layout, pl["bm"], pl["bn"], pl["bk"], pl["grid"], len(np.unique(cu)), span * 1e6,
              float(np.median(clock))))
    print("| phase | median cycles | 10th percentile | 90th percentile | share of the median tile |")
    print("|---|---|---|---|---|")
    for k, v in cyc.items():
        print("| %s | %.0f | %.0f | %.0f | %.1f %% |" % (k, np.median(v), np.percentile(v, 10), np.percentile(v, 90),
                                                      100.0 * np.median(v) / total))
    if gaps:
        print("| gap to the next tile on the same CU | %.0f | %.0f | %.0f | |" % (
            np.median(gaps), np.percentile(gaps, 10), np.percentile(gaps, 90)))
    mfma = pl["bm"] * pl["bn"] * p.K * 2 / 4096.0
    print("\nIdeal matrix-core cycles per tile (2.BM.BN.K / 4096 FLOP per CU per cycle): %.0f; the median tile "
          "takes %.2fx that." % (mfma, total / mfma))
    return 0


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
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="minimum warm-up wall time before the timed window (the board's clock settles)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--group-m", type=int, default=0)
    ap.add_argument("--xcd-remap", type=int, default=-1)
    ap.add_argument("--path", type=int, choices=(0, 1), default=0,
                    help="1: every tile through the register-staged path (the path unaligned operands take)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--workload", default="accum8192")
    ap.add_argument("--shape", type=int, nargs=3, metavar=("M", "N", "K"),
                    help="GPU steps only, on an M x N x K product of N(0,1) inputs (seed 12, beta 0)")
    ap.add_argument("--layout", choices=("NN", "NT", "TN", "TT"), default="NN",
                    help="GPU steps only: A (first letter) and B (second) as given (N) or stored transposed (T)")
    ap.add_argument("--ld", type=int, default=0,
                    help="GPU steps only: leading dimension of A, B and C (rows padded to ld elements)")
    ap.add_argument("--configs", action="store_true")
    ap.add_argument("--splitk", action="store_true")
    ap.add_argument("--skinny", action="store_true")
    ap.add_argument("--skinny-shapes", nargs="+", metavar="MxNxK", default=None,
                    help="with --skinny: only these problems (e.g. 16x8192x28672)")
    ap.add_argument("--softmax", action="store_true")
    ap.add_argument("--softmax-shapes", nargs="+", metavar="MxN", default=None,
                    help="with --softmax: only these shapes (e.g. 256x131072)")
    ap.add_argument("--unaligned", action="store_true")
    ap.add_argument("--ksweep", action="store_true")
    ap.add_argument("--mfma-ceiling", action="store_true")
    ap.add_argument("--lds-probe", action="store_true")
    ap.add_argument("--phases", action="store_true",
                    help="per-phase cycles of one call of the chosen workload (measurement build)")
    ap.add_argument("--latency-probe", action="store_true")
    ap.add_argument("--lds-mix-probe", action="store_true")
    ap.add_argument("--vmem-probe", action="store_true")
    ap.add_argument("--power", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--variant", choices=("product", "noswizzle"), default="product",
                    help="noswizzle: time the measurement build without the LDS swizzle (same C ABI)")
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
    if args.variant == "noswizzle" or args.phases:
        from dense_tiled_gemm_f16_amd import build as hb
        lib.load(hb.PHASES_LIB_PATH if args.phases else hb.NOSWIZZLE_LIB_PATH)
        args.no_secondary = args.no_cpu_baseline = args.no_ceiling = True
    lib.load()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return 0
    if args.configs:
        return run_configs(args)
    if args.splitk:
        return run_splitk(args)
    if args.skinny:
        return run_skinny(args)
    if args.softmax:
        return run_softmax(args)
    if args.unaligned:
        return run_unaligned(args)
    if args.ksweep:
        return run_ksweep(args)
    if args.power:
        return run_power(args)
    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling()), flush=True)
        return 0
    if args.lds_probe:
        return run_lds_probe(args)
    if args.lds_mix_probe:
        return run_lds_mix_probe(args)
    if args.vmem_probe:
        return run_vmem_probe(args)
    if args.latency_probe:
        return run_latency_probe(args)

    opts = {"tile": args.tile, "group_m": args.group_m, "xcd_remap": args.xcd_remap, "path": args.path}
    if args.shape:
        from gemm_inputs import Problem
        p = Problem("shape%dx%dx%d" % tuple(args.shape), *args.shape, 12)
    else:
        p = PROBLEMS[args.workload]
    if args.workload != "accum8192" or args.shape or args.ld or args.layout != "NN":
        args.no_secondary = args.no_cpu_baseline = args.no_ceiling = True
    ta, tb = args.layout[0] == "T", args.layout[1] == "T"
    if (ta or tb) and args.ld:
        raise SystemExit("--layout and --ld do not combine")
    print("bench: generating %s inputs" % p.name, file=sys.stderr, flush=True)
    A, B, C = problem_arrays(p)
    if args.ld:
        if args.ld < max(p.K, p.N):
            raise SystemExit("--ld must be at least max(K, N)")
        dA = torch.zeros((p.M, args.ld), dtype=torch.float16, device="cuda")[:, :p.K]
        dB = torch.zeros((p.K, args.ld), dtype=torch.float16, device="cuda")[:, :p.N]
        dC = torch.zeros((p.M, args.ld), dtype=torch.float32, device="cuda")[:, :p.N]
        dA.copy_(torch.from_numpy(A))
        dB.copy_(torch.from_numpy(B))
        if C is not None:
            dC.copy_(torch.from_numpy(C))
    else:
        dA = torch.from_numpy(np.ascontiguousarray(A.T) if ta else A).cuda()
        dB = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).cuda()
        dC = torch.from_numpy(C).cuda() if C is not None else torch.zeros((p.M, p.N), dtype=torch.float32, device="cuda")
    # the plain product (one kernel, or two for a row/column split), whose launches the roofline times
    if ta or tb:
        gemm_call = lambda: lib.gemm(dA, dB, dC, beta=p.beta, opts=opts, trans_a=ta, trans_b=tb, splits=1)
    else:
        gemm_call = lambda: lib.gemm(dA, dB, dC, beta=p.beta, opts=opts, splits=1)
    plan = lib.plan(dA, dB, dC, opts, trans_a=ta, trans_b=tb)
    flops = 2.0 * p.M * p.N * p.K
    if args.phases:
        return run_phases(args, lib, gemm_call, plan, p)

    ceil_before = None
    if not args.no_ceiling:
        print("bench: measuring the matrix-core ceiling (before)", file=sys.stderr, flush=True)
        ceil_before = mfma_ceiling()
    print("bench: warming up (at least %d calls, %.1f s)" % (args.warmup, args.warmup_seconds), file=sys.stderr,
          flush=True)
    warm_calls, warm_s, warm_last = settle(gemm_call, args.warmup, args.warmup_seconds)
    print("bench: timing %d steps after %d warm-up calls (%.2f s)" % (args.steps, warm_calls, warm_s),
          file=sys.stderr, flush=True)
    sec, wall = time_calls(gemm_call, args.steps)
    tflops = flops / sec / 1e12

    out = {
        "metric": METRIC,
        "value": round(flops * args.steps / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls_run": warm_calls,
        "warmup_s": round(warm_s, 2),
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": ("D = A.B + C" if p.beta else "C = A.B") + ", M=%d N=%d K=%d, A,B fp16 N(0,1)%s, "
                               "fp32 accumulate" % (p.M, p.N, p.K, ", C fp32 N(0,1)" if p.beta else ""),
                   "M": p.M, "N": p.N, "K": p.K, "beta": p.beta, "seed": p.seed, "accumulate": "f32",
                   "tile": "%dx%d" % (plan["bm"], plan["bn"]), "bk": plan["bk"], "group_m": plan["group_m"],
                   "xcd_remap": plan["xcd_remap"], "grid": plan["grid"], "parallelism": "single GPU"},
    }
    if args.variant != "product":
        out["config"]["variant"] = args.variant
    if args.ld:
        out["config"]["ld"] = args.ld
    if args.layout != "NN":
        out["config"]["layout"] = args.layout
    main_line = args.variant == "product" and args.workload == "accum8192" and not args.shape and not args.ld
    traffic = read_traffic(flops) if main_line else None
    out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": round(PEAK_TFLOPS, 1),
                       "unit": "TFLOP/s", "frac": round(tflops / PEAK_TFLOPS, 4),
                       "traffic": traffic, "kernel_ms": round(sec * 1e3, 4),
                       "kernel": "gemm_f16_f32_kernel<Tile<%d,%d,...>>" % (plan["bm"], plan["bn"]),
                       "kernel_source_sha256": kernel_source_hash(),
                       "warmup_last_batch_ms": round(warm_last * 1e3, 4)}
    cycles = read_summary_value(COUNTER_SUMMARY, "grbm_cycles_per_xcd_per_dispatch") if main_line else None
    # The effective shader clock of the timed window: the kernel's GPU-active cycles per dispatch
    # (GRBM_GUI_ACTIVE per XCD, from the committed counter run of the same kernel source) over the
    # timed per-call duration.  A probe kernel run just outside the window reads the clock the
    # board returns to within microseconds of the matrix load stopping, not the GEMM's.
    out["roofline"]["clock_ghz_timed"] = round(cycles / sec / 1e9, 3) if cycles else None
    if not args.no_ceiling:
        print("bench: measuring the matrix-core ceiling (after)", file=sys.stderr, flush=True)
        ceil_after = mfma_ceiling()
        out["mfma_ceiling"] = {"before": ceil_before, "after": ceil_after,
                               "frac_before": round(tflops / ceil_before["tflops"], 4),
                               "frac_after": round(tflops / ceil_after["tflops"], 4)}

    if not args.no_secondary:
        # The same operation through torch (FP16 operands, FP32 result: addmm with out_dtype, the
        # vendor GEMM library behind torch), on the same operands, for context.
        if not args.shape and not args.ld and args.layout == "NN":
            t_vendor = vendor_seconds(dA, dB, dC, p.beta)
            if t_vendor:
                out["secondary"] = {"torch_same_op_tflops": round(flops / t_vendor / 1e12, 2),
                                    "torch_same_op_ms": round(t_vendor * 1e3, 4)}
        del dA, dB, dC
        torch.cuda.empty_cache()
        q = PROBLEMS["square4096"]
        A4, B4, _ = problem_arrays(q)
        dA4, dB4 = torch.from_numpy(A4).cuda(), torch.from_numpy(B4).cuda()
        dC4 = torch.empty((q.M, q.N), dtype=torch.float32, device="cuda")
        # The two orders alternate over five rounds (medians), so neither absorbs the clock change
        # that follows the 8192^3 run.  With the default 256x256 tile the 4096^3 grid is 256 tiles,
        # one wave on 256 CUs, so the order cannot change what a wave fetches; the forced 128x128
        # tile (1024 tiles, four waves) is where the grouped order can save traffic.
        f4 = 2.0 * q.M * q.N * q.K
        out.setdefault("secondary", {})["square4096_tile"] = "%dx%d" % tuple(lib.plan(dA4, dB4, dC4)[k]
                                                                              for k in ("bm", "bn"))
        for label, tile in (("", 0), ("_tile128", 2)):
            rounds_g, rounds_r = [], []
            for _ in range(5):
                rounds_g.append(time_gemm(lib, dA4, dB4, dC4, 0.0, {"group_m": 8, "tile": tile}, 20, 5)[0])
                rounds_r.append(time_gemm(lib, dA4, dB4, dC4, 0.0, {"group_m": 1, "xcd_remap": 0, "tile": tile},
                                          20, 5)[0])
            out["secondary"]["square4096%s_group_m8_tflops" % label] = round(f4 / statistics.median(rounds_g) / 1e12, 2)
            out["secondary"]["square4096%s_row_major_tflops" % label] = round(f4 / statistics.median(rounds_r) / 1e12, 2)
        del dA4, dB4, dC4

    if not args.no_cpu_baseline:
        print("bench: timing the oracle on the host cores", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(A, B, C, p.beta, args.cpu_budget)

    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
