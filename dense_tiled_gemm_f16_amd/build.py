"""Build the gfx950 library libgemm_f16.so in place (hipcc; no torch involvement).

    python -m dense_tiled_gemm_f16_amd.build          # writes dense_tiled_gemm_f16_amd/libgemm_f16.so

Flags: -O3 for gfx950 only; packed-FP32 instructions disabled (-packed-fp32-ops), so the
compiler never emits v_pk_{add,mul,fma}_f32.

The product kernels (gemm_f16_f32.hip) are compiled as four objects, one per operand layout
(-DGEMM_F16_TA/TB), in parallel with the other sources, then linked into one shared library with
-Bsymbolic (the entry points call each other inside the library, never through another library
that exports the same names).  Besides the product library, the build writes two measurement
libraries that the product never loads:
  - libgemm_f16_measure.so: the board's sustained matrix-core ceiling, the LDS fragment-read
    microbenchmark and the direct-to-LDS load latency probe;
  - libgemm_f16_noswizzle.so: the same C ABI built with -DGEMM_F16_SWIZZLE=0 (LDS panel rows kept
    in order); tests check it gives the same bits, and profiles compare its LDS counters;
  - libgemm_f16_phases.so: the same C ABI whose kernels stamp the shader clock at their phase
    boundaries (-DGEMM_F16_PHASES=1 on the kernel objects; gemm_f16_phase_buffer_<layout> sets where).
Identical compile jobs are shared between the libraries.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgemm_f16.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
KERNEL_SOURCE = os.path.join(CSRC, "gemm_f16_f32.hip")
OTHER_SOURCES = [os.path.join(CSRC, f) for f in ("splitk_reduce.hip", "gemm_api.hip", "softmax_rows.hip")]
SOURCES = [KERNEL_SOURCE] + OTHER_SOURCES
LAYOUTS = ((0, 0), (0, 1), (1, 0), (1, 1))
# Measurement-only libraries, kept out of the product.
MEASURE_LIB_PATH = os.path.join(PKG, "libgemm_f16_measure.so")
MEASURE_SOURCES = [os.path.join(CSRC, "mfma_ceiling.hip"), os.path.join(CSRC, "probes.hip")]
NOSWIZZLE_LIB_PATH = os.path.join(PKG, "libgemm_f16_noswizzle.so")
PHASES_LIB_PATH = os.path.join(PKG, "libgemm_f16_phases.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def compile_flags(extra: list[str] | None = None) -> list[str]:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC] + (extra or [])


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        if os.environ.get(var, "").isdigit():
            return max(1, min(16, int(os.environ[var])))
    return max(1, min(16, os.cpu_count() or 1))


def _units(extra: list[str] | None, sources: list[str], kernel_extra: list[str] | None = None,
           all_layouts: bool = False) -> list[tuple[str, list[str]]]:
    """(source, flags) of every object: the kernel source once per operand layout (kernel_extra: more
    flags for the A-and-B-as-given kernel object, or for every kernel object with all_layouts)."""
    units = []
    for src in sources:
        if src == KERNEL_SOURCE:
            for ta, tb in LAYOUTS:
                more = (kernel_extra or []) if (all_layouts or (ta, tb) == (0, 0)) else []
                units.append((src, compile_flags((extra or []) + more + ["-DGEMM_F16_TA=%d" % ta,
                                                                         "-DGEMM_F16_TB=%d" % tb])))
        else:
            units.append((src, compile_flags(extra)))
    return units


def build_many(targets: list[tuple], verbose: bool = False) -> list[str]:
    """Build several shared libraries, every distinct object of all of them compiled once, in
    parallel.  targets: (output path, extra flags, sources[, extra kernel-object flags[, all layouts]])."""
    with tempfile.TemporaryDirectory(prefix="gemm_f16_build_") as tmpdir:
        jobs, links, seen = [], [], {}
        for target in targets:
            out, extra, sources = target[:3]
            kernel_extra = target[3] if len(target) > 3 else None
            all_layouts = target[4] if len(target) > 4 else False
            objs = []
            for src, flags in _units(extra, sources, kernel_extra, all_layouts):
                key = (src, tuple(flags))
                if key not in seen:
                    seen[key] = os.path.join(tmpdir, "u%d_%s.o" % (len(seen), os.path.splitext(os.path.basename(src))[0]))
                    jobs.append([hipcc()] + flags + ["-c", src, "-o", seen[key]])
                objs.append(seen[key])
            links.append((out, objs))
        with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as pool:
            for cmd, rc in zip(jobs, pool.map(lambda c: _run(c, verbose), jobs)):
                if rc != 0:
                    raise subprocess.CalledProcessError(rc, cmd)
        done = []
        for out, objs in links:
            tmp = out + ".tmp%d" % os.getpid()
            cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-Wl,-Bsymbolic"] + objs + ["-o", tmp]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            os.replace(tmp, out)
            done.append(out)
        return done


def _run(cmd: list[str], verbose: bool) -> int:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd).returncode


def build(out: str = LIB_PATH, extra: list[str] | None = None, verbose: bool = False,
          sources: list[str] | None = None) -> str:
    """Compile the HIP sources (the product library by default) into one shared library; returns its path."""
    return build_many([(out, extra, sources or SOURCES)], verbose)[0]


def build_all(verbose: bool = False) -> list[str]:
    """The product library and the measurement libraries, in one parallel build."""
    return build_many([(LIB_PATH, None, SOURCES),
                       (NOSWIZZLE_LIB_PATH, ["-DGEMM_F16_SWIZZLE=0"], SOURCES),
                       (PHASES_LIB_PATH, None, SOURCES, ["-DGEMM_F16_PHASES=1"], True),
                       (MEASURE_LIB_PATH, None, MEASURE_SOURCES)], verbose)


def emit_asm(out_dir: str, extra: list[str] | None = None, sources: list[str] | None = None) -> list[str]:
    """Write the gfx950 assembly of each object (for inspection of this build's own code)."""
    os.makedirs(out_dir, exist_ok=True)
    jobs, outs = [], []
    for ui, (src, flags) in enumerate(_units(extra, sources or SOURCES)):
        base = os.path.splitext(os.path.basename(src))[0]
        dst = os.path.join(out_dir, "%s_%d.s" % (base, ui))
        jobs.append([hipcc()] + flags + ["--offload-device-only", "-S", src, "-o", dst])
        outs.append(dst)
    with concurrent.futures.ThreadPoolExecutor(max_workers=_jobs()) as pool:
        for cmd, rc in zip(jobs, pool.map(lambda c: _run(c, False), jobs)):
            if rc != 0:
                raise subprocess.CalledProcessError(rc, cmd)
    return outs


def build_measure(verbose: bool = False) -> str:
    """Compile the measurement-only library (ceiling and probes)."""
    return build(MEASURE_LIB_PATH, verbose=verbose, sources=MEASURE_SOURCES)


if __name__ == "__main__":
    for path in build_all(verbose="-v" in sys.argv):
        print(path)
