"""Build the gfx950 library libgemm_f16.so in place (hipcc; no torch involvement).

    python -m dense_tiled_gemm_f16_amd.build          # writes dense_tiled_gemm_f16_amd/libgemm_f16.so

Flags: -O3 for gfx950 only; packed-FP32 instructions disabled (-packed-fp32-ops), so the
compiler never emits v_pk_{add,mul,fma}_f32.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libgemm_f16.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, f) for f in ("gemm_f16_f32.hip", "splitk_reduce.hip", "gemm_api.hip", "softmax_rows.hip")]
# Measurement-only library (the board's sustained matrix-core ceiling), kept out of the product.
CEILING_LIB_PATH = os.path.join(PKG, "libgemm_f16_ceiling.so")
CEILING_SOURCES = [os.path.join(CSRC, "mfma_ceiling.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def compile_flags(extra: list[str] | None = None) -> list[str]:
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + INCLUDE, "-I" + CSRC] + (extra or [])


def build(out: str = LIB_PATH, extra: list[str] | None = None, verbose: bool = False,
          sources: list[str] | None = None) -> str:
    """Compile the HIP sources (the product library by default) into one shared library; returns its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags(extra) + ["-shared"] + (sources or SOURCES) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def emit_asm(out_dir: str, extra: list[str] | None = None) -> list[str]:
    """Write the gfx950 assembly of each source (for inspection of this build's own code)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src in SOURCES:
        base = os.path.splitext(os.path.basename(src))[0]
        dst = os.path.join(out_dir, base + ".s")
        cmd = [hipcc()] + compile_flags(extra) + ["--offload-device-only", "-S", src, "-o", dst]
        subprocess.run(cmd, check=True)
        outs.append(dst)
    return outs


def build_ceiling(verbose: bool = False) -> str:
    """Compile the measurement-only matrix-core ceiling library."""
    return build(CEILING_LIB_PATH, verbose=verbose, sources=CEILING_SOURCES)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_ceiling(verbose="-v" in sys.argv))
