"""Seeded synthetic inputs for the FP16 -> FP32 matrix product.

This module is shared by the oracle side (tests, the CPU baseline) and the GPU side (tests, bench);
it draws random numbers and nothing else -- no part of the product is computed here.

Recipe (the pages' generator idiom, 04_tensor_cores.py demos 1-2 and 06_triton_style.py demo 4):
``rng = numpy.random.default_rng(seed)``; ``A = rng.standard_normal((M, K)).astype(float16)``;
``B = rng.standard_normal((K, N)).astype(float16)``; and, when the accumulate form D = A.B + C is
used, ``C = rng.standard_normal((M, N)).astype(float32)`` -- drawn in that order.  ``astype``
rounds to nearest even.  The pages measure on no public dataset; these draws stand in for the
N(0, 1) matrices their demos use.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Problem:
    name: str
    M: int
    N: int
    K: int
    seed: int
    beta: float = 0.0


# The workloads: one small square case, ragged edges, the wave-quantization pair, the
# launch-order comparison and the full accumulate form.
PROBLEMS = {
    "square256": Problem("square256", 256, 256, 256, 0),
    "ragged300x200x150": Problem("ragged300x200x150", 300, 200, 150, 1),
    "ragged129x65x33": Problem("ragged129x65x33", 129, 65, 33, 2),
    "skinny1x1000x64": Problem("skinny1x1000x64", 1, 1000, 64, 3),
    "square1792": Problem("square1792", 1792, 1792, 1792, 4),
    "square1793": Problem("square1793", 1793, 1793, 1793, 5),
    "square4096": Problem("square4096", 4096, 4096, 4096, 6),
    "accum8192": Problem("accum8192", 8192, 8192, 8192, 7, beta=1.0),
}


def normal_problem(M: int, N: int, K: int, seed: int, with_c: bool = False):
    """(A fp16 M x K, B fp16 K x N, C fp32 M x N or None), N(0,1) draws in the order A, B, C."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((M, K)).astype(np.float16)
    B = rng.standard_normal((K, N)).astype(np.float16)
    C = rng.standard_normal((M, N)).astype(np.float32) if with_c else None
    return A, B, C


def problem_arrays(p: Problem):
    return normal_problem(p.M, p.N, p.K, p.seed, with_c=(p.beta != 0.0))


def integer_problem(M: int, N: int, K: int, seed: int, lo: int = -2, hi: int = 2, with_c: bool = False):
    """Integer-valued entries in [lo, hi]; with small K every partial sum is an exactly
    representable integer in FP32, so any summation order gives the same bits."""
    rng = np.random.default_rng(seed)
    A = rng.integers(lo, hi + 1, size=(M, K)).astype(np.float16)
    B = rng.integers(lo, hi + 1, size=(K, N)).astype(np.float16)
    C = rng.integers(lo, hi + 1, size=(M, N)).astype(np.float32) if with_c else None
    return A, B, C


def subnormal_problem(M: int, N: int, K: int, seed: int):
    """A holds binary16 subnormals (|x| < 2^-14) and B holds values around 2^10, so every
    product is a normal FP32 number that a flush-to-zero of the inputs would lose."""
    rng = np.random.default_rng(seed)
    frac = rng.integers(1, 1024, size=(M, K)).astype(np.uint16)
    sign = (rng.integers(0, 2, size=(M, K)).astype(np.uint16) << 15)
    A = (frac | sign).view(np.float16)
    B = (rng.standard_normal((K, N)) * 1024.0).astype(np.float16)
    return A, B, None


def padded(x: np.ndarray, ld: int, fill: float = np.nan) -> np.ndarray:
    """Copy a 2-D array into a buffer whose rows are ``ld`` elements long (padding = ``fill``);
    return the view of the logical part (row stride ld)."""
    rows, cols = x.shape
    if ld < cols:
        raise ValueError("ld < cols")
    buf = np.full((max(rows, 1), ld), fill, dtype=x.dtype)
    buf[:rows, :cols] = x
    return buf[:rows, :cols]
