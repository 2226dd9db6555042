"""Comparison rules shared by the parity tests (test helpers, not part of either implementation).

- N(0,1) inputs: max |C_gpu - C_oracle| <= 1e-4 * sqrt(K) (the acceptance bound for this path),
  and <= 1e-5 for a single 16x16x16 tile.
- Any inputs: the a-priori bound for FP32 accumulation in any order,
  |err| <= gamma_K * sum_k |a_ik b_kj| + 2u |beta c_ij|, gamma_K = K u / (1 - K u), u = 2^-24,
  plus a final FP32 rounding of the result.
- Integer-valued inputs whose partial sums are exact in FP32: bitwise equality.
"""
import math

import numpy as np

U32 = 2.0 ** -24


def tol_normal(K: int) -> float:
    return 1e-4 * math.sqrt(max(K, 1))


TOL_TILE16 = 1e-5


def max_abs_err(c_gpu: np.ndarray, d_oracle: np.ndarray) -> float:
    if c_gpu.size == 0:
        return 0.0
    return float(np.max(np.abs(c_gpu.astype(np.float64) - d_oracle)))


def fp32_bound(A: np.ndarray, B: np.ndarray, beta: float = 0.0, C: np.ndarray | None = None) -> np.ndarray:
    """Element-wise a-priori error bound for an FP32-accumulated product (any summation order)."""
    K = A.shape[1]
    absprod = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    g = K * U32 / (1 - K * U32) if K > 0 else 0.0
    bound = g * absprod
    if beta != 0.0 and C is not None:
        bound = bound + 2 * U32 * abs(beta) * np.abs(C.astype(np.float64))
    # final rounding of the stored FP32 value
    return bound + U32 * (absprod + (abs(beta) * np.abs(C.astype(np.float64)) if (beta != 0.0 and C is not None) else 0.0))
