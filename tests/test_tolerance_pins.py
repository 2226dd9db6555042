"""Pins for the parity rule itself (tests/tolerance.py), on the CPU.

06_triton_style.py (CS349E lecture 10, block programming), demo 4: a block kernel that forgets the
K mask reads the next row's data in its last K block; on the page it passes every shape whose
sizes are multiples of the block size and fails the others, which is why the test set must hold
ragged shapes.  Here that mistake is planted on the CPU -- the oracle is run on operands extended
the way the unmasked kernel reads them -- and the parity rule must reject it exactly where the
page says it shows.
"""
import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from tolerance import max_abs_err, tol_normal

BLOCK_K = 32


def unmasked_k_product(A, B, block=BLOCK_K):
    """What the kernel without the K mask computes: K padded up to a multiple of `block`, the extra
    A columns read from the flat array (the next row's elements) and the extra B rows read from
    the flat array past row K-1, clamped to the last element (the page clamps indices the same
    way so the simulation stays in bounds)."""
    M, K = A.shape
    N = B.shape[1]
    Kp = -(-K // block) * block
    if Kp == K:
        return oracle.gemm(A, B)
    fa, fb = A.ravel(), B.ravel()
    A_ext = np.empty((M, Kp), np.float16)
    B_ext = np.empty((Kp, N), np.float16)
    for i in range(M):
        idx = np.minimum(i * K + np.arange(Kp), fa.size - 1)
        A_ext[i] = fa[idx]
    for k in range(Kp):
        idx = np.minimum(k * N + np.arange(N), fb.size - 1)
        B_ext[k] = fb[idx]
    return oracle.gemm(A_ext, B_ext)


@pytest.mark.parametrize("shape", [(64, 64, 64), (128, 64, 96), (1, 1, 1), (17, 33, 65), (100, 70, 50),
                                   (64, 64, 40), (300, 200, 150), (129, 65, 33)])
def test_parity_rule_catches_missing_k_mask_exactly_on_ragged_k(shape):
    M, N, K = shape
    A, B, _ = normal_problem(M, N, K, 500 + K)
    ref = oracle.gemm(A, B)
    bug = unmasked_k_product(A, B)
    passes = max_abs_err(bug.astype(np.float32), ref) <= tol_normal(K)
    assert passes == (K % BLOCK_K == 0), (shape, max_abs_err(bug, ref))


def test_parity_rule_accepts_fp32_rounding_of_the_exact_result():
    """The rule accepts what a correct FP32-accumulating kernel can produce: the oracle's result
    rounded to FP32, and sequential FP32 accumulation, at K up to 4096."""
    for K in (16, 256, 4096):
        A, B, _ = normal_problem(48, 40, K, 900 + K)
        ref = oracle.gemm(A, B)
        assert max_abs_err(ref.astype(np.float32), ref) <= tol_normal(K)
        acc = np.zeros((48, 40), np.float32)
        for k in range(K):
            acc += A[:, k:k + 1].astype(np.float32) * B[k:k + 1, :].astype(np.float32)
        assert max_abs_err(acc, ref) <= tol_normal(K)
