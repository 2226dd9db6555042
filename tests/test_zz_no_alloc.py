"""gemm_f16_f32_splitk_noalloc: split-K with its partial products in the library's fixed scratch
(for callers that cannot allocate).  Through the C ABI, against gemm_f16_f32_splitk with a caller
workspace (the same kernels and split count, so the same bits) and against the oracle; two calls
in a row, the second smaller, so the scratch holds the first call's partials when the second
starts; a problem past the scratch limit is refused before any GPU work and leaves C alone."""
import numpy as np
import pytest

import oracle
from gemm_inputs import normal_problem
from tolerance import max_abs_err, tol_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dense_tiled_gemm_f16_amd as lib
    lib.load()
    yield


def _with_workspace(A, B, C, beta, splits, ta, tb):
    from gpu_helpers import run
    return run(A, B, C, beta=beta, splits=splits, trans_a=ta, trans_b=tb)


def _noalloc(A, B, C, beta, splits, ta, tb):
    """gemm_f16_f32_splitk_noalloc through the C ABI on guarded device buffers."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    from gpu_helpers import DevMat
    M, K = A.shape
    N = B.shape[1]
    dA = DevMat(np.ascontiguousarray(A.T) if ta else A)
    dB = DevMat(np.ascontiguousarray(B.T) if tb else B)
    dC = DevMat((C if C is not None else np.full((M, N), np.nan, np.float32)).astype(np.float32))
    rc = lib.gemm_f16_f32_splitk_noalloc(ta, tb, M, N, K, dA.ptr, dA.ld, dB.ptr, dB.ld, dC.ptr, dC.ld, float(beta),
                                         splits, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.gemm_f16_f32_strerror(rc)
    torch.cuda.synchronize()
    assert dC.outside_untouched() and dA.outside_untouched() and dB.outside_untouched()
    return dC.read()


def test_noalloc_matches_caller_workspace_two_calls():
    import dense_tiled_gemm_f16_amd as lib
    cases = [((512, 768, 16384), 8, 1.0, False, False, 3001),    # 8 x 512 x 768 x 4 B = 12 MiB of partials
             ((300, 200, 4160), 4, 0.0, True, False, 3002)]      # then smaller, ragged, A transposed
    for (M, N, K), splits, beta, ta, tb, seed in cases:
        assert lib.gemm_f16_f32_splitk_workspace(M, N, splits) <= lib._abi.SCRATCH_BYTES
        print("case noalloc", (M, N, K), splits, beta, ta, tb, flush=True)
        A, B, C = normal_problem(M, N, K, seed, with_c=True)
        Cin = C if beta else None
        ref = _with_workspace(A, B, Cin, beta, splits, ta, tb)
        out = _noalloc(A, B, Cin, beta, splits, ta, tb)
        assert np.array_equal(out, ref)
        assert max_abs_err(out, oracle.gemm(A, B, beta=beta, C=Cin)) <= tol_normal(K)


def test_noalloc_refuses_past_the_scratch_and_leaves_c_alone():
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M = N = 2048
    K = 8192
    splits = 4                                   # 4 x 2048 x 2048 x 4 B = 64 MiB > 32 MiB
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    B = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    C = torch.full((M, N), 7.0, device="cuda")
    rc = lib.gemm_f16_f32_splitk_noalloc(0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N, 0.0,
                                         splits, torch.cuda.current_stream().cuda_stream)
    assert rc == -9 and "scratch" in lib.gemm_f16_f32_strerror(rc)
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())
