"""GPU parity of split-K (gemm_f16_f32_splitk): K cut into ranges computed by separate workgroups,
the partial products summed in a fixed order by a second kernel.  Same bars as the unsplit call:
max |C_gpu - C_oracle| <= 1e-4 sqrt(K) for N(0,1) inputs, bitwise for integer-valued inputs.  The
workspace starts NaN-filled inside guard bands, so a partial product that is read but never written,
or a write outside the workspace or C, is detected."""
import sys

import numpy as np
import pytest

import oracle
from gemm_inputs import integer_problem, normal_problem
from tolerance import max_abs_err, tol_normal

pytestmark = pytest.mark.gpu

TILES = {"256x256": 1, "128x128": 2, "64x64": 3, "256x128": 4, "128x128k4": 5}
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import dense_tiled_gemm_f16_amd as lib
    lib.load()
    yield


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(C, D, K):
    assert np.all(np.isfinite(C)), "non-finite output"
    err = max_abs_err(C, D)
    assert err <= tol_normal(K), (err, tol_normal(K))


@pytest.mark.parametrize("shape,splits", [((256, 256, 8192), 8), ((300, 200, 4000), 3), ((129, 65, 1000), 7),
                                          ((1, 1000, 5000), 5), ((64, 64, 16384), 16), ((100, 70, 100), 64),
                                          ((513, 257, 2047), 4)])
@pytest.mark.parametrize("tile", list(TILES))
def test_splitk_every_tile(shape, splits, tile):
    """Split counts that divide K, that leave a short last range, and that exceed K / BK (the call
    then uses fewer ranges); beta = 1 with a random C."""
    from gpu_helpers import run
    M, N, K = shape
    _say("case splitk", shape, splits, tile)
    A, B, C = normal_problem(M, N, K, 2100 + M + splits, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    _check(run(A, B, C, beta=1.0, opts={"tile": TILES[tile]}, splits=splits), D, K)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(256, 256, 4096), (129, 65, 1000), (77, 1000, 3000)])
def test_splitk_layouts(ta, tb, shape):
    from gpu_helpers import run
    M, N, K = shape
    _say("case splitk layout", ta, tb, shape)
    A, B, C = normal_problem(M, N, K, 2200 + M, with_c=True)
    D = oracle.gemm(A, B, beta=0.5, C=C)
    _check(run(A, B, C, beta=0.5, trans_a=ta, trans_b=tb, splits=6), D, K)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_splitk_padded_unaligned_and_register_path(ta, tb):
    """Padded leading dimensions, operands off 16-byte alignment (register-staged loads) and the
    forced register path, each split."""
    from gpu_helpers import run
    M, N, K = 200, 150, 2000
    _say("case splitk padded", ta, tb)
    A, B, C = normal_problem(M, N, K, 2300, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    lda = (M if ta else K) + 9
    ldb = (K if tb else N) + 5
    _check(run(A, B, C, beta=1.0, lda=lda, ldb=ldb, ldc=N + 3, offs=(1, 3, 1), trans_a=ta, trans_b=tb, splits=5),
           D, K)
    _check(run(A, B, C, beta=1.0, opts={"path": 1}, trans_a=ta, trans_b=tb, splits=5), D, K)


@pytest.mark.parametrize("tile", list(TILES))
def test_splitk_integer_inputs_bitwise(tile):
    """Integer-valued operands: every partial sum and the sum of partials are exact in FP32."""
    from gpu_helpers import run
    A, B, C = integer_problem(257, 263, 3000, 2400, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    out = run(A, B, C, beta=1.0, opts={"tile": TILES[tile]}, splits=9)
    assert np.array_equal(out, D.astype(np.float32))


def test_splitk_deterministic_and_one_split_is_the_plain_call():
    from gpu_helpers import run
    A, B, _ = normal_problem(192, 320, 6000, 2500)
    a = run(A, B, splits=12)
    b = run(A, B, splits=12)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(run(A, B, splits=1).view(np.uint32), run(A, B).view(np.uint32))
    _check(a, oracle.gemm(A, B), 6000)


def test_splitk_workspace_errors_and_k_zero():
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M, N, K = 64, 64, 4096
    A = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    B = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    need = lib.gemm_f16_f32_splitk_workspace(M, N, 4)
    assert need == 4 * M * N * 4
    W = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (0, 0, M, N, K, A.data_ptr(), K, B.data_ptr(), N, C.data_ptr(), N, 1.0, 4)
    assert lib.gemm_f16_f32_splitk(*args, W.data_ptr(), need - 4, s) == -8
    assert lib.gemm_f16_f32_splitk(*args, None, need, s) == -8
    assert lib.gemm_f16_f32_splitk(*args, W.data_ptr() + 4, need, s) == -7
    assert lib.gemm_f16_f32_splitk(*args[:-1], 0, W.data_ptr(), need, s) == -4
    assert lib.gemm_f16_f32_splitk(*args[:-1], 1025, W.data_ptr(), need, s) == -4
    # K = 0: C <- beta * C with no workspace needed
    assert lib.gemm_f16_f32_splitk(0, 0, M, N, 0, A.data_ptr(), 1, B.data_ptr(), N, C.data_ptr(), N, 0.5, 4,
                                   None, 0, s) == 0
    torch.cuda.synchronize()
    assert torch.all(C == 1.5)


def test_splitk_full_size_deep_k_sampled():
    """A deep-K problem with few output tiles (512 x 512 x 65536) at full size, split 32 ways and
    the library's own way; stratified rows and columns (tests/sampling.py: every output tile, band
    and lane row) against the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    from sampling import strata
    M, N, K = 512, 512, 65536
    g = torch.Generator().manual_seed(2600)
    A = torch.randn((M, K), generator=g).half()
    B = torch.randn((K, N), generator=g).half()
    An, Bn = A.numpy(), B.numpy()
    dA, dB = A.cuda(), B.cuda()
    rows, cols = strata(M), strata(N)
    ref_rows = oracle.gemm(An[rows], Bn)
    ref_cols = oracle.gemm(An, np.ascontiguousarray(Bn[:, cols]))
    for splits in (32, None):      # None: the library's own split count
        C = torch.empty((M, N), dtype=torch.float32, device="cuda")
        lib.gemm_splitk(dA, dB, C, splits=splits)
        torch.cuda.synchronize()
        out = C.cpu().numpy()
        assert np.all(np.isfinite(out))
        assert max_abs_err(out[rows], ref_rows) <= tol_normal(K), splits
        assert max_abs_err(out[:, cols], ref_cols) <= tol_normal(K), splits


@pytest.mark.parametrize("shape,beta,tb", [((1, 4096, 4096), 0.0, False), ((16, 8192, 8192), 1.0, False),
                                           ((16, 8192, 8192), 0.0, True), ((8, 5120, 13824), 0.0, False),
                                           ((64, 1024, 32768), 1.0, False), ((8192, 64, 8192), 0.0, False),
                                           ((3, 2000, 9001), 0.5, True), ((1, 16384, 4096), 0.0, False)])
def test_library_call_on_skinny_problems(shape, beta, tb):
    """gemm() with the library's choice on skinny problems (a few rows or columns, long K): split-K
    wherever the cost model prefers it -- every shape here but the last, whose plain grid already
    fills the chip -- with the workspace from torch, against the oracle on stratified rows (every
    row when there are few)."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    from sampling import strata
    M, N, K = shape
    _say("case library call skinny", shape, beta, tb)
    s = lib.gemm_f16_f32_splitk_choose(M, N, K)
    assert (s > 1) == (shape != (1, 16384, 4096)), s
    A, B, C = normal_problem(M, N, K, 2700 + M + N, with_c=True)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).cuda()
    dC = torch.from_numpy(C).cuda()
    lib.gemm(dA, dB, dC, beta=beta, trans_b=tb)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    assert np.all(np.isfinite(out)), "non-finite output"
    rows = strata(M) if M > 256 else np.arange(M)
    ref = oracle.gemm(np.ascontiguousarray(A[rows]), B, beta=beta, C=np.ascontiguousarray(C[rows]))
    assert max_abs_err(out[rows], ref) <= tol_normal(K)
