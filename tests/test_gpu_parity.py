"""GPU parity: the HIP library against the FP64 oracle, element by element, on the same seeded inputs.

Bars: max |C_gpu - C_oracle| <= 1e-4 sqrt(K) for N(0,1) inputs (1e-5 on single 16x16x16 tiles);
bitwise equality for integer-valued inputs (every partial sum exact in FP32); the a-priori FP32
accumulation bound for other distributions.  Operands sit inside NaN-filled padding and guard
bands, so a read outside A or B turns outputs into NaN and a write outside C is detected.
"""
import sys

import numpy as np
import pytest

import oracle
from gemm_inputs import PROBLEMS, integer_problem, normal_problem, problem_arrays, subnormal_problem
from tolerance import TOL_TILE16, fp32_bound, max_abs_err, tol_normal

pytestmark = pytest.mark.gpu

TILES = {"256x256": 1, "128x128": 2, "64x64": 3, "256x128": 4, "128x128k4": 5}


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


def _check_normal(C, D, K, tol=None):
    tol = tol_normal(K) if tol is None else tol
    assert np.all(np.isfinite(C)), "non-finite output (read outside an operand?)"
    err = max_abs_err(C, D)
    assert err <= tol, (err, tol)
    return err


# ---------------------------------------------------------------- workload shapes
@pytest.mark.parametrize("name", ["square256", "ragged300x200x150", "ragged129x65x33", "skinny1x1000x64",
                                  "square1792", "square1793"])
def test_workload_shapes(name):
    from gpu_helpers import run
    p = PROBLEMS[name]
    _say("case", name)
    A, B, C = problem_arrays(p)
    D = oracle.gemm(A, B)
    _check_normal(run(A, B), D, p.K)


@pytest.mark.parametrize("shape", [(64, 64, 64), (128, 64, 96), (1, 1, 1), (17, 33, 65), (100, 70, 50),
                                   (64, 64, 40), (1000, 1100, 700), (513, 257, 191), (2, 3, 1000)])
@pytest.mark.parametrize("tile", list(TILES))
def test_edge_shapes_every_tile(shape, tile):
    """The pages' edge-shape set (prime, off-by-one and tiny sizes) plus several-tile ragged
    shapes, on every tile configuration."""
    from gpu_helpers import run
    M, N, K = shape
    _say("case", shape, tile)
    A, B, _ = normal_problem(M, N, K, 100 + M + N + K)
    D = oracle.gemm(A, B)
    _check_normal(run(A, B, opts={"tile": TILES[tile]}), D, K)


@pytest.mark.parametrize("shape", [(256, 256, 256), (1000, 1100, 704), (512, 768, 96), (300, 200, 150)])
@pytest.mark.parametrize("tile", list(TILES))
def test_register_staged_path_every_tile(shape, tile):
    """The register-staged path (the one unaligned operands take) forced on every tile, here also
    on aligned, full tiles."""
    from gpu_helpers import run
    M, N, K = shape
    _say("case", shape, tile, "register path")
    A, B, C = normal_problem(M, N, K, 900 + M + N + K, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    _check_normal(run(A, B, C, beta=1.0, opts={"tile": TILES[tile], "path": 1}), D, K)


def test_single_16x16x16_tiles():
    from gpu_helpers import run
    for seed in range(8):
        A, B, C = normal_problem(16, 16, 16, 300 + seed, with_c=True)
        D = oracle.gemm(A, B, beta=1.0, C=C)
        _check_normal(run(A, B, C, beta=1.0), D, 16, tol=TOL_TILE16)


# ---------------------------------------------------------------- exactness
@pytest.mark.parametrize("shape", [(257, 263, 129), (512, 512, 512), (33, 1000, 70), (640, 384, 1024)])
@pytest.mark.parametrize("tile", list(TILES))
def test_integer_inputs_bitwise(shape, tile):
    """Integer entries in [-2, 2]: every partial sum is an integer below 2^24, so the FP32 result
    is exact whatever the summation order and must equal the oracle bit for bit."""
    from gpu_helpers import run
    M, N, K = shape
    A, B, C = integer_problem(M, N, K, 7 + M, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    out = run(A, B, C, beta=1.0, opts={"tile": TILES[tile]})
    assert np.array_equal(out.astype(np.float64), D)


def test_subnormal_inputs_not_flushed():
    from gpu_helpers import run
    A, B, _ = subnormal_problem(130, 70, 200, 9)
    D = oracle.gemm(A, B)
    out = run(A, B)
    assert np.all(np.abs(out.astype(np.float64) - D) <= fp32_bound(A, B))
    assert np.max(np.abs(D)) > 1e-3       # a flush of the inputs would give all zeros


# ---------------------------------------------------------------- beta and degenerate sizes
@pytest.mark.parametrize("beta", [1.0, 0.5, -2.0])
def test_beta_accumulate(beta):
    from gpu_helpers import run
    A, B, C = normal_problem(300, 200, 150, 41, with_c=True)
    D = oracle.gemm(A, B, beta=beta, C=C)
    _check_normal(run(A, B, C, beta=beta), D, 150)


def test_beta_zero_does_not_read_c():
    from gpu_helpers import run
    A, B, _ = normal_problem(129, 65, 33, 42)
    out = run(A, B, None, beta=0.0, c_fill=np.nan)
    assert np.all(np.isfinite(out))
    _check_normal(out, oracle.gemm(A, B), 33)


def test_k_zero_scales_c():
    from gpu_helpers import run
    A = np.zeros((70, 0), np.float16)
    B = np.zeros((0, 90), np.float16)
    C = np.random.default_rng(3).standard_normal((70, 90)).astype(np.float32)
    assert np.array_equal(run(A, B, C, beta=0.5), (0.5 * C.astype(np.float64)).astype(np.float32))
    assert np.array_equal(run(A, B, C, beta=0.0), np.zeros((70, 90), np.float32))


def test_empty_m_n_leave_c_alone():
    import torch
    import dense_tiled_gemm_f16_amd as lib
    C = torch.full((4, 4), 7.0, device="cuda")
    for M, N in ((0, 4), (4, 0)):
        rc = lib.gemm_f16_f32(M, N, 4, 0, 4, 0, 4, C.data_ptr(), 4, 0.0, 0)
        assert rc == 0
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())


# ---------------------------------------------------------------- strides and alignment
@pytest.mark.parametrize("lds,offs", [((160, 208, 205), (0, 0, 0)), ((151, 201, 200), (0, 0, 0)),
                                      ((152, 200, 200), (1, 3, 1)), ((1800, 1800, 1800), (0, 0, 0))])
def test_padded_and_unaligned_operands(lds, offs):
    from gpu_helpers import run
    M, N, K = 300, 200, 150
    A, B, C = normal_problem(M, N, K, 43, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    out = run(A, B, C, beta=1.0, lda=lds[0], ldb=lds[1], ldc=lds[2], offs=offs)
    _check_normal(out, D, K)


@pytest.mark.parametrize("shape", [(300, 200, 150), (129, 65, 33), (1000, 1100, 704), (513, 257, 192),
                                   (77, 1000, 64), (257, 300, 32), (1, 1000, 64), (512, 512, 544), (601, 520, 1056)])
@pytest.mark.parametrize("tile", list(TILES))
def test_ragged_tiles_with_aligned_rows_every_tile(shape, tile):
    """Ragged M, N and K with 16-byte aligned rows: tiles that cross M or N take the direct-to-LDS
    path with clamped sources, and with K a multiple of the slice the last slice of a tile that
    crosses N goes through the masked path.  Operands sit in NaN padding, so a clamped read that
    reached a stored output would show."""
    from gpu_helpers import run
    M, N, K = shape
    r8 = lambda x: -(-x // 8) * 8
    A, B, C = normal_problem(M, N, K, 800 + M + K, with_c=True)
    beta = 1.0 if (M + N) % 2 else 0.0
    D = oracle.gemm(A, B, beta=beta, C=C if beta else None)
    _say("case", shape, tile, beta)
    out = run(A, B, C if beta else None, beta=beta, lda=r8(K) + 8, ldb=r8(N), ldc=N + 3, opts={"tile": TILES[tile]})
    _check_normal(out, D, K)


LAYOUTS = [(False, True), (True, False), (True, True)]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("shape", [(256, 256, 256), (300, 200, 150), (129, 65, 33), (1000, 1100, 704),
                                   (513, 257, 192), (1, 1000, 64), (77, 1000, 96), (512, 512, 544)])
@pytest.mark.parametrize("tile", list(TILES))
def test_transposed_layouts_every_tile(ta, tb, shape, tile):
    """op(A) = A^T and/or op(B) = B^T on every tile, ragged shapes; operands stored transposed with
    dense and with padded, 16-byte aligned leading dimensions (direct-to-LDS and register paths)."""
    from gpu_helpers import run
    M, N, K = shape
    _say("case layout", ta, tb, shape, tile)
    A, B, C = normal_problem(M, N, K, 1300 + M + N, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    _check_normal(run(A, B, C, beta=1.0, opts={"tile": TILES[tile]}, trans_a=ta, trans_b=tb), D, K)
    r8 = lambda x: -(-x // 8) * 8
    lda = r8(M if ta else K) + 8
    ldb = r8(K if tb else N)
    _check_normal(run(A, B, opts={"tile": TILES[tile]}, trans_a=ta, trans_b=tb, lda=lda, ldb=ldb), oracle.gemm(A, B), K)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_transposed_layouts_register_path_and_unaligned(ta, tb):
    from gpu_helpers import run
    A, B, C = normal_problem(300, 260, 170, 1400, with_c=True)
    D = oracle.gemm(A, B, beta=1.0, C=C)
    _say("case layout unaligned", ta, tb)
    _check_normal(run(A, B, C, beta=1.0, trans_a=ta, trans_b=tb, offs=(1, 3, 0)), D, 170)
    _check_normal(run(A, B, C, beta=1.0, trans_a=ta, trans_b=tb, opts={"path": 1}), D, 170)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_transposed_layouts_integer_inputs_bitwise(ta, tb):
    """Integer-valued inputs: every partial sum is exact, so all layouts give the oracle's bits."""
    from gpu_helpers import run
    A, B, _ = integer_problem(256, 512, 384, 1500)
    D = oracle.gemm(A, B)
    for tile in (1, 5):
        out = run(A, B, trans_a=ta, trans_b=tb, opts={"tile": tile})
        assert np.array_equal(out.astype(np.float64), D), (ta, tb, tile)


@pytest.mark.parametrize("ta,tb", [(False, False)] + LAYOUTS)
@pytest.mark.parametrize("tile", list(TILES))
def test_register_path_integer_inputs_bitwise(ta, tb, tile):
    """The register-staged path forced on every tile and layout with integer inputs (exact partial
    sums, so bit-equal to the oracle): K of 1, 2, 3 and 32 slices plus a ragged tail, an odd number
    of full slices, and M, N that cross the tile edges."""
    from gpu_helpers import run
    for M, N, K in [(257, 263, 129), (640, 384, 1024), (300, 520, 64), (130, 200, 96), (200, 130, 32),
                    (513, 300, 224)]:
        _say("case register integer", ta, tb, (M, N, K), tile)
        A, B, C = integer_problem(M, N, K, 1600 + M + K, with_c=True)
        D = oracle.gemm(A, B, beta=1.0, C=C)
        out = run(A, B, C, beta=1.0, trans_a=ta, trans_b=tb, opts={"tile": TILES[tile], "path": 1})
        assert np.array_equal(out.astype(np.float64), D), ((M, N, K), ta, tb, tile)


def test_1793_with_padded_leading_dimension():
    """The wave-quantization shape with rows padded to 1800 elements (16-byte aligned rows)."""
    from gpu_helpers import run
    A, B, _ = problem_arrays(PROBLEMS["square1793"])
    D = oracle.gemm(A, B)
    _check_normal(run(A, B, lda=1800, ldb=1800, ldc=1800), D, 1793)


# ---------------------------------------------------------------- order and determinism
def test_launch_order_does_not_change_bits():
    """Launch order only changes which tiles run when; each output's arithmetic is the same."""
    from gpu_helpers import run
    A, B, _ = normal_problem(1000, 1100, 700, 44)
    ref = run(A, B, opts={"tile": 2, "group_m": 1, "xcd_remap": 0})
    for g, x in ((8, 1), (8, 0), (3, 1), (1, 1), (16, 1)):
        assert np.array_equal(run(A, B, opts={"tile": 2, "group_m": g, "xcd_remap": x}), ref), (g, x)


def test_repeated_runs_bitwise_identical():
    """Five runs of the same call give the same bits (no races between waves)."""
    from gpu_helpers import run
    A, B, C = normal_problem(700, 900, 1000, 45, with_c=True)
    outs = [run(A, B, C, beta=1.0) for _ in range(5)]
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])


# ---------------------------------------------------------------- full sizes, stratified
def _compare_rows(out_rows, A_rows, B, K, beta=0.0, C_rows=None):
    """Sampled rows of the GPU result (every column) against the oracle on those rows of A (and C)."""
    assert np.all(np.isfinite(out_rows)), "non-finite output"
    err = max_abs_err(out_rows, oracle.gemm(A_rows, B, beta=beta, C=C_rows))
    assert err <= tol_normal(K), ("rows", err, tol_normal(K))


def _compare_cols(out_cols, A, B_cols, K, beta=0.0, C_cols=None):
    """Sampled columns of the GPU result (every row) against the oracle on those columns of B (and C)."""
    assert np.all(np.isfinite(out_cols)), "non-finite output"
    err = max_abs_err(out_cols, oracle.gemm(A, np.ascontiguousarray(B_cols), beta=beta,
                                             C=(np.ascontiguousarray(C_cols) if C_cols is not None else None)))
    assert err <= tol_normal(K), ("columns", err, tol_normal(K))


def _check_full_host(out, A, B, K, beta=0.0, C=None):
    """Stratified rows and columns (tests/sampling.py) of a result held on the host: together they
    reach every output tile, band and lane row."""
    from sampling import strata
    rows, cols = strata(out.shape[0]), strata(out.shape[1])
    _compare_rows(out[rows], A[rows], B, K, beta, C[rows] if C is not None else None)
    _compare_cols(out[:, cols], A, B[:, cols], K, beta, C[:, cols] if C is not None else None)
    return rows, cols


def _full_size(name, opts):
    import torch
    import dense_tiled_gemm_f16_amd as lib
    p = PROBLEMS[name]
    _say("full size", name, opts)
    A, B, C = problem_arrays(p)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.from_numpy(C).cuda() if C is not None else torch.empty((p.M, p.N), dtype=torch.float32, device="cuda")
    lib.gemm(dA, dB, dC, beta=p.beta, opts=opts)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    del dA, dB, dC
    assert np.all(np.isfinite(out))
    _check_full_host(out, A, B, p.K, p.beta, C)


def test_full_size_4096_grouped_and_row_major():
    _full_size("square4096", {"group_m": 8})
    _full_size("square4096", {"group_m": 1, "xcd_remap": 0})


def test_full_size_8192_accumulate():
    """D = A.B + C at 8192^3 in the launch configuration the benchmark times."""
    _full_size("accum8192", None)


def _full_size_general(M, N, K, seed, beta, ta=False, tb=False):
    """Stratified rows and columns of a full-size product against the oracle; A and B are stored
    transposed when ta / tb."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    _say("full size", (M, N, K), "beta", beta, "layout", ta, tb)
    A, B, C = normal_problem(M, N, K, seed, with_c=beta != 0.0)
    dA = torch.from_numpy(np.ascontiguousarray(A.T) if ta else A).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).cuda()
    dC = torch.from_numpy(C).cuda() if C is not None else torch.empty((M, N), dtype=torch.float32, device="cuda")
    lib.gemm(dA, dB, dC, beta=beta, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    del dA, dB, dC
    assert np.all(np.isfinite(out))
    _check_full_host(out, A, B, K, beta, C)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_full_size_8192_accumulate_transposed_layouts(ta, tb):
    """The benchmark's 8192^3 D = A.B + C with A and/or B stored transposed."""
    _full_size_general(8192, 8192, 8192, 71, 1.0, ta, tb)


@pytest.mark.parametrize("n", [4097, 8191])
def test_full_size_unaligned_register_path(n):
    """Odd squares: rows that are not 16-byte aligned take the register-staged ring at full size
    (4097: a second round of edge tiles; 8191: four rounds with non-temporal C accesses)."""
    _full_size_general(n, n, n, 80 + n % 7, 1.0)


@pytest.mark.parametrize("ta", [False, True])
def test_row_split_two_launches(ta):
    """4352^3 runs as two launches (15 tile rows of 256x256, then the last 512 rows with another
    tile); stratified rows (both sides of the seam among them) and columns against the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M = N = K = 4352
    _say("row split", (M, N, K), "trans_a", ta)
    A, B, C = normal_problem(M, N, K, 90 + ta, with_c=True)
    dA = torch.from_numpy(np.ascontiguousarray(A.T) if ta else A).cuda()
    dB = torch.from_numpy(B).cuda()
    dC = torch.from_numpy(C).cuda()
    p = lib.plan(dA, dB, dC, trans_a=ta)
    assert p["tile2"] != 0 and p["split_at"] == 3840, p
    lib.gemm(dA, dB, dC, beta=1.0, trans_a=ta)
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    del dA, dB, dC
    assert np.all(np.isfinite(out))
    rows, _ = _check_full_host(out, A, B, K, 1.0, C)
    assert {3839, 3840} <= set(rows.tolist())   # both sides of the seam


def test_c_beyond_two_gi_elements():
    """65536 x 32768 outputs (2^31 FP32 elements, 8 GiB) with K = 128: element offsets of C pass
    2^31, so any 32-bit index in the epilogue would wrap.  C starts as NaN; stratified rows and
    columns (every output tile, the last rows and columns included) against the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M, N, K = 65536, 32768, 128
    _say("largest C", (M, N, K))
    A, B, _ = normal_problem(M, N, K, 95)
    dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lib.gemm(dA, dB, dC)
    torch.cuda.synchronize()
    from sampling import strata
    rows, cols = strata(M), strata(N)
    out_rows = dC[torch.from_numpy(rows).cuda()].cpu().numpy()
    out_cols = dC[:, torch.from_numpy(cols).cuda()].cpu().numpy()
    del dA, dB, dC
    torch.cuda.empty_cache()
    _compare_rows(out_rows, A[rows], B, K)
    _compare_cols(out_cols, A, B[:, cols], K)


@pytest.mark.parametrize("which", ["A", "B"])
def test_operands_beyond_two_gi_elements(which):
    """An operand of 2^31 FP16 elements (4 GiB): A as 131072 x 16384 (row offsets of A pass 2^31)
    or B as 16384 x 131072 (the columns far right of B).  The operands are drawn on the GPU from a
    seeded generator; the oracle gets the stratified rows of A (or columns of B) it needs, which
    reach every output tile."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    K = 16384
    M, N = (131072, 128) if which == "A" else (128, 131072)
    _say("largest operand", which, (M, N, K))
    gen = torch.Generator(device="cuda").manual_seed(97)
    dA = torch.randn((M, K), device="cuda", generator=gen).half()
    dB = torch.randn((K, N), device="cuda", generator=gen).half()
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    lib.gemm(dA, dB, dC)
    torch.cuda.synchronize()
    from sampling import strata
    if which == "A":
        # N = 128: every column of the sampled rows is compared, so each tile is reached
        rows = strata(M)
        idx = torch.from_numpy(rows).cuda()
        A, B = dA[idx].cpu().numpy(), dB.cpu().numpy()
        out = dC[idx].cpu().numpy()
        del dA, dB, dC
        torch.cuda.empty_cache()
        _compare_rows(out, A, B, K)
    else:
        # M = 128: every row of the sampled columns is compared
        cols = strata(N)
        idx = torch.from_numpy(cols).cuda()
        A, B = dA.cpu().numpy(), dB[:, idx].contiguous().cpu().numpy()
        out = dC[:, idx].cpu().numpy()
        del dA, dB, dC
        torch.cuda.empty_cache()
        _compare_cols(out, A, B, K)


@pytest.mark.parametrize("layout", ["NT", "TN"])
@pytest.mark.parametrize("tile", [0, 1])
def test_transposed_operands_beyond_two_gi_elements(layout, tile):
    """A transposed operand of 2^31 FP16 elements (4 GiB), on the direct-to-LDS paths (NT with both operands
    in pairs of slices, TN with its single-slice ring): B^T as
    131072 x 16384 (NT: its row offsets pass 2^31 elements, so the byte offsets of the loads cross
    4 GiB and every 64-bit address add carries into its high half), or A^T as 16384 x 131072 (TN: the
    columns far right of A^T).  A slip in that arithmetic -- a lost carry -- reads 4 GiB away.  The
    library's tile and the 256x256 tile; stratified columns of C (NT) or rows (TN) against the oracle,
    every row (column) of each, so every output tile is reached."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    K = 16384
    ta, tb = layout == "TN", layout == "NT"
    M, N = (128, 131072) if tb else (131072, 128)
    _say("largest transposed operand", layout, tile, (M, N, K))
    gen = torch.Generator(device="cuda").manual_seed(98)
    dA = (torch.randn((K, M), device="cuda", generator=gen) if ta else
          torch.randn((M, K), device="cuda", generator=gen)).half()
    dB = (torch.randn((N, K), device="cuda", generator=gen) if tb else
          torch.randn((K, N), device="cuda", generator=gen)).half()
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    opts = {"tile": tile} if tile else None
    assert lib.plan(dA, dB, dC, opts, trans_a=ta, trans_b=tb)["vec_b" if tb else "vec_a"] == 1
    lib.gemm(dA, dB, dC, opts=opts, trans_a=ta, trans_b=tb)
    torch.cuda.synchronize()
    from sampling import strata
    if tb:
        cols = strata(N)
        idx = torch.from_numpy(cols).cuda()
        A = dA.cpu().numpy()
        Bc = dB[idx].cpu().numpy().T                 # K x len(cols): those columns of op(B)
        out = dC[:, idx].cpu().numpy()
        del dA, dB, dC
        torch.cuda.empty_cache()
        _compare_cols(out, A, Bc, K)
    else:
        rows = strata(M)
        idx = torch.from_numpy(rows).cuda()
        Ar = np.ascontiguousarray(dA[:, idx].cpu().numpy().T)   # len(rows) x K: those rows of op(A)
        B = dB.cpu().numpy()
        out = dC[idx].cpu().numpy()
        del dA, dB, dC
        torch.cuda.empty_cache()
        _compare_rows(out, Ar, B, K)


@pytest.mark.parametrize("n", [4097, 4608])
def test_row_split_bitwise_equal_to_one_launch(n):
    """The split launches' tiles (256x256 then 128x128 or 256x128) all take K in the same 32-deep
    slices and k16 steps, so each output sees the same additions in the same order: the split call
    must equal the single 256x256 launch bit for bit, over the whole matrix; stratified rows and
    columns of the split call are also compared with the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    _say("row split bitwise", n)
    g = torch.Generator(device="cuda").manual_seed(99)
    A = torch.randn((n, n), device="cuda", generator=g).half()
    B = torch.randn((n, n), device="cuda", generator=g).half()
    C0 = torch.randn((n, n), device="cuda", generator=g)
    C1 = C0.clone()
    p = lib.plan(A, B, C0)
    assert p["tile"] == 1 and p["tile2"] in (2, 4) and p["split_at"] < n, p
    Cin = C0.cpu().numpy()
    lib.gemm(A, B, C0, beta=1.0)
    lib.gemm(A, B, C1, beta=1.0, opts={"tile": 1})
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)
    _check_full_host(C0.cpu().numpy(), A.cpu().numpy(), B.cpu().numpy(), n, 1.0, Cin)


@pytest.mark.parametrize("ta,tb", [(False, False)] + LAYOUTS)
@pytest.mark.parametrize("shape", [(1000, 1100, 704), (601, 520, 1056), (300, 260, 170), (129, 65, 33)])
def test_tiles_and_paths_bitwise_identical(ta, tb, shape):
    """Every tile whose waves do not split K (256x256, 128x128, 64x64, 256x128) adds each output's
    products in the same order: 32-deep K slices, k16 steps in order, then beta*C.  So do the
    direct-to-LDS and register-staged paths.  All eight results must agree bit for bit (ragged M,
    N and K, odd slice counts, a K tail)."""
    from gpu_helpers import run
    M, N, K = shape
    _say("tiles bitwise", shape, ta, tb)
    A, B, C = normal_problem(M, N, K, 1700 + M + K, with_c=True)
    ref = None
    for tile in (1, 2, 3, 4):
        for path in (0, 1):
            out = run(A, B, C, beta=1.0, opts={"tile": tile, "path": path}, trans_a=ta, trans_b=tb)
            if ref is None:
                ref = out
            assert np.array_equal(out, ref), (tile, path)


@pytest.mark.parametrize("tb", [False, True])
def test_column_split_bitwise_equal_to_one_launch(tb):
    """1024 x 16640 splits by columns (256x256 tiles for the first 16384 columns, 64x64 for the
    rest): both tiles take K in the same slices and steps, so the split call equals the single
    256x256 launch bit for bit; with B as given and stored transposed (the second launch then
    starts 16384 rows into B).  Sampled rows also against the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as lib
    M, N, K = 1024, 16640, 2048
    _say("column split", (M, N, K), "trans_b", tb)
    A, B, C = normal_problem(M, N, K, 110 + tb, with_c=True)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(np.ascontiguousarray(B.T) if tb else B).cuda()
    C0 = torch.from_numpy(C).cuda()
    C1 = C0.clone()
    p = lib.plan(dA, dB, C0, trans_b=tb)
    assert p["split_dim"] == 1 and p["split_at"] == 16384 and p["tile2"] == 3, p
    lib.gemm(dA, dB, C0, beta=1.0, trans_b=tb)
    lib.gemm(dA, dB, C1, beta=1.0, opts={"tile": 1}, trans_b=tb)
    torch.cuda.synchronize()
    assert torch.equal(C0, C1)
    _check_full_host(C0.cpu().numpy(), A, B, K, 1.0, C)

