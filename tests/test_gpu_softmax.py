"""GPU parity of the fused row softmax (softmax_rows_f32) against the FP64 oracle.

Bar: per element |y - y_oracle| <= y_oracle * (N + 2R + 16) * 2^-24 + 1e-37, with R the largest
|x - max| of the row: FP32 rounding of x - max (relative error R * 2^-24 in exp), of exp itself
(a few ulp), of the row sum (at most N roundings) and of the division.  Rows sit inside NaN
padding, so a read past a row's end shows up as NaN and a write past it is detected.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _run(x, ldx=None, ldy=None, offs=(0, 0), inplace=False):
    from gpu_helpers import softmax_run
    return softmax_run(x, ldx=ldx, ldy=ldy, offs=offs, inplace=inplace)


def _check(x, y):
    from gpu_helpers import softmax_check
    return softmax_check(x, y)


def _x(seed, M, N, scale=1.0):
    return (np.random.default_rng(seed).standard_normal((M, N)) * scale).astype(np.float32)


def test_page_configuration():
    """06_triton_style.py demo 3: M = 4096 rows, N = 1024 columns, FP32, N(0,1) from seed 2."""
    x = np.random.default_rng(2).standard_normal((4096, 1024)).astype(np.float32)
    print("case softmax 4096x1024", flush=True)
    _check(x, _run(x))


@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (7, 64), (2, 255), (5, 256), (5, 257), (9, 1000), (6, 2048), (5, 8192), (3, 10240), (3, 10241),
                                   (3, 4096), (3, 4097), (2, 10000), (130, 33), (3, 16384), (2, 16383), (2, 20000),
                                   (2, 32768), (2, 32769), (1, 50000), (5, 3000), (3, 7000), (3, 40000),
                                   (2, 49152), (2, 49153), (3, 65536), (2, 65535), (2, 65537), (1, 100003),
                                   (512, 10000), (600, 16383), (520, 20000), (512, 24576), (513, 32768),
                                   (700, 12289), (2, 65540), (2, 65544), (3, 105984), (2, 105988), (3, 131072),
                                   (2, 200000), (300, 131072), (2, 81920), (2, 81924), (2, 138752), (2, 138756),
                                   (600, 131072), (1536, 49152)])
def test_shapes(shape):
    """Every kernel and row length band; the last two have inputs over 256 MiB (non-temporal loads)."""
    M, N = shape
    print("case softmax", shape, flush=True)
    x = _x(10 + M + N, M, N)
    _check(x, _run(x))


@pytest.mark.parametrize("shape,ld,offs", [((64, 1024), (1028, 1032), (0, 0)), ((64, 1000), (1003, 1001), (1, 3)),
                                           ((16, 5000), (5004, 5001), (0, 1)), ((8, 300), (300, 300), (2, 0)),
                                           ((4, 20000), (20004, 20001), (1, 1)), ((3, 40000), (40000, 40004), (0, 0)),
                                           ((3, 60000), (60004, 60008), (0, 0)), ((2, 60000), (60001, 60004), (1, 0)),
                                           ((2, 65537), (65540, 65540), (0, 0)), ((2, 105985), (105988, 105992), (0, 0)),
                                           ((2, 131073), (131076, 131080), (0, 0)), ((2, 131073), (131076, 131077), (0, 1)),
                                           ((3, 8191), (8192, 8196), (0, 0)), ((4, 20001), (20004, 20004), (0, 0)),
                                           ((2, 32767), (32768, 32772), (0, 0)), ((3, 49153), (49156, 49160), (0, 0)),
                                           ((2, 65535), (65536, 65540), (0, 0)), ((300, 49152), (49152, 49152), (0, 0)),
                                           ((257, 65535), (65536, 65536), (0, 0)), ((600, 60001), (60004, 60008), (0, 0)),
                                           ((300, 45057), (45060, 45060), (0, 0)), ((400, 32769), (32772, 32772), (0, 0)),
                                           ((300, 45056), (45056, 45060), (0, 0)), ((512, 40001), (40004, 40004), (0, 0))])
def test_strides_and_alignment(shape, ld, offs):
    """Padded and offset rows; rows whose length is not a multiple of 4 but whose starts stay
    16-byte aligned take the 16-byte paths with their last N % 4 elements handled apart."""
    M, N = shape
    print("case softmax", shape, ld, offs, flush=True)
    x = _x(20 + N, M, N)
    _check(x, _run(x, ldx=ld[0], ldy=ld[1], offs=offs))


@pytest.mark.parametrize("N", [100, 1001, 1024, 6000, 20000, 40000, 50257, 65536, 131071, 131072])
def test_wide_value_range_and_in_place(N):
    """|x| up to a few hundred: the row maximum keeps exp finite; the output may overwrite X."""
    print("case softmax wide", N, flush=True)
    x = _x(30 + N, 17, N, scale=80.0)
    _check(x, _run(x, inplace=True))


@pytest.mark.parametrize("N", [3000, 50257, 60000, 131071, 150000])
def test_deterministic(N):
    x = _x(40, 257 if N < 10000 else 9, N)
    a, b = _run(x), _run(x)
    assert np.array_equal(a, b)


def test_more_rows_than_one_launch_holds():
    """2^25 + 5 rows of 3 elements: more waves than one launch's 32-bit work-item count allows, so
    the rows go in two launches; stratified rows (tests/sampling.py: both launches, the seam and
    every four-row workgroup position included) against the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as g
    M, N = (1 << 25) + 5, 3
    print("case softmax", (M, N), flush=True)
    x = _x(50, M, N)
    dx = torch.from_numpy(x).cuda()
    dy = torch.empty_like(dx)
    g.softmax_rows(dx, dy)
    torch.cuda.synchronize()
    y = dy.cpu().numpy()
    del dx, dy
    from sampling import strata
    rows = np.union1d(strata(M), np.r_[(1 << 25) - 64:(1 << 25) + 5])
    _check(x[rows], y[rows])


def test_two_gi_elements():
    """65536 rows of 32768 elements: 2^31 FP32 elements in and out (8 GiB each), so row offsets pass
    2^31 elements; drawn on the GPU from a seeded generator, stratified rows (tests/sampling.py)
    against the oracle."""
    import torch
    import dense_tiled_gemm_f16_amd as g
    M, N = 65536, 32768
    print("case softmax", (M, N), flush=True)
    gen = torch.Generator(device="cuda").manual_seed(52)
    dx = torch.randn((M, N), device="cuda", generator=gen)
    dy = torch.full_like(dx, float("nan"))
    g.softmax_rows(dx, dy)
    torch.cuda.synchronize()
    from sampling import strata
    rows = strata(M)
    idx = torch.from_numpy(rows).cuda()
    x, y = dx[idx].cpu().numpy(), dy[idx].cpu().numpy()
    del dx, dy
    torch.cuda.empty_cache()
    _check(x, y)

