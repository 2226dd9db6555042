"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched): it loads, exports
every entry point the header declares, validates arguments, plans launches and computes the
launch order the kernels use."""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_tiled_gemm_f16_amd as g
from dense_tiled_gemm_f16_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    return names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(_abi.LIB_PATH)
    declared = _declared_functions()
    assert {"gemm_f16_f32", "gemm_f16_f32_ex", "gemm_f16_f32_plan", "gemm_f16_f32_tile_order",
            "gemm_f16_f32_strerror"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(_abi.SIGNATURES), "binding and header disagree"


def test_strerror_is_total():
    for code in range(-10, 2):
        assert isinstance(g.gemm_f16_f32_strerror(code), str)


@pytest.mark.parametrize("args,code", [
    ((-1, 4, 4, 4, 4, 4), -1), ((4, -1, 4, 4, 4, 4), -1), ((4, 4, -1, 4, 4, 4), -1),
    ((1 << 31, 4, 4, 4, 4, 4), -1),
    ((4, 4, 8, 7, 4, 4), -2), ((4, 8, 4, 4, 7, 8), -2), ((4, 8, 4, 4, 8, 7), -2),
    ((4, 4, 0, 0, 4, 4), -2),
])
def test_argument_validation(args, code):
    M, N, K, lda, ldb, ldc = args
    assert g.gemm_f16_f32(M, N, K, 16, lda, 16, ldb, 16, ldc, 0.0, None) == code
    assert g.gemm_f16_f32_plan(M, N, K, 16, lda, 16, ldb, 16, ldc)[0] == code


@pytest.mark.parametrize("n,lda,tile,rows1,tile2", [(4097, 4097, 1, 3840, 2), (4352, 4352, 1, 3840, 5),
                                                    (6144, 6144, 1, 5376, 4), (8193, 8193, 1, 7936, 2)])
def test_row_split_against_wave_quantisation(n, lda, tile, rows1, tile2):
    """289 tiles of 256x256 would take two waves of 256 workgroups for 1.13 waves of work: the
    planner launches the 15 tile rows that fill one wave, then the remaining rows with a smaller
    tile.  Explicit tiles, whole-wave grids and the split-K entry point never split."""
    rc, p = g.gemm_f16_f32_plan(n, n, n, 256, lda, 256, lda, 256, lda)
    assert rc == 0 and (p["tile"], p["split_at"], p["tile2"]) == (tile, rows1, tile2), p
    tn = -(-n // 256)
    assert p["grid"] == rows1 // 256 * tn and p["grid"] % 256 > 256 - tn and p["grid2"] > 0
    rc, p = g.gemm_f16_f32_plan(n, n, n, 256, lda, 256, lda, 256, lda, {"tile": 1})
    assert rc == 0 and p["split_at"] == n and p["tile2"] == 0 and p["grid"] == tn * tn
    rc, p = g.gemm_f16_f32_plan_tt(1, 0, n, n, n, 256, lda, 256, lda, 256, lda)
    assert rc == 0 and p["split_at"] == rows1 and p["tile2"] == tile2
    # 6143 (register path): the split is predicted 8.3 % faster, under that path's 10 % bar
    for m in (4096, 8192, 1793, 3073, 5120, 5376, 6143):
        rc, p = g.gemm_f16_f32_plan(m, m, m, 256, m, 256, m, 256, m)
        assert rc == 0 and p["split_at"] == m and p["tile2"] == 0 and p["grid2"] == 0 and p["split_dim"] == 0


@pytest.mark.parametrize("M,N,at,tile2", [(1024, 16640, 16384, 3), (512, 33024, 32768, 3), (256, 65600, 65536, 3),
                                         (2048, 50264, 49152, 5)])
def test_column_split_for_wide_grids(M, N, at, tile2):
    """A grid with few tile rows cannot fill whole waves by rows: 1024 x 16640 in 256x256 tiles is
    4 x 65 = 260 tiles, two waves for 1.02.  The planner splits the columns instead: the 256 tiles
    of the first 16384 columns, then the last columns with a smaller tile; squares keep splitting
    by rows."""
    K = 4096
    rc, p = g.gemm_f16_f32_plan(M, N, K, 256, K, 256, N, 256, N)
    assert rc == 0 and (p["tile"], p["split_dim"], p["split_at"], p["tile2"]) == (1, 1, at, tile2), p
    assert p["grid"] == (M // 256) * (at // 256) and p["grid2"] > 0
    rc, p = g.gemm_f16_f32_plan_tt(0, 1, M, N, K, 256, K, 256, K, 256, N)
    assert rc == 0 and (p["split_dim"], p["split_at"]) == (1, at)
    rc, p = g.gemm_f16_f32_plan(4097, 4097, 4097, 256, 4097, 256, 4097, 256, 4097)
    assert rc == 0 and p["split_dim"] == 0


def test_grid_too_large_for_one_launch():
    """Workgroups x threads must fit the launch's 32-bit work-item count: 524288^2 outputs fit as
    2048^2 tiles of 256x256 (2^30 threads) but not as 8192^2 tiles of 64x64 (2^34 threads)."""
    n = 1 << 19
    rc, p = g.gemm_f16_f32_plan(n, n, 64, 256, 64, 256, n, 256, n, {"tile": 1})
    assert rc == 0 and p["grid"] == 2048 * 2048
    rc, _ = g.gemm_f16_f32_plan(n, n, 64, 256, 64, 256, n, 256, n, {"tile": 3})
    assert rc == -5
    assert g.gemm_f16_f32_ex(n, n, 64, 256, 64, 256, n, 256, n, 0.0, None, {"tile": 3}) == -5
    rc, _ = g.gemm_f16_f32_plan(1 << 30, 1 << 30, 64, 256, 64, 256, 1 << 30, 256, 1 << 30)
    assert rc == -5
    assert "too large" in g.gemm_f16_f32_strerror(-5)


def test_null_pointers_rejected_before_launch():
    assert g.gemm_f16_f32(4, 4, 4, None, 4, 16, 4, 16, 4, 0.0, None) == -3
    assert g.gemm_f16_f32(4, 4, 4, 16, 4, None, 4, 16, 4, 0.0, None) == -3
    assert g.gemm_f16_f32(4, 4, 4, 16, 4, 16, 4, None, 4, 0.0, None) == -3


def test_misaligned_pointers_rejected_before_launch():
    assert g.gemm_f16_f32(4, 4, 4, 17, 4, 16, 4, 16, 4, 0.0, None) == -7      # A odd
    assert g.gemm_f16_f32(4, 4, 4, 16, 4, 17, 4, 16, 4, 0.0, None) == -7      # B odd
    assert g.gemm_f16_f32(4, 4, 4, 16, 4, 16, 4, 18, 4, 0.0, None) == -7      # C not 4-byte aligned
    assert g.gemm_f16_f32_plan(4, 4, 4, 18, 4, 18, 4, 20, 4)[0] == 0         # element-aligned is enough
    assert "align" in g.gemm_f16_f32_strerror(-7)


@pytest.mark.parametrize("args,code", [((-1, 4, 4, 4), -1), ((4, -1, 4, 4), -1), ((4, 8, 7, 8), -2), ((4, 8, 8, 7), -2)])
def test_softmax_argument_validation(args, code):
    M, N, ldx, ldy = args
    assert g.softmax_rows_f32(M, N, 16, ldx, 16, ldy, None) == code


def test_softmax_rejects_null_and_misaligned_and_accepts_empty():
    assert g.softmax_rows_f32(4, 4, None, 4, 16, 4, None) == -3
    assert g.softmax_rows_f32(4, 4, 18, 4, 16, 4, None) == -7
    assert g.softmax_rows_f32(0, 4, None, 4, None, 4, None) == 0
    assert g.softmax_rows_f32(4, 0, None, 1, None, 1, None) == 0


@pytest.mark.parametrize("ta,tb,lds,code", [
    (1, 0, (300, 200, 200), 0), (1, 0, (299, 200, 200), -2),     # A stored K x M: lda >= M
    (0, 1, (150, 150, 200), 0), (0, 1, (150, 149, 200), -2),     # B stored N x K: ldb >= K
    (1, 1, (300, 150, 200), 0), (2, 0, (300, 200, 200), -4), (0, -1, (150, 200, 200), -4)])
def test_transposed_leading_dimensions(ta, tb, lds, code):
    M, N, K = 300, 200, 150
    rc, _ = g.gemm_f16_f32_plan_tt(ta, tb, M, N, K, 256, lds[0], 256, lds[1], 256, lds[2])
    assert rc == code
    if code != 0:   # errors return before anything is launched (no device memory needed)
        assert g.gemm_f16_f32_tt(ta, tb, M, N, K, 256, lds[0], 256, lds[1], 256, lds[2], 0.0, None) == code


def test_empty_m_or_n_is_a_no_op():
    assert g.gemm_f16_f32(0, 4, 4, None, 4, None, 4, None, 4, 0.0, None) == 0
    assert g.gemm_f16_f32(4, 0, 4, None, 4, None, 1, None, 1, 0.0, None) == 0


@pytest.mark.parametrize("opts", [{"tile": 9}, {"tile": -1}, {"group_m": -2}, {"group_m": 70000},
                                  {"xcd_remap": 2}, {"xcd_remap": -5}, {"path": 2}, {"path": -1}])
def test_bad_options(opts):
    assert g.gemm_f16_f32_ex(64, 64, 64, 16, 64, 16, 64, 16, 64, 0.0, None, opts) == -4


def test_plan_choices():
    rc, p = g.gemm_f16_f32_plan(8192, 8192, 8192, 256, 8192, 256, 8192, 256, 8192)
    assert rc == 0 and p["tile"] == 1 and p["grid"] == 1024 and p["vec_a"] and p["vec_b"]
    rc, p = g.gemm_f16_f32_plan(1792, 1792, 1792, 256, 1800, 256, 1800, 256, 1800)
    assert rc == 0 and p["vec_a"] and p["vec_b"]
    assert p["tile"] == 5 and (p["bm"], p["bn"], p["bk"]) == (128, 128, 64)   # K-split 128x128 tile
    rc, p = g.gemm_f16_f32_plan(1793, 1793, 1793, 256, 1800, 256, 1800, 256, 1800)
    assert rc == 0 and p["vec_a"] and p["vec_b"]
    assert p["tile"] == 2 and (p["bm"], p["bn"], p["bk"]) == (128, 128, 32)   # K tail: plain 128x128
    rc, p = g.gemm_f16_f32_plan(1793, 1793, 1793, 256, 1793, 256, 1793, 256, 1793)
    assert rc == 0 and not p["vec_a"] and not p["vec_b"]
    assert p["tile"] == 2 and (p["bm"], p["bn"], p["bk"]) == (128, 128, 32)   # register path: plain 128x128
    rc, p = g.gemm_f16_f32_plan(4096, 4096, 4096, 256, 4096, 256, 4096, 256, 4096)
    assert rc == 0 and p["tile"] == 1


@pytest.mark.parametrize("n,tile", [(256, 3), (1024, 3), (1792, 5), (2048, 5), (3072, 1), (4096, 1), (8192, 1)])
def test_tile_choice_counts_whole_waves(n, tile):
    """The default tile minimises whole waves x tile work / the tile's measured efficiency: at 3072
    the 256x256 grid (144 tiles, one wave) beats the 128x128 grid (576 tiles, three waves)."""
    rc, p = g.gemm_f16_f32_plan(n, n, n, 256, n, 256, n, 256, n)
    assert rc == 0 and p["tile"] == tile, (n, p["tile"])
    rc, p = g.gemm_f16_f32_plan(8192, 8192, 8192, 256, 8192, 256, 8192, 256, 8192, {"path": 1})
    assert rc == 0 and not p["vec_a"] and not p["vec_b"]      # register-staged path forced
    rc, p = g.gemm_f16_f32_plan(256, 256, 256, 258, 256, 256, 256, 256, 256)
    assert rc == 0 and not p["vec_a"] and p["vec_b"]         # A base not 16-byte aligned
    rc, p = g.gemm_f16_f32_plan(300, 200, 150, 256, 150, 256, 200, 256, 200, {"tile": 4, "group_m": 3})
    assert rc == 0 and (p["bm"], p["bn"], p["group_m"]) == (256, 128, 3)
    assert p["tiles_m"] == 2 and p["tiles_n"] == 2


@pytest.mark.parametrize("m,n,k,tile", [(1792, 1792, 1800, 2), (2048, 2048, 2600, 2), (1536, 1536, 2808, 2),
                                        (1536, 1536, 2816, 5), (1792, 1792, 4104, 5), (1792, 1792, 2048, 5),
                                        (1792, 1792, 1792, 5)])
def test_k_tail_prefers_the_plain_128_tile(m, n, k, tile):
    """Where the waves pick the 128x128 grid, a K that leaves a partial 64-deep slice switches the
    K-split tile for the plain one below K = 2816 (both measured on aligned rows)."""
    rc, p = g.gemm_f16_f32_plan(m, n, k, 256, k, 256, n, 256, n)
    assert rc == 0 and p["vec_a"] and p["vec_b"] and p["tile"] == tile, (m, n, k, p["tile"])
    rc, p = g.gemm_f16_f32_plan(m, n, k, 256, k, 256, n, 256, n, {"tile": 5})
    assert rc == 0 and p["tile"] == 5   # an explicit tile is kept


@pytest.mark.parametrize("n,tile", [(1025, 2), (1793, 2), (2049, 4), (2561, 4), (3073, 1), (4097, 1), (6143, 1),
                                    (8191, 1)])
def test_register_path_tile_choice(n, tile):
    """Rows that are not 16-byte aligned take the register-staged path, whose tiles rank
    differently (measured on unaligned squares): the K-split tile is never chosen there."""
    rc, p = g.gemm_f16_f32_plan(n, n, n, 256, n, 256, n, 256, n)
    assert rc == 0 and not p["vec_a"] and p["tile"] == tile, (n, p["tile"])


# ---------------------------------------------------------------- launch order
def test_grouped_order_matches_page_example(golden):
    """06_triton_style.py demo 2: 9x9 tiles, GROUP_M = 3: the first nine programs cover a 3x3 block
    of tiles and read 54 blocks (27 of A, 27 of B) instead of 90 for row-major order."""
    gg = golden["page_launch_counts"]["grouped_order_9x9"]
    rc, pm, pn = g.gemm_f16_f32_tile_order(9, 9, 3, 0)
    assert rc == 0
    assert [[m, n] for m, n in zip(pm[:9], pn[:9])] == gg["group_m_3_first_nine"]
    blocks = len(set(pm[:9])) * 9 + len(set(pn[:9])) * 9
    assert blocks == gg["group_m_3_blocks_read"]
    rc, pm, pn = g.gemm_f16_f32_tile_order(9, 9, 1, 0)
    assert (pm[:9], pn[:9]) == ([0] * 9, list(range(9)))
    assert len(set(pm[:9])) * 9 + len(set(pn[:9])) * 9 == gg["row_major_blocks_read"]


@pytest.mark.parametrize("tm,tn,gm", [(32, 32, 8), (15, 15, 8), (7, 13, 3), (1, 1, 1), (5, 1, 8), (1, 9, 4),
                                      (33, 31, 16), (225, 1, 8)])
@pytest.mark.parametrize("xcd", [0, 1])
def test_launch_order_is_a_bijection(tm, tn, gm, xcd):
    rc, pm, pn = g.gemm_f16_f32_tile_order(tm, tn, gm, xcd)
    assert rc == 0
    assert sorted(zip(pm, pn)) == [(m, n) for m in range(tm) for n in range(tn)]


def test_xcd_renumbering_gives_each_xcd_a_contiguous_run():
    """Workgroup w runs on XCD w % 8; after renumbering, the workgroups of one XCD walk a
    contiguous stretch of the grouped order."""
    tm, tn, gm = 32, 32, 8
    rc, pm_x, pn_x = g.gemm_f16_f32_tile_order(tm, tn, gm, 1)
    rc, pm_0, pn_0 = g.gemm_f16_f32_tile_order(tm, tn, gm, 0)
    order = {(m, n): i for i, (m, n) in enumerate(zip(pm_0, pn_0))}
    tiles = tm * tn
    for x in range(8):
        pos = [order[(pm_x[w], pn_x[w])] for w in range(x, tiles, 8)]
        assert pos == list(range(pos[0], pos[0] + len(pos)))


def test_tile_order_errors():
    assert g.gemm_f16_f32_tile_order(3, 3, 0, 0)[0] == -4
    assert g.gemm_f16_f32_tile_order(3, 3, 1, 2)[0] == -4
    assert g.gemm_f16_f32_tile_order(3, 3, 1, 0, count=10)[0] == -1


# ---------------------------------------------------------------- split-K
def test_splitk_workspace_size():
    assert g.gemm_f16_f32_splitk_workspace(4, 4, 2) == 2 * 4 * 4 * 4
    assert g.gemm_f16_f32_splitk_workspace(512, 512, 32) == 32 * 512 * 512 * 4
    assert g.gemm_f16_f32_splitk_workspace(4, 4, 1) == 0
    assert g.gemm_f16_f32_splitk_workspace(0, 4, 3) == 0
    assert "workspace" in g.gemm_f16_f32_strerror(-8)


def test_splitk_errors_before_launch():
    """Argument errors return before anything is launched (fake device addresses suffice)."""
    M, N, K = 64, 64, 4096
    base = (0, 0, M, N, K, 256, K, 256, N, 256, N, 0.0)
    need = g.gemm_f16_f32_splitk_workspace(M, N, 4)
    assert g.gemm_f16_f32_splitk(*base, 4, 4096, need - 1, None) == -8      # too small
    assert g.gemm_f16_f32_splitk(*base, 4, None, need, None) == -8          # missing
    assert g.gemm_f16_f32_splitk(*base, 4, 4100, need, None) == -7          # not 16-byte aligned
    assert g.gemm_f16_f32_splitk(*base, 0, 4096, need, None) == -4          # split count out of range
    assert g.gemm_f16_f32_splitk(*base, 1025, 4096, need, None) == -4
    assert g.gemm_f16_f32_splitk(0, 0, M, N, K, 256, K - 1, 256, N, 256, N, 0.0, 4, 4096, need, None) == -2
    assert g.gemm_f16_f32_splitk(0, 0, 0, N, K, None, K, None, N, None, N, 0.0, 4, None, 0, None) == 0



@pytest.mark.parametrize("shape,lo,hi", [((8192, 8192, 8192), 1, 1), ((4096, 4096, 4096), 1, 1),
                                         ((1792, 1792, 1792), 1, 1), ((2048, 2048, 2048), 1, 1),
                                         ((3072, 3072, 3072), 1, 1), ((2048, 2048, 16384), 1, 4),
                                         ((128, 128, 131072), 64, 128), ((256, 256, 65536), 24, 128),
                                         ((512, 512, 65536), 8, 64), ((1024, 1024, 32768), 4, 16),
                                         ((1, 4096, 4096), 3, 8), ((16, 8192, 28672), 2, 8),
                                         ((64, 1024, 32768), 8, 32), ((8192, 64, 8192), 2, 4),
                                         ((1, 16384, 4096), 1, 1), ((16, 16384, 4096), 1, 1),
                                         ((32, 32768, 8192), 1, 1), ((512, 8192, 8192), 1, 1)])
def test_splitk_choice(shape, lo, hi):
    """The split count the cost model picks lies where the measured times are within about 10 % of
    the fastest count (one MI355X; counts 2-128 timed): large squares fill the chip unsplit; deep-K
    problems with few output tiles and skinny problems (a few rows or columns, long K) split, into
    ranges of at least 1024 K rows; skinny problems whose plain grid already fills the chip
    (1 x 16384 x 4096: 256 tiles) measured slower split and stay plain."""
    M, N, K = shape
    s = g.gemm_f16_f32_splitk_choose(M, N, K)
    assert lo <= s <= hi, s
    assert s == 1 or -(-K // s) >= 1024
    assert g.gemm_f16_f32_splitk_choose(0, 4, 4) == 1 and g.gemm_f16_f32_splitk_choose(4, 4, 0) == 1


def test_default_launch_order():
    """GROUP_M 4 by default; the XCD renumbering only for grids under 8 tile rows (measured)."""
    rc, p = g.gemm_f16_f32_plan(8192, 8192, 8192, 256, 8192, 256, 8192, 256, 8192)
    assert rc == 0 and p["tiles_m"] == 32 and (p["group_m"], p["xcd_remap"]) == (4, 0)
    rc, p = g.gemm_f16_f32_plan(1024, 8192, 8192, 256, 8192, 256, 8192, 256, 8192)
    assert rc == 0 and p["tiles_m"] == 4 and (p["group_m"], p["xcd_remap"]) == (4, 1)
    rc, p = g.gemm_f16_f32_plan(8192, 8192, 8192, 256, 8192, 256, 8192, 256, 8192, {"group_m": 8, "xcd_remap": 1})
    assert rc == 0 and (p["group_m"], p["xcd_remap"]) == (8, 1)


def test_noalloc_splitk_refuses_past_its_scratch_without_touching_the_gpu():
    """gemm_f16_f32_splitk_noalloc checks the partials' size against its fixed 32 MiB scratch before
    any GPU call (this runs without a GPU): 4 x 2048 x 2048 FP32 partials are 64 MiB."""
    assert g.gemm_f16_f32_splitk_workspace(2048, 2048, 4) == 64 << 20 > _abi.SCRATCH_BYTES
    assert g.gemm_f16_f32_splitk_noalloc(0, 0, 2048, 2048, 8192, 256, 8192, 256, 2048, 256, 2048, 0.0, 4, None) == -9
    assert g.gemm_f16_f32_splitk_noalloc(0, 0, 2048, 2048, 8192, 256, 8192, 256, 2048, 256, 2048, 0.0, 0, None) == -4
    assert g.gemm_f16_f32_splitk_noalloc(0, 0, -1, 4, 4, 256, 4, 256, 4, 256, 4, 0.0, 2, None) == -1
