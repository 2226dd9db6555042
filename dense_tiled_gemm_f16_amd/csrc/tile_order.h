// Launch order: workgroup id -> output tile (tile row, tile column).
//
// Two steps, both bijections on [0, tiles):
//  1. XCD renumbering.  The dispatcher hands consecutive workgroup ids to the 8 XCDs in turn
//     (id w runs on XCD w % 8), and each XCD has its own L2.  Renumbering gives XCD x the
//     contiguous run [start(x), start(x) + count(x)) of the launch order, so tiles that the
//     grouped order places next to each other also share an L2.
//  2. Grouped order (06_triton_style.py, CS349E lecture 10, "block programming": the matmul
//     kernel's program-id mapping and demo 2).  Tile rows are taken GROUP_M at a time; inside
//     a group, consecutive programs walk down the tile rows of one tile column before moving
//     to the next column; the last group may hold fewer rows.  GROUP_M = 1 is row-major order.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define TILE_ORDER_HD __host__ __device__ __forceinline__
#else
#define TILE_ORDER_HD inline
#endif

namespace gemm_f16 {

constexpr int kNumXcd = 8;

// Workgroup id as dispatched -> position in the launch order, so that each XCD gets a
// contiguous run.  count(x) = floor(tiles/8) + (x < tiles % 8).
TILE_ORDER_HD int64_t xcd_renumber(int64_t wg, int64_t tiles)
{
    const int64_t per = tiles / kNumXcd;
    const int64_t rem = tiles % kNumXcd;
    const int64_t x = wg % kNumXcd;
    const int64_t j = wg / kNumXcd;
    const int64_t start = x * per + (x < rem ? x : rem);
    return start + j;
}

// Position in the launch order -> (tile row, tile column) under the grouped order, in closed
// form.  The tile rows form bands of group_m rows (the last band may be shorter); every band
// before the one holding `pid` contributes group_m * tiles_n positions, so the band's first tile
// row is a multiple of group_m and its first position is that row times tiles_n.  Inside the
// band, positions run down the band's rows one tile column at a time (column-major in the band):
// the column is the offset divided by the band's height, the row the rest.
TILE_ORDER_HD void grouped_tile(int64_t pid, int64_t tiles_m, int64_t tiles_n, int64_t group_m,
                                int64_t *pm, int64_t *pn)
{
    const int64_t band_row0 = pid / (group_m * tiles_n) * group_m;
    const int64_t height = tiles_m - band_row0 < group_m ? tiles_m - band_row0 : group_m;
    const int64_t offset = pid - band_row0 * tiles_n;
    const int64_t col = offset / height;
    *pn = col;
    *pm = band_row0 + (offset - col * height);
}

TILE_ORDER_HD void tile_of_workgroup(int64_t wg, int64_t tiles_m, int64_t tiles_n, int64_t group_m,
                                     int xcd_remap, int64_t *pm, int64_t *pn)
{
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t pid = xcd_remap ? xcd_renumber(wg, tiles) : wg;
    grouped_tile(pid, tiles_m, tiles_n, group_m, pm, pn);
}

}  // namespace gemm_f16
