// Host side of the FP16 -> FP32 block-tiled product: argument checks, tile choice, launch plan
// (one launch, or two when the rows or columns are split against wave quantisation), the split-K
// cost model and the C ABI (include/gemm_f16.h).  No kernels: they and their launchers are in
// gemm_f16_f32.hip (the product) and splitk_reduce.hip (split-K's second pass), reached through
// gemm_launch.h.  The one device object here is the fixed scratch of the no-allocation split-K
// entry point.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "gemm_f16.h"
#include "gemm_launch.h"
#include "tile_order.h"

namespace {

using gemm_f16::Params;
using gemm_f16::launch_splitk_reduce;
using gemm_f16::launch_tile;
using gemm_f16::tile_info;
using gemm_f16::TileInfo;

constexpr int64_t kMaxDim = int64_t(1) << 30;  // keeps every in-kernel int index below 2^31
constexpr int kMaxSplits = 1024;
constexpr int64_t kK4TailMaxK = 2816;   // below this K, a partial 64-deep slice makes the plain 128x128 tile faster

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile choice: the tile with the least predicted time, counting whole waves of one workgroup per
// CU over the 256 CUs (wave quantization) and each tile's sustained share of a CU's matrix-core
// rate as measured on full grids.  Ties go to the larger tile, which reads less from L2 per FLOP.
struct Choice {
    int tile;
    double eff;
};
// Direct-to-LDS loads (16-byte aligned rows).
constexpr Choice kChoices[] = {{GEMM_F16_TILE_256x256, 0.72},
                               {GEMM_F16_TILE_256x128, 0.50},
                               {GEMM_F16_TILE_128x128_K4, 0.50},
                               {GEMM_F16_TILE_64x64, 0.15}};
// Register-staged loads (rows not 16-byte aligned, or the forced register path): every tile is
// slower, the large ones least, and the K-split tile is never the fastest.
constexpr Choice kRegChoices[] = {{GEMM_F16_TILE_256x256, 0.55},
                                  {GEMM_F16_TILE_256x128, 0.375},
                                  {GEMM_F16_TILE_128x128, 0.30},
                                  {GEMM_F16_TILE_64x64, 0.15}};

// `units`: workgroups per output tile (the split count of a split-K call, else 1).  `reg`: the
// operands take the register-staged path.
int choose_tile(int64_t M, int64_t N, int64_t units = 1, bool reg = false)
{
    int best = GEMM_F16_TILE_256x256;
    double best_cost = 0.0;
    for (const Choice &c : reg ? kRegChoices : kChoices) {
        const TileInfo t = tile_info(c.tile);
        const int64_t waves = cdiv(cdiv(M, t.bm) * cdiv(N, t.bn) * units, 256);
        const double cost = (double)waves * t.bm * t.bn / c.eff;
        if (best_cost == 0.0 || cost < best_cost * 0.999) {
            best = c.tile;
            best_cost = cost;
        }
    }
    return best;
}

// Split-K cost model (gemm_f16_f32_splitk_choose).  A call asked for s ranges runs on the tile the
// planner picks for s ranges, with `used` ranges of `per` K rows (whole slices of that tile) on
// tiles_m x tiles_n x used workgroups.  Its time is the largest of three bounds, plus the second
// pass when used > 1:
//  - matrix cores: whole waves of 256 workgroups, each doing bm x bn x per multiply-adds at the
//    tile's sustained share of the chip's rate under the board power limit;
//  - load path: each workgroup streams (bm + bn) x per FP16 elements of A and B through its ring at
//    the rate the ring's depth and the load latency allow (stream_rate), as many workgroups per CU
//    as the LDS holds sharing one CU's rate (kCuStream);
//  - HBM: A, B and C once, at the rate these kernels reach from HBM (kHbmStream);
//  - second pass: the used partial products and C read, C written (kPassRate), and its launch.
// Skinny and deep-K problems (few rows or columns, long K) sit on the load-path and HBM bounds,
// which is where splitting pays: more workgroups keep more loads in flight.  The rates are fitted to
// 61 problems measured on one MI355X (1 to 16384 rows, K up to 131072, 1-128 ranges): the split
// counts the model picks run within 2.5 % of the fastest measured count (geometric mean) and never
// more than 1 % slower than the plain call.
constexpr double kCuFlops = 1.6e15 / 256;
constexpr double kCuStream = 150e9;
constexpr double kHbmStream = 3.9e12;
constexpr double kPassRate = 4.24e12;
constexpr double kSecondPass = 2.8e-6;
constexpr int64_t kMinSplitK = 1024;   // shorter ranges spend too much time filling and draining the ring
constexpr double kSplitGain = 0.9;     // a split must be predicted this much faster than the plain call
constexpr int64_t kLdsPerCu = 160 * 1024;

// Bytes per second one workgroup of the tile streams from memory when nothing else limits it.
double stream_rate(int tile)
{
    switch (tile) {
    case GEMM_F16_TILE_256x256: return 150e9;
    case GEMM_F16_TILE_256x128: return 120e9;
    case GEMM_F16_TILE_128x128_K4: return 100e9;
    case GEMM_F16_TILE_128x128: return 60e9;
    default: return 45e9;
    }
}

// Row stride of the split-K workspace slices: N rounded up to a multiple of 4 elements.
int64_t splitk_ldw(int64_t N) { return (N + 3) & ~int64_t(3); }

// The fixed scratch of gemm_f16_f32_splitk_noalloc: split-K partial products for callers that
// cannot allocate.  Every GPU the library runs on holds its own copy (GEMM_F16_SCRATCH_BYTES) from
// the first use until the process ends.  Host code never passes the array's name to a kernel: the
// name is a host-side stand-in, and the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) float scratch[GEMM_F16_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's scratch, or an error code.
int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_F16_ERR_LAUNCH;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
    if (slot.err != hipSuccess || slot.ptr == nullptr) return GEMM_F16_ERR_LAUNCH;
    *out = slot.ptr;
    return GEMM_F16_OK;
}

double splitk_cost(int64_t M, int64_t N, int64_t K, int64_t s)
{
    const int tile = choose_tile(M, N, s);
    const TileInfo ti = tile_info(tile);
    double eff = 0.0;
    for (const Choice &c : kChoices)
        if (c.tile == tile) eff = c.eff;
    const int64_t per = cdiv(cdiv(K, s), ti.bk) * ti.bk;
    const int64_t used = cdiv(K, per);
    const int64_t wgs = cdiv(M, ti.bm) * cdiv(N, ti.bn) * used;
    const double t_mma = (double)cdiv(wgs, 256) * 2.0 * ti.bm * ti.bn * (double)per / (kCuFlops * eff);
    int64_t per_cu = kLdsPerCu / ti.lds_bytes;
    if (per_cu < 1) per_cu = 1;
    if (per_cu > cdiv(wgs, 256)) per_cu = cdiv(wgs, 256);
    const double rate = stream_rate(tile) < kCuStream / (double)per_cu ? stream_rate(tile) : kCuStream / (double)per_cu;
    const double t_load = (double)cdiv(wgs, 256 * per_cu) * (double)(ti.bm + ti.bn) * (double)per * 2.0 / rate;
    const double t_hbm = (2.0 * ((double)M * K + (double)K * N) + 4.0 * (double)M * N) / kHbmStream;
    double t = t_mma > t_load ? t_mma : t_load;
    if (t_hbm > t) t = t_hbm;
    if (used > 1) t += (double)(2 * used + 1) * (double)M * (double)N * 4.0 / kPassRate + kSecondPass;
    return t;
}

// The tile a K tail makes faster: the K-split tile takes K in 64-deep slices, and when K leaves a
// partial one its masked last slice costs it 1-3 us more than the plain 128x128 tile pays for its
// own tail.  The plain tile (same grid) measured 3.5-11 % faster for K up to 2600; from K = 4096
// the K-split tile leads by 12-17 % without a tail, more than the tail takes back.
int k_tail_tile(int tile, int64_t K)
{
    return tile == GEMM_F16_TILE_128x128_K4 && K % 64 != 0 && K < kK4TailMaxK ? GEMM_F16_TILE_128x128 : tile;
}

// Predicted seconds of one launch: whole waves of 256 workgroups, each tile at its sustained share
// of a CU's matrix-core rate (the tile-choice model in time units).
double launch_seconds(int64_t M, int64_t N, int64_t K, const Choice &c)
{
    const TileInfo t = tile_info(c.tile);
    const int64_t waves = cdiv(cdiv(M, t.bm) * cdiv(N, t.bn), 256);
    return (double)waves * 2.0 * t.bm * t.bn * (double)(K > 0 ? K : 1) / (kCuFlops * c.eff);
}

// Split against wave quantisation.  A grid a little over whole waves (4097^2 in 256x256 tiles: 289
// tiles, two waves for 1.13 waves of work) spends a whole wave on its last few tiles.  Two launches
// on the stream instead: the tile rows (or tile columns) that fill whole waves with one tile, then
// the remaining rows (columns) with the tile that finishes them soonest.  Each output is still
// computed by one tile of one launch.  Taken when predicted clearly faster, counting the second
// launch's fixed cost.  Measured gains ran at about 0.8 of the predicted ones on the direct path
// (6144^3: 8.6 % predicted, 7 % measured; 4352^3: 23 % and 15 %) and 4-9 points under them on
// the register-staged path (8193^3: 10.6 % and 3 %; 6143^3: 8.3 % and none), hence two thresholds.
constexpr double kSplitLaunchGain = 0.92;
constexpr double kSplitLaunchGainReg = 0.90;
constexpr double kLaunchSeconds = 4e-6;

struct Split {
    int dim = 0;          // 0: rows of C, 1: columns
    int64_t at = 0;       // rows (columns) the first launch covers
    int tile1 = 0, tile2 = 0;
};

bool choose_split(int64_t M, int64_t N, int64_t K, bool reg, int tile, Split *out)
{
    const Choice *tab = reg ? kRegChoices : kChoices;
    const int count = reg ? (int)(sizeof(kRegChoices) / sizeof(Choice)) : (int)(sizeof(kChoices) / sizeof(Choice));
    double single = 0.0;
    for (int i = 0; i < count; ++i)
        if (tab[i].tile == tile) single = launch_seconds(M, N, K, tab[i]);
    if (single == 0.0) return false;
    double best = single * (reg ? kSplitLaunchGainReg : kSplitLaunchGain);
    bool found = false;
    for (int dim = 0; dim < 2; ++dim) {
        const int64_t D = dim ? N : M, O = dim ? M : N;   // the split extent and the other one
        for (int i = 0; i < count; ++i) {
            const TileInfo ta = tile_info(tab[i].tile);
            const int64_t bd = dim ? ta.bn : ta.bm, bo = dim ? ta.bm : ta.bn;
            const int64_t td = cdiv(D, bd), to = cdiv(O, bo);
            const int64_t k = td * to / 256 * 256 / to;   // tile rows (columns) that fill the whole waves
            if (k <= 0 || k >= td) continue;
            const int64_t d1 = k * bd;
            for (int j = 0; j < count; ++j) {
                const double t = (dim ? launch_seconds(M, d1, K, tab[i]) + launch_seconds(M, N - d1, K, tab[j])
                                      : launch_seconds(d1, N, K, tab[i]) + launch_seconds(M - d1, N, K, tab[j])) +
                                 kLaunchSeconds;
                if (t < best) {
                    best = t;
                    found = true;
                    out->dim = dim;
                    out->at = d1;
                    out->tile1 = tab[i].tile;
                    out->tile2 = tab[j].tile;
                }
            }
        }
    }
    return found;
}

// LDS a workgroup of `tile` takes in operand layout (ta, tb).  The K-split tile and the TN layout (no
// K-contiguous operand) keep four one-slice stages of both operands (ti.lds_bytes).  Every other case
// keeps the K-contiguous operand -- A in NN and NT, B in TT -- in three stages of two slices and the
// other operand in four stages of one.  tests/test_build_asm.py checks this against the LDS each
// compiled kernel declares.
int lds_bytes_in_layout(int tile, const TileInfo &ti, bool ta, bool tb)
{
    if (tile == GEMM_F16_TILE_128x128_K4 || (ta && !tb)) return ti.lds_bytes;
    const bool b_paired = ta;                       // TT pairs B; NN and NT pair A
    const int slice_a = ti.bm * ti.bk * 2, slice_b = ti.bn * ti.bk * 2;
    return b_paired ? 3 * 2 * slice_b + 4 * slice_a : 3 * 2 * slice_a + 4 * slice_b;
}

int make_plan(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
              int64_t ldb, const void *C, int64_t ldc, const gemm_f16_f32_opts *opts, gemm_f16_f32_plan_t *plan,
              int splits = 1, bool allow_split = false)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_F16_ERR_DIM;
    if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return GEMM_F16_ERR_OPTS;
    const int64_t amin = (trans_a ? M : K) > 1 ? (trans_a ? M : K) : 1;   // row length of A as stored
    const int64_t bmin = (trans_b ? K : N) > 1 ? (trans_b ? K : N) : 1;   // row length of B as stored
    const int64_t nmin = N > 1 ? N : 1;
    if (lda < amin || ldb < bmin || ldc < nmin) return GEMM_F16_ERR_LD;
    if (lda > kMaxDim || ldb > kMaxDim || ldc > kMaxDim) return GEMM_F16_ERR_LD;
    if ((uintptr_t)A % 2 != 0 || (uintptr_t)B % 2 != 0 || (uintptr_t)C % 4 != 0) return GEMM_F16_ERR_ALIGN;
    gemm_f16_f32_opts o = {0, 0, -1, 0};
    if (opts) o = *opts;
    if (o.tile < 0 || o.tile >= GEMM_F16_TILE_COUNT || o.group_m < 0 || o.group_m > 65535 ||
        o.xcd_remap < -1 || o.xcd_remap > 1 || o.path < 0 || o.path > 1)
        return GEMM_F16_ERR_OPTS;
    const bool vec_a = o.path == GEMM_F16_PATH_AUTO && ((uintptr_t)A % 16 == 0) && (lda % 8 == 0);
    const bool vec_b = o.path == GEMM_F16_PATH_AUTO && ((uintptr_t)B % 16 == 0) && (ldb % 8 == 0);
    int tile = o.tile ? o.tile : choose_tile(M, N, splits, !(vec_a && vec_b));
    Split sp;
    if (!o.tile && splits == 1) {
        if (allow_split && choose_split(M, N, K, !(vec_a && vec_b), tile, &sp)) tile = sp.tile1;
        tile = k_tail_tile(tile, K);
        if (sp.tile2) sp.tile2 = k_tail_tile(sp.tile2, K);
    }
    const int64_t M1 = sp.tile2 && sp.dim == 0 ? sp.at : M;   // the first launch's extent
    const int64_t N1 = sp.tile2 && sp.dim == 1 ? sp.at : N;
    const TileInfo ti = tile_info(tile);
    gemm_f16_f32_plan_t pl{};
    pl.tile = tile;
    pl.bm = ti.bm;
    pl.bn = ti.bn;
    pl.bk = ti.bk;
    pl.threads = ti.threads;
    pl.lds_bytes = lds_bytes_in_layout(tile, ti, trans_a != 0, trans_b != 0);
    pl.tiles_m = cdiv(M1, ti.bm);
    pl.tiles_n = cdiv(N1, ti.bn);
    pl.grid = pl.tiles_m * pl.tiles_n;
    pl.split_at = sp.dim ? N1 : M1;
    pl.split_dim = sp.tile2 ? sp.dim : 0;
    pl.tile2 = sp.tile2;
    if (sp.tile2) {
        const TileInfo t2 = tile_info(sp.tile2);
        pl.grid2 = sp.dim ? cdiv(M, t2.bm) * cdiv(N - N1, t2.bn) : cdiv(M - M1, t2.bm) * cdiv(N, t2.bn);
    }
    // Default launch order, measured on MI355X after A and B were loaded as whole cache lines:
    // GROUP_M 4, and the XCD renumbering only for grids under 8 tile rows (taller grids ran 1-2 %
    // faster in the hardware's round-robin order, a 4-row grid 2 % slower).
    pl.group_m = o.group_m ? o.group_m : 4;
    pl.xcd_remap = o.xcd_remap >= 0 ? o.xcd_remap : (pl.tiles_m < 8 ? 1 : 0);
    pl.vec_a = vec_a;
    pl.vec_b = vec_b;
    // A launch counts its work-items along x in 32 bits: workgroups x threads must stay below 2^32.
    if (pl.grid * ti.threads > (int64_t)0xffffffff) return GEMM_F16_ERR_TOO_LARGE;
    if (plan) *plan = pl;
    return GEMM_F16_OK;
}

// Parameters of one call (shared by the plain and the split-K entry points).
Params make_params(const gemm_f16_f32_plan_t &pl, int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t lda, const void *B, int64_t ldb, float *C, int64_t ldc, float beta)
{
    Params p;
    p.A = static_cast<const uint16_t *>(A);
    p.B = static_cast<const uint16_t *>(B);
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.tiles_m = (int)pl.tiles_m;
    p.tiles_n = (int)pl.tiles_n;
    p.group_m = pl.group_m;
    p.xcd_remap = pl.xcd_remap;
    // Direct-to-LDS loads take 32-bit per-lane byte offsets from a panel's base: (rows-1)*ld*2 plus
    // one row must stay below 2^31, where a panel has BM (A) or BN (B) rows when K-contiguous and
    // BK rows otherwise.
    const int64_t a_rows = trans_a ? pl.bk : pl.bm, b_rows = trans_b ? pl.bn : pl.bk;
    p.a_dma = pl.vec_a && (a_rows * lda * 2 < ((int64_t)1 << 31));
    p.b_dma = pl.vec_b && (b_rows * ldb * 2 < ((int64_t)1 << 31));
    p.c_vec = ((uintptr_t)C % 16 == 0) && (ldc % 4 == 0);
    // Non-temporal C accesses when later rounds of tiles still stream A and B through the caches
    // (more than one round over the 256 compute units), and whenever beta = 0, where C is only
    // written: single-round grids measured 2-7 % faster at beta = 0 (1792^3 +6.7 %, 4096^3 +2 %)
    // but 3.3 % slower at beta = 1 (4096^3), where C is also read.
    p.c_nt = pl.grid > 256 || beta == 0.0f;
    p.beta = beta;
    p.split_k = 0;
    p.c_split = 0;
    return p;
}


}  // namespace


extern "C" {

int gemm_f16_f32_plan(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, const gemm_f16_f32_opts *opts, gemm_f16_f32_plan_t *plan)
{
    return make_plan(0, 0, M, N, K, A, lda, B, ldb, C, ldc, opts, plan, 1, true);
}

int gemm_f16_f32_plan_tt(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                         const void *B, int64_t ldb, const void *C, int64_t ldc, const gemm_f16_f32_opts *opts,
                         gemm_f16_f32_plan_t *plan)
{
    return make_plan(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, opts, plan, 1, true);
}

int gemm_f16_f32_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                    float *C, int64_t ldc, float beta, void *stream, const gemm_f16_f32_opts *opts)
{
    return gemm_f16_f32_tt(0, 0, M, N, K, A, lda, B, ldb, C, ldc, beta, stream, opts);
}

int gemm_f16_f32_tt(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                    const void *B, int64_t ldb, float *C, int64_t ldc, float beta, void *stream,
                    const gemm_f16_f32_opts *opts)
{
    gemm_f16_f32_plan_t pl;
    const int rc = make_plan(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, opts, &pl, 1, true);
    if (rc != GEMM_F16_OK) return rc;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return GEMM_F16_ERR_NULL;
    if (pl.tile2) {
        // Split: rows (columns) [0, split_at) with the first tile, then the rest with the second,
        // each an ordinary call on offset pointers (the explicit tiles keep them from splitting
        // again).
        gemm_f16_f32_opts o = {0, 0, -1, 0};
        if (opts) o = *opts;
        const int64_t at = pl.split_at;
        const uint16_t *a = static_cast<const uint16_t *>(A), *b = static_cast<const uint16_t *>(B);
        o.tile = pl.tile;
        int rc1;
        if (pl.split_dim == 0) {
            rc1 = gemm_f16_f32_tt(trans_a, trans_b, at, N, K, A, lda, B, ldb, C, ldc, beta, stream, &o);
            if (rc1 != GEMM_F16_OK) return rc1;
            o.tile = pl.tile2;
            const int64_t a_off = trans_a ? at : at * lda;   // elements to row `at` of op(A)
            return gemm_f16_f32_tt(trans_a, trans_b, M - at, N, K, a + a_off, lda, B, ldb, C + at * ldc, ldc, beta,
                                   stream, &o);
        }
        rc1 = gemm_f16_f32_tt(trans_a, trans_b, M, at, K, A, lda, B, ldb, C, ldc, beta, stream, &o);
        if (rc1 != GEMM_F16_OK) return rc1;
        o.tile = pl.tile2;
        const int64_t b_off = trans_b ? at * ldb : at;   // elements to column `at` of op(B)
        return gemm_f16_f32_tt(trans_a, trans_b, M, N - at, K, A, lda, b + b_off, ldb, C + at, ldc, beta, stream, &o);
    }

    const Params p = make_params(pl, trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta);
    const hipError_t err = launch_tile(pl.tile, p, pl.grid, static_cast<hipStream_t>(stream), trans_a, trans_b, 1);
    return err == hipSuccess ? GEMM_F16_OK : GEMM_F16_ERR_LAUNCH;
}

int gemm_f16_f32_splitk_choose(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 1;
    // The count returned is the one modelled: a call with it takes the tile and the ranges costed.
    const double plain = splitk_cost(M, N, K, 1);
    double best = 0.0;
    int64_t best_s = 1;
    for (int64_t s = 2; s <= 256 && cdiv(K, s) >= kMinSplitK; ++s) {
        const double t = splitk_cost(M, N, K, s);
        if (best == 0.0 || t < best * 0.999) {
            best = t;
            best_s = s;
        }
    }
    return best > 0.0 && best < kSplitGain * plain ? (int)best_s : 1;
}

size_t gemm_f16_f32_splitk_workspace(int64_t M, int64_t N, int splits)
{
    if (M <= 0 || N <= 0 || splits <= 1) return 0;
    return (size_t)splits * (size_t)M * (size_t)splitk_ldw(N) * sizeof(float);
}

// K per range and the number of ranges a split-K call with this plan uses (K ranges are whole
// multiples of BK, so every range starts on a slice boundary).
static void splitk_ranges(const gemm_f16_f32_plan_t &pl, int64_t K, int splits, int64_t *per, int *used)
{
    *per = cdiv(cdiv(K, splits), pl.bk) * pl.bk;
    *used = K > 0 ? (int)cdiv(K, *per) : 1;
}

int gemm_f16_f32_splitk(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                        const void *B, int64_t ldb, float *C, int64_t ldc, float beta, int splits, void *workspace,
                        size_t workspace_bytes, void *stream, const gemm_f16_f32_opts *opts)
{
    if (splits < 1 || splits > kMaxSplits) return GEMM_F16_ERR_OPTS;
    gemm_f16_f32_plan_t pl;
    const int rc = make_plan(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, opts, &pl, splits);
    if (rc != GEMM_F16_OK) return rc;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    int64_t per;
    int used;
    splitk_ranges(pl, K, splits, &per, &used);
    if (used <= 1) return gemm_f16_f32_tt(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta, stream, opts);
    if (C == nullptr || A == nullptr || B == nullptr) return GEMM_F16_ERR_NULL;
    if (workspace == nullptr || workspace_bytes < gemm_f16_f32_splitk_workspace(M, N, used)) return GEMM_F16_ERR_WORKSPACE;
    if ((uintptr_t)workspace % 16 != 0) return GEMM_F16_ERR_ALIGN;
    float *W = static_cast<float *>(workspace);
    const int64_t ldw = splitk_ldw(N);
    Params p = make_params(pl, trans_a, trans_b, M, N, K, A, lda, B, ldb, W, ldw, 0.0f);
    p.split_k = (int)per;
    p.c_split = M * ldw;
    p.c_nt = 0;   // the partial products are read back at once by the second pass
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_tile(pl.tile, p, pl.grid, s, trans_a, trans_b, used) != hipSuccess) return GEMM_F16_ERR_LAUNCH;
    const int c_vec = ((uintptr_t)C % 16 == 0) && (ldc % 4 == 0);
    return launch_splitk_reduce(W, used, M * ldw, ldw, (int)M, (int)N, C, ldc, beta, c_vec, s) == hipSuccess
               ? GEMM_F16_OK
               : GEMM_F16_ERR_LAUNCH;
}

int gemm_f16_f32_splitk_noalloc(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A,
                                int64_t lda, const void *B, int64_t ldb, float *C, int64_t ldc, float beta, int splits,
                                void *stream, const gemm_f16_f32_opts *opts)
{
    if (splits < 1 || splits > kMaxSplits) return GEMM_F16_ERR_OPTS;
    gemm_f16_f32_plan_t pl;
    const int rc = make_plan(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, opts, &pl, splits);
    if (rc != GEMM_F16_OK) return rc;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    int64_t per;
    int used;
    splitk_ranges(pl, K, splits, &per, &used);
    if (used <= 1) return gemm_f16_f32_tt(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta, stream, opts);
    const size_t need = gemm_f16_f32_splitk_workspace(M, N, used);
    if (need > GEMM_F16_SCRATCH_BYTES) return GEMM_F16_ERR_SCRATCH;   // checked before any GPU call
    void *ws = nullptr;
    const int sr = scratch_address(&ws);
    if (sr != GEMM_F16_OK) return sr;
    return gemm_f16_f32_splitk(trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, beta, splits, ws,
                               GEMM_F16_SCRATCH_BYTES, stream, opts);
}

int gemm_f16_f32(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb, float *C,
                 int64_t ldc, float beta, void *stream)
{
    return gemm_f16_f32_ex(M, N, K, A, lda, B, ldb, C, ldc, beta, stream, nullptr);
}

int gemm_f16_f32_tile_order(int64_t tiles_m, int64_t tiles_n, int32_t group_m, int32_t xcd_remap, int64_t count,
                            int64_t *pid_m, int64_t *pid_n)
{
    if (tiles_m < 0 || tiles_n < 0 || count < 0 || count > tiles_m * tiles_n) return GEMM_F16_ERR_DIM;
    if (group_m < 1 || (xcd_remap != 0 && xcd_remap != 1)) return GEMM_F16_ERR_OPTS;
    if (count > 0 && (pid_m == nullptr || pid_n == nullptr)) return GEMM_F16_ERR_NULL;
    for (int64_t w = 0; w < count; ++w)
        gemm_f16::tile_of_workgroup(w, tiles_m, tiles_n, group_m, xcd_remap, &pid_m[w], &pid_n[w]);
    return GEMM_F16_OK;
}

const char *gemm_f16_f32_strerror(int code)
{
    switch (code) {
    case GEMM_F16_OK: return "success";
    case GEMM_F16_ERR_DIM: return "invalid dimension (negative or above 2^30)";
    case GEMM_F16_ERR_LD: return "leading dimension too small (or above 2^30)";
    case GEMM_F16_ERR_NULL: return "null pointer for an operand that is used";
    case GEMM_F16_ERR_OPTS: return "invalid option";
    case GEMM_F16_ERR_TOO_LARGE: return "tile grid too large for one launch";
    case GEMM_F16_ERR_LAUNCH: return "kernel launch failed";
    case GEMM_F16_ERR_ALIGN: return "operand not aligned to its element size";
    case GEMM_F16_ERR_WORKSPACE: return "split-K workspace missing or too small";
    case GEMM_F16_ERR_SCRATCH: return "split-K partial products exceed the library's fixed 32 MiB scratch";
    default: return "unknown error code";
    }
}

}  // extern "C"

