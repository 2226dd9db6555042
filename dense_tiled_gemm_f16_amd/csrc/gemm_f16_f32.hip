// gfx950 (MI355X, CDNA4) FP16-input, FP32-accumulate block-tiled matrix product behind a C ABI.
//
// C <- A.B + beta.C, A (M x K) and B (K x N) binary16 row-major, C (M x N) binary32 row-major.
//
// The method follows the block-tiled design the pages describe (04_tensor_cores.py, CS349E
// lecture 10, "Tensor Core kernels": one workgroup per BM x BN output tile, K streamed in BK
// slices through on-chip shared memory into matrix-instruction fragments, an XOR swizzle
// against bank conflicts, more than one stage in flight; 06_triton_style.py, "block
// programming": grouped launch order and masks for ragged edges), re-designed for gfx950:
//
//  * Matrix instruction: v_mfma_f32_32x32x16_f16 on 64-lane waves.  Lane l supplies row
//    (l % 32) of the 32 x 16 A block and column (l % 32) of the 16 x 32 B block, each as 8
//    consecutive k (k = 8*(l/32) .. +7); it receives 16 FP32 results, column l % 32, rows
//    8*(r/4) + 4*(l/32) + r%4 for accumulator register r.
//  * Fragments need 8 consecutive k per lane for BOTH operands (the page's block kernel keeps
//    B transposed in shared memory for the same reason).  A is k-contiguous already.  B is
//    n-contiguous, so each thread loads the same 8-column chunk from 8 consecutive k rows and
//    transposes the 8x8 block in registers before writing LDS as Bt[n][k].
//  * LDS rows are BK = 64 halfs = 128 bytes = eight 16-byte chunks.  Chunk c of row r is stored
//    at chunk c ^ ((r ^ (r >> 3)) & 7).  8 consecutive rows at one logical chunk (a fragment
//    read) land in 8 different chunks, and so do rows 8 apart (the transposed B writes, where
//    consecutive lanes hold rows n = 8c + e for one e).
//  * Two LDS stages: while the waves compute on one stage, the next K slice is already in
//    registers (issued before the compute) and is written to the other stage after it; one
//    barrier per K slice.
//  * Launch order: XCD renumbering + grouped order (tile_order.h).
//  * Edges: interior tiles use unmasked 16-byte loads; tiles that cross M, N or K (and
//    operands without 16-byte aligned rows) take the masked path, where out-of-range elements
//    read as 0 and are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "gemm_f16.h"
#include "tile_order.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;           // k per pipeline stage (one 128-byte LDS row)
constexpr int64_t kMaxDim = int64_t(1) << 30;  // keeps every in-kernel int index below 2^31

struct Params {
    const uint16_t *A;
    const uint16_t *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;
    int xcd_remap;
    int a_vec, b_vec;
    float beta;
};

template <int BM_, int BN_, int WGM_, int WGN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = kBK;
    static constexpr int WGM = WGM_, WGN = WGN_;
    static constexpr int T = 64 * WGM * WGN;            // threads per workgroup
    static constexpr int WTM = BM / WGM, WTN = BN / WGN; // per-wave output tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;  // 32x32 MFMA blocks per wave
    static constexpr int KC = BK / 8;                   // 16-byte chunks per LDS row
    static constexpr int A_CHUNKS = BM * KC;            // per stage
    static constexpr int A_PER_T = (A_CHUNKS + T - 1) / T;
    static constexpr int B_NCH = BN / 8;                // 8-column chunks per B row
    static constexpr int B_PAIRS = B_NCH * (BK / 8);    // (column chunk, 8-row k group)
    static constexpr int B_PER_T = (B_PAIRS + T - 1) / T;
    static constexpr int A_STAGE = BM * BK;             // halfs per stage
    static constexpr int B_STAGE = BN * BK;
    static constexpr int LDS_HALFS = 2 * (A_STAGE + B_STAGE);
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(KC == 8, "swizzle assumes eight 16-byte chunks per row");
};

__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row ^ (row >> 3)) & 7);
}

// ---------------------------------------------------------------- global -> registers
// A: chunk q = t + i*T of the BM x 64 slice: row q / 8, k-chunk q % 8 (8 lanes cover a row).
template <class TL>
__device__ __forceinline__ void load_a(const Params &p, int m0, int k0, bool fast, u32x4 (&ra)[TL::A_PER_T])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < TL::A_PER_T; ++i) {
        const int q = t + i * TL::T;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (TL::A_PER_T * TL::T == TL::A_CHUNKS || q < TL::A_CHUNKS) {
            const int row = m0 + (q >> 3);
            const int k = k0 + (q & 7) * 8;
            const uint16_t *src = p.A + (int64_t)row * p.lda + k;
            if (fast) {
                v = *reinterpret_cast<const u32x4 *>(src);
            } else if (row < p.M) {
                if (p.a_vec && k + 8 <= p.K) {
                    v = *reinterpret_cast<const u32x4 *>(src);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = (k + e < p.K) ? (uint32_t)src[e] : 0u;
                    v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
        }
        ra[i] = v;
    }
}

// B: pair pr = t + i*T: column chunk pr % B_NCH, k group pr / B_NCH; 8 loads of rows 8g..8g+7.
template <class TL>
__device__ __forceinline__ void load_b(const Params &p, int n0, int k0, bool fast, u32x4 (&rb)[TL::B_PER_T][8])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < TL::B_PER_T; ++i) {
        const int pr = t + i * TL::T;
        const bool live = (TL::B_PER_T * TL::T == TL::B_PAIRS) || pr < TL::B_PAIRS;
        const int n = n0 + (pr % TL::B_NCH) * 8;
        const int kb = k0 + (pr / TL::B_NCH) * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            u32x4 v = {0u, 0u, 0u, 0u};
            const int k = kb + r;
            const uint16_t *src = p.B + (int64_t)k * p.ldb + n;
            if (live) {
                if (fast) {
                    v = *reinterpret_cast<const u32x4 *>(src);
                } else if (k < p.K) {
                    if (p.b_vec && n + 8 <= p.N) {
                        v = *reinterpret_cast<const u32x4 *>(src);
                    } else {
                        uint32_t h[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) h[e] = (n + e < p.N) ? (uint32_t)src[e] : 0u;
                        v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                    }
                }
            }
            rb[i][r] = v;
        }
    }
}

// ---------------------------------------------------------------- registers -> LDS
template <class TL>
__device__ __forceinline__ void store_a(uint16_t *sa, const u32x4 (&ra)[TL::A_PER_T])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < TL::A_PER_T; ++i) {
        const int q = t + i * TL::T;
        if (TL::A_PER_T * TL::T == TL::A_CHUNKS || q < TL::A_CHUNKS) {
            const int row = q >> 3;
            const int c = q & 7;
            *reinterpret_cast<u32x4 *>(sa + row * TL::BK + swz(row, c) * 8) = ra[i];
        }
    }
}

// Transpose an 8 (k) x 8 (n) block of halfs held as 8 row vectors into 8 column vectors.
__device__ __forceinline__ void transpose8x8(const u32x4 (&v)[8], u32x4 (&o)[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int d = e >> 1;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = v[2 * j][d], hi = v[2 * j + 1][d];
            w[j] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
        }
        o[e] = u32x4{w[0], w[1], w[2], w[3]};
    }
}

template <class TL>
__device__ __forceinline__ void store_b(uint16_t *sb, const u32x4 (&rb)[TL::B_PER_T][8])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < TL::B_PER_T; ++i) {
        const int pr = t + i * TL::T;
        if ((TL::B_PER_T * TL::T == TL::B_PAIRS) || pr < TL::B_PAIRS) {
            const int nb = (pr % TL::B_NCH) * 8;
            const int g = pr / TL::B_NCH;
            u32x4 o[8];
            transpose8x8(rb[i], o);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int n = nb + e;
                *reinterpret_cast<u32x4 *>(sb + n * TL::BK + swz(n, g) * 8) = o[e];
            }
        }
    }
}

// ---------------------------------------------------------------- LDS -> MFMA
template <class TL>
__device__ __forceinline__ void compute_stage(const uint16_t *sa, const uint16_t *sb, int wm, int wn,
                                              floatx16 (&acc)[TL::TM][TL::TN])
{
    const int lane = threadIdx.x & 63;
    const int lr = lane & 31;
    const int hk = lane >> 5;
#pragma unroll
    for (int s = 0; s < TL::BK / 16; ++s) {
        half8_t a[TL::TM], b[TL::TN];
#pragma unroll
        for (int mi = 0; mi < TL::TM; ++mi) {
            const int row = wm * TL::WTM + mi * 32 + lr;
            a[mi] = *reinterpret_cast<const half8_t *>(sa + row * TL::BK + swz(row, 2 * s + hk) * 8);
        }
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni) {
            const int n = wn * TL::WTN + ni * 32 + lr;
            b[ni] = *reinterpret_cast<const half8_t *>(sb + n * TL::BK + swz(n, 2 * s + hk) * 8);
        }
#pragma unroll
        for (int mi = 0; mi < TL::TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TL::TN; ++ni)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
    }
}

// ---------------------------------------------------------------- the kernel
template <class TL>
__global__ void __launch_bounds__(TL::T) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_f16_f32_kernel(Params p)
{
    __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS_HALFS];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / TL::WGN;
    const int wn = wave % TL::WGN;
    const int lane = threadIdx.x & 63;

    int64_t pm64, pn64;
    gemm_f16::tile_of_workgroup(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, &pm64, &pn64);
    const int m0 = (int)pm64 * TL::BM;
    const int n0 = (int)pn64 * TL::BN;

    const bool a_full = p.a_vec && (m0 + TL::BM <= p.M);
    const bool b_full = p.b_vec && (n0 + TL::BN <= p.N);
    const int nk = (p.K + TL::BK - 1) / TL::BK;
    const int nk_full = p.K / TL::BK;

    floatx16 acc[TL::TM][TL::TN];
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    u32x4 ra[TL::A_PER_T];
    u32x4 rb[TL::B_PER_T][8];

    if (nk > 0) {
        load_a<TL>(p, m0, 0, a_full && nk_full > 0, ra);
        load_b<TL>(p, n0, 0, b_full && nk_full > 0, rb);
        store_a<TL>(smem, ra);
        store_b<TL>(smem + TL::A_STAGE, rb);
        __syncthreads();
    }

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const bool kfull = kt + 1 < nk_full;
            load_a<TL>(p, m0, (kt + 1) * TL::BK, a_full && kfull, ra);
            load_b<TL>(p, n0, (kt + 1) * TL::BK, b_full && kfull, rb);
        }
        const uint16_t *sa = smem + cur * (TL::A_STAGE + TL::B_STAGE);
        compute_stage<TL>(sa, sa + TL::A_STAGE, wm, wn, acc);
        if (more) {
            uint16_t *na = smem + (cur ^ 1) * (TL::A_STAGE + TL::B_STAGE);
            store_a<TL>(na, ra);
            store_b<TL>(na + TL::A_STAGE, rb);
        }
        __syncthreads();
    }

    // Epilogue: C <- acc + beta*C, masked at the M and N edges.
    const bool full = (m0 + TL::BM <= p.M) && (n0 + TL::BN <= p.N);
    const float beta = p.beta;
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) {
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni) {
            const int col = n0 + wn * TL::WTN + ni * 32 + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * TL::WTM + mi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (full || (row < p.M && col < p.N)) {
                    float *dst = p.C + (int64_t)row * p.ldc + col;
                    float v = acc[mi][ni][r];
                    if (beta != 0.0f) v = __builtin_fmaf(beta, *dst, v);
                    *dst = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- host side
using Tile256 = Tile<256, 256, 2, 2>;
using Tile128 = Tile<128, 128, 2, 2>;
using Tile64 = Tile<64, 64, 2, 2>;
using Tile256x128 = Tile<256, 128, 2, 2>;

struct TileInfo {
    int bm, bn, threads, lds_bytes;
};

template <class TL>
constexpr TileInfo info_of()
{
    return TileInfo{TL::BM, TL::BN, TL::T, (int)(TL::LDS_HALFS * sizeof(uint16_t))};
}

TileInfo tile_info(int tile)
{
    switch (tile) {
    case GEMM_F16_TILE_256x256: return info_of<Tile256>();
    case GEMM_F16_TILE_128x128: return info_of<Tile128>();
    case GEMM_F16_TILE_64x64: return info_of<Tile64>();
    case GEMM_F16_TILE_256x128: return info_of<Tile256x128>();
    default: return TileInfo{0, 0, 0, 0};
    }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile choice: the largest tile that still gives the 256 CUs about a full wave of workgroups.
int choose_tile(int64_t M, int64_t N)
{
    if (cdiv(M, 256) * cdiv(N, 256) >= 192) return GEMM_F16_TILE_256x256;
    if (cdiv(M, 128) * cdiv(N, 128) >= 96) return GEMM_F16_TILE_128x128;
    return GEMM_F16_TILE_64x64;
}

int make_plan(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
              int64_t ldc, const gemm_f16_f32_opts *opts, gemm_f16_f32_plan_t *plan)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_F16_ERR_DIM;
    const int64_t kmin = K > 1 ? K : 1;
    const int64_t nmin = N > 1 ? N : 1;
    if (lda < kmin || ldb < nmin || ldc < nmin) return GEMM_F16_ERR_LD;
    gemm_f16_f32_opts o = {0, 0, -1, 0};
    if (opts) o = *opts;
    if (o.tile < 0 || o.tile >= GEMM_F16_TILE_COUNT || o.group_m < 0 || o.group_m > 65535 ||
        o.xcd_remap < -1 || o.xcd_remap > 1 || o.reserved != 0)
        return GEMM_F16_ERR_OPTS;
    const int tile = o.tile ? o.tile : choose_tile(M, N);
    const TileInfo ti = tile_info(tile);
    gemm_f16_f32_plan_t pl{};
    pl.tile = tile;
    pl.bm = ti.bm;
    pl.bn = ti.bn;
    pl.bk = kBK;
    pl.threads = ti.threads;
    pl.lds_bytes = ti.lds_bytes;
    pl.tiles_m = cdiv(M, ti.bm);
    pl.tiles_n = cdiv(N, ti.bn);
    pl.grid = pl.tiles_m * pl.tiles_n;
    pl.group_m = o.group_m ? o.group_m : 8;
    pl.xcd_remap = o.xcd_remap >= 0 ? o.xcd_remap : 1;
    pl.vec_a = ((uintptr_t)A % 16 == 0) && (lda % 8 == 0);
    pl.vec_b = ((uintptr_t)B % 16 == 0) && (ldb % 8 == 0);
    if (pl.grid > (int64_t)0x7fffffff) return GEMM_F16_ERR_TOO_LARGE;
    if (plan) *plan = pl;
    return GEMM_F16_OK;
}

template <class TL>
hipError_t launch(const Params &p, int64_t grid, hipStream_t stream)
{
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_f16_f32_kernel<TL>), dim3((unsigned)grid),
                           dim3(TL::T), args, 0, stream);
}

}  // namespace

extern "C" {

int gemm_f16_f32_plan(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                      const void *C, int64_t ldc, const gemm_f16_f32_opts *opts, gemm_f16_f32_plan_t *plan)
{
    (void)C;
    return make_plan(M, N, K, A, lda, B, ldb, ldc, opts, plan);
}

int gemm_f16_f32_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb,
                    float *C, int64_t ldc, float beta, void *stream, const gemm_f16_f32_opts *opts)
{
    gemm_f16_f32_plan_t pl;
    const int rc = make_plan(M, N, K, A, lda, B, ldb, ldc, opts, &pl);
    if (rc != GEMM_F16_OK) return rc;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return GEMM_F16_ERR_NULL;

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
    p.a_vec = pl.vec_a;
    p.b_vec = pl.vec_b;
    p.beta = beta;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    switch (pl.tile) {
    case GEMM_F16_TILE_256x256: err = launch<Tile256>(p, pl.grid, s); break;
    case GEMM_F16_TILE_128x128: err = launch<Tile128>(p, pl.grid, s); break;
    case GEMM_F16_TILE_64x64: err = launch<Tile64>(p, pl.grid, s); break;
    case GEMM_F16_TILE_256x128: err = launch<Tile256x128>(p, pl.grid, s); break;
    default: return GEMM_F16_ERR_OPTS;
    }
    return err == hipSuccess ? GEMM_F16_OK : GEMM_F16_ERR_LAUNCH;
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
    case GEMM_F16_ERR_LD: return "leading dimension too small";
    case GEMM_F16_ERR_NULL: return "null pointer for an operand that is used";
    case GEMM_F16_ERR_OPTS: return "invalid option";
    case GEMM_F16_ERR_TOO_LARGE: return "tile grid too large for one launch";
    case GEMM_F16_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
    }
}

}  // extern "C"
