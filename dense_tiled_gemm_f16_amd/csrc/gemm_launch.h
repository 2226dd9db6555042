// Internal interface between the host side of the library (gemm_api.hip: argument checks, plans,
// the C ABI) and its kernels (gemm_f16_f32.hip, splitk_reduce.hip).  Not installed, not part of
// the C ABI; the symbols are hidden in the shared library.
#ifndef GEMM_F16_LAUNCH_H
#define GEMM_F16_LAUNCH_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GEMM_F16_INTERNAL __attribute__((visibility("hidden")))

namespace gemm_f16 {

// Kernel arguments of one launch of the product kernel.
struct Params {
    const uint16_t *A;
    const uint16_t *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n;
    int group_m;
    int xcd_remap;
    int a_dma, b_dma;  // direct-to-LDS loads allowed (16-byte aligned rows, offsets fit 31 bits)
    int c_vec;         // 16-byte stores allowed (16-byte aligned C, ldc % 4 == 0)
    int c_nt;          // C accessed non-temporally (later rounds of tiles still stream A and B, or beta = 0)
    float beta;
    int split_k;       // > 0: K per split; workgroup row blockIdx.y takes K range [y*split_k, ...)
    int64_t c_split;   // elements between the output slices of consecutive splits
};

// Shape of a tile configuration (GEMM_F16_TILE_*); all zero for an unknown id.
struct TileInfo {
    int bm, bn, bk, threads, lds_bytes;
};

GEMM_F16_INTERNAL TileInfo tile_info(int tile);

// Launch the product kernel of tile configuration `tile` for one operand layout (nn: A and B as
// given; nt: B transposed; tn: A transposed; tt: both): `grid` workgroups along x (one per output
// tile, in launch order), `splits` along y (split-K).  Each layout's kernels live in their own object
// of gemm_f16_f32.hip.
GEMM_F16_INTERNAL hipError_t launch_tile_nn(int tile, const Params &p, int64_t grid, hipStream_t s, int splits);
GEMM_F16_INTERNAL hipError_t launch_tile_nt(int tile, const Params &p, int64_t grid, hipStream_t s, int splits);
GEMM_F16_INTERNAL hipError_t launch_tile_tn(int tile, const Params &p, int64_t grid, hipStream_t s, int splits);
GEMM_F16_INTERNAL hipError_t launch_tile_tt(int tile, const Params &p, int64_t grid, hipStream_t s, int splits);

// The launcher of the call's layout (trans_a, trans_b).
inline hipError_t launch_tile(int tile, const Params &p, int64_t grid, hipStream_t s, int trans_a, int trans_b,
                              int splits)
{
    if (!trans_a) return trans_b ? launch_tile_nt(tile, p, grid, s, splits) : launch_tile_nn(tile, p, grid, s, splits);
    return trans_b ? launch_tile_tt(tile, p, grid, s, splits) : launch_tile_tn(tile, p, grid, s, splits);
}

// Split-K second pass: C <- (sum of the S slices of W) + beta*C (see splitk_reduce.hip).
GEMM_F16_INTERNAL hipError_t launch_splitk_reduce(const float *W, int S, int64_t slice, int64_t ldw, int M, int N,
                                                  float *C, int64_t ldc, float beta, int c_vec, hipStream_t s);

}  // namespace gemm_f16

#endif  // GEMM_F16_LAUNCH_H
