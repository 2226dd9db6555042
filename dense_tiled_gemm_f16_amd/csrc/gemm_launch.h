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

// Launch the product kernel of tile configuration `tile` and operand layout (trans_a, trans_b):
// `grid` workgroups along x (one per output tile, in launch order), `splits` along y (split-K).
GEMM_F16_INTERNAL hipError_t launch_tile(int tile, const Params &p, int64_t grid, hipStream_t s, int trans_a,
                                         int trans_b, int splits);

// Split-K second pass: C <- (sum of the S slices of W) + beta*C (see splitk_reduce.hip).
GEMM_F16_INTERNAL hipError_t launch_splitk_reduce(const float *W, int S, int64_t slice, int64_t ldw, int M, int N,
                                                  float *C, int64_t ldc, float beta, int c_vec, hipStream_t s);

}  // namespace gemm_f16

#endif  // GEMM_F16_LAUNCH_H
