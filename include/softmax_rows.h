/*
 * softmax_rows.h -- C ABI of the gfx950 (MI355X) fused row softmax, the second workload of the
 * block-programming page (06_triton_style.py, CS349E lecture 10, "block programming", demo 3):
 *
 *     Y[i][j] = exp(X[i][j] - max_j X[i][j]) / sum_j exp(X[i][j] - max_j X[i][j])
 *
 * for an M x N FP32 matrix, computed in one kernel that reads every row once and writes it once
 * (rows up to 65536 elements stay in registers; longer rows keep 65536 or 81920 elements in
 * registers and, when X and Y are 16-byte aligned with ldx, ldy multiples of 4, the next 40448 in
 * LDS, and read only the rest twice).  Results are FP32; the maximum, the exponentials and the sum
 * are FP32 (the page's kernel computes in the input precision).
 *
 * Layout: row-major with unit column stride; ldx, ldy are row strides in ELEMENTS,
 * ldx >= max(1, N), ldy >= max(1, N).  X and Y are DEVICE pointers, 4-byte aligned; Y may equal X
 * (in place) but must not overlap it otherwise.  Loads and stores move 16 bytes per lane at any
 * 4-byte alignment.
 *
 * The caller owns both buffers; the library allocates nothing and keeps no state.  `stream` is a
 * hipStream_t passed as void* (NULL = default stream); the call is asynchronous.
 *
 * Errors: 0 on success, or the GEMM_F16_ERR_* codes of gemm_f16.h: _DIM (M or N negative or above
 * 2^30), _LD (ld too small), _NULL (NULL pointer with M, N > 0), _ALIGN (not 4-byte aligned),
 * _LAUNCH.  M == 0 or N == 0 is a no-op.  NaN and infinite inputs are out of scope.
 */
#ifndef SOFTMAX_ROWS_H
#define SOFTMAX_ROWS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int softmax_rows_f32(int64_t M, int64_t N, const float *X, int64_t ldx, float *Y, int64_t ldy, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SOFTMAX_ROWS_H */
