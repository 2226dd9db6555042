// Measurement only (not on the product path): the sustained FP16 matrix-core ceiling of the
// GPU this runs on.
//
// Every wave issues independent v_mfma_f32_32x32x16_f16 back to back with operands that change
// from one instruction to the next (N(0,1)-like FP16 values supplied by the caller), so the
// matrix cores run at their full issue rate with realistic bit activity.  Under a board power
// limit the shader clock then settles where the matrix cores alone draw the allowed power; the
// FLOP rate reached here bounds what any FP16 GEMM can sustain on this board.
//
// Each workgroup records, from its first wave, the elapsed shader-clock ticks (s_memtime) and
// the elapsed 100 MHz reference ticks (s_memrealtime), so the caller can derive the clock and
// check that a 32x32x16 instruction takes 32 shader cycles.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

namespace {

// src: 16 x 64 half8 values (8 A and 8 B operand sets, one per lane).  out: 4 x u64 per block.
__global__ void __launch_bounds__(256) mfma_ceiling_kernel(const half8_t *src, unsigned long long *out, int iters)
{
    const int lane = threadIdx.x & 63;
    half8_t a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = src[i * 64 + lane];
        b[i] = src[(8 + i) * 64 + lane];
    }
    floatx16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[j][r] = 0.0f;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[(j + u) & 7], b[(3 * j + u) & 7], c[j], 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += c[j][r];
    if (threadIdx.x == 0) {
        unsigned long long *d = out + (size_t)blockIdx.x * 4;
        d[0] = t1 - t0;
        d[1] = r1 - r0;
        d[2] = (unsigned long long)(uint64_t)iters * 64;   // MFMAs per wave
        d[3] = (s != s) ? 1u : 0u;                          // keeps the sums live
    }
}

}  // namespace

extern "C" {

// Launch `grid` workgroups of 256 threads, each wave issuing iters*64 MFMAs.  src: 1024 half8
// (16 KiB) device buffer; out: grid*4 u64 device buffer.  Returns 0, -1 for bad arguments, -6 if
// the launch failed.
int gemm_f16_mfma_ceiling(const void *src, void *out, int grid, int iters, void *stream)
{
    if (src == nullptr || out == nullptr || grid <= 0 || iters <= 0) return -1;
    void *args[] = {(void *)&src, (void *)&out, (void *)&iters};
    return hipLaunchKernel(reinterpret_cast<const void *>(&mfma_ceiling_kernel), dim3((unsigned)grid), dim3(256), args,
                           0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : -6;
}

}  // extern "C"
