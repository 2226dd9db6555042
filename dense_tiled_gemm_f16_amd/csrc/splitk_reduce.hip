// gfx950 (MI355X) second pass of split-K: the fixed-order sum of the FP32 partial products that
// the K ranges of a split-K call wrote into the caller's workspace, plus beta*C.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_launch.h"

namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Split-K second pass: C <- (sum of the S partial products W[0..S-1]) + beta*C.  W[s] is an M x N
// FP32 slice with row stride ldw (a multiple of 4, so every partial is read 16 bytes at a time),
// slices `slice` elements apart.  A thread owns 4 consecutive outputs of a row and one of G groups
// of consecutive slices; it sums its group in slice order, and the G group sums are added in group
// order through LDS.  G depends only on M, N and S, so the order of every addition is fixed and
// results are deterministic.  Bandwidth-bound: the loads of four slices are issued together.
template <int G>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float *W, int S, int64_t slice, int64_t ldw, int M,
                                                            int N, float *C, int64_t ldc, float beta, int c_vec)
{
    constexpr int QB = 256 / G;   // output quads per workgroup
    __shared__ float4_t part[G > 1 ? 256 : 1];
    const int q = threadIdx.x % QB;
    const int g = threadIdx.x / QB;
    const int per = (S + G - 1) / G;
    const int s0 = g * per;
    const int s1 = S < s0 + per ? S : s0 + per;
    const int64_t n4 = (N + 3) / 4;
    const int64_t total = (int64_t)M * n4;
    for (int64_t base = (int64_t)blockIdx.x * QB; base < total; base += (int64_t)gridDim.x * QB) {
        const int64_t t = base + q;
        const int i = (int)(t / n4);
        const int j = (int)(t % n4) * 4;
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (t < total && s0 < s1) {
            const float *w = W + (int64_t)i * ldw + j;
            acc = *reinterpret_cast<const float4_t *>(w + (int64_t)s0 * slice);
            int s = s0 + 1;
            for (; s + 4 <= s1; s += 4) {
                const float4_t v0 = *reinterpret_cast<const float4_t *>(w + (int64_t)s * slice);
                const float4_t v1 = *reinterpret_cast<const float4_t *>(w + (int64_t)(s + 1) * slice);
                const float4_t v2 = *reinterpret_cast<const float4_t *>(w + (int64_t)(s + 2) * slice);
                const float4_t v3 = *reinterpret_cast<const float4_t *>(w + (int64_t)(s + 3) * slice);
                acc += v0;
                acc += v1;
                acc += v2;
                acc += v3;
            }
            for (; s < s1; ++s) acc += *reinterpret_cast<const float4_t *>(w + (int64_t)s * slice);
        }
        if constexpr (G > 1) {
            part[threadIdx.x] = acc;
            __syncthreads();
            if (g == 0)
                for (int h = 1; h < G; ++h) acc += part[h * QB + q];
            __syncthreads();   // the next pass overwrites part
        }
        if (g == 0 && t < total) {
            float *c = C + (int64_t)i * ldc + j;
            if (c_vec && j + 4 <= N) {
                if (beta != 0.0f) {
                    const float4_t old = *reinterpret_cast<const float4_t *>(c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(beta, old[e], acc[e]);
                }
                *reinterpret_cast<float4_t *>(c) = acc;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < N) c[e] = beta != 0.0f ? __builtin_fmaf(beta, c[e], acc[e]) : acc[e];
            }
        }
    }
}

// Slice groups per output for the second pass: enough threads to cover the chip (about 64K) when
// the output alone has fewer quads, never more groups than slices.
int reduce_groups(int64_t quads, int S)
{
    int G = 1;
    while (G < 16 && quads * G < 65536 && 2 * G <= S) G *= 2;
    return G;
}

}  // namespace

namespace gemm_f16 {

hipError_t launch_splitk_reduce(const float *W, int S, int64_t slice, int64_t ldw, int M, int N, float *C, int64_t ldc,
                         float beta, int c_vec, hipStream_t s)
{
    const int64_t quads = (int64_t)M * ((N + 3) / 4);
    const int G = reduce_groups(quads, S);
    const int64_t blocks = cdiv(quads, 256 / G);
    const dim3 grid((unsigned)(blocks < 4096 ? blocks : 4096));
    void *args[] = {(void *)&W, (void *)&S, (void *)&slice, (void *)&ldw, (void *)&M, (void *)&N, (void *)&C,
                    (void *)&ldc, (void *)&beta, (void *)&c_vec};
    const void *k = G == 1   ? reinterpret_cast<const void *>(&splitk_reduce_kernel<1>)
                    : G == 2 ? reinterpret_cast<const void *>(&splitk_reduce_kernel<2>)
                    : G == 4 ? reinterpret_cast<const void *>(&splitk_reduce_kernel<4>)
                    : G == 8 ? reinterpret_cast<const void *>(&splitk_reduce_kernel<8>)
                             : reinterpret_cast<const void *>(&splitk_reduce_kernel<16>);
    return hipLaunchKernel(k, grid, dim3(256), args, 0, s);
}

}  // namespace gemm_f16
