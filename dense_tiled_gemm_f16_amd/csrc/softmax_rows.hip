// gfx950 (MI355X) fused row softmax behind a C ABI (include/softmax_rows.h).
//
// The operation is the block-programming page's second workload (06_triton_style.py, CS349E
// lecture 10, "block programming", demo 3): per row, subtract the maximum, exponentiate, divide
// by the sum -- fused into one kernel, so each element is read from memory once and written once
// (the page's operator-by-operator version makes five passes).  It is bandwidth-bound: a few
// arithmetic operations per 8 bytes moved, so the design is about memory access, not math:
//
//  * Rows of up to 2048 elements: one 64-lane wave per row, four rows per workgroup.  Longer rows:
//    the waves of a workgroup share one row (a wave per row leaves too few waves in flight,
//    measured 1.6-3x slower on long rows): four waves up to 8192 elements, eight up to 32768,
//    sixteen beyond.  Rows of up to 65536 elements stay in registers between the three phases
//    (maximum, exp and sum, scale), so HBM sees exactly one read and one write per element.
//    (Holding rows in LDS instead was measured slower: a quarter of LDS per row leaves four waves
//    per CU.)  Each lane moves 16 bytes per access, so a wave covers 1 KiB of consecutive memory
//    per instruction.  FP32 rows start 4-byte aligned, and a 16-byte access needs no more than
//    that for (nearly) full rate, so rows of any stride take these 16-byte paths; the row's last
//    N % 4 elements are handled one per lane.
//  * Maximum and sum across a wave are xor butterflies: every lane ends with the same value, and
//    the order of the additions is fixed; across the waves of a workgroup their results are
//    combined through LDS in wave order, so results are deterministic.
//  * Longer rows keep 65536 elements in registers (81920 for 81921-138752 elements), 16-byte
//    aligned rows also the next 40448 in LDS (the whole CU's LDS for one row, loaded by
//    direct-to-LDS loads); only the rest is read twice, once for its running maximum and sum (the
//    sum rescaled whenever the maximum grows) and once for its outputs.
//  * Everything is FP32.  Every exponent here is x - max <= 0; e^d is taken as the hardware's
//    base-2 exponential of d*log2(e) with the product's rounding error put back (exp_nonpos, about
//    8 instructions where the library's expf takes about 20), and each row is scaled by one
//    reciprocal of its sum instead of a division per element.  The element loop is then about half
//    the vector instructions it was: on long rows, where every CU runs one or two rows in
//    lockstep, the vector work does not overlap the memory traffic and adds to it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm_f16.h"
#include "softmax_rows.h"


namespace {

typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float4_u __attribute__((ext_vector_type(4), aligned(4)));   // 16 bytes at 4-byte alignment

constexpr int kRowsPerBlock = 4;
constexpr int64_t kMaxDim = int64_t(1) << 30;

// Outputs are written once and not read again by the kernel: non-temporal 16-byte stores
// (measured 26 % faster at 4096 x 1024 and 14 % at 65536 x 1024 than ordinary stores, which let Y
// displace X from the caches; non-temporal loads of X measured slower).
__device__ __forceinline__ void store_out(float *dst, float4_t v)
{
    __builtin_nontemporal_store(float4_u{v[0], v[1], v[2], v[3]}, reinterpret_cast<float4_u *>(dst));
}

// 16 bytes of a row at its 4-byte alignment (one global_load_dwordx4).  NTL: a non-temporal load,
// for inputs larger than the 256 MB memory-attached cache, which cannot keep them between calls
// anyway.  There the register kernels measured 1-8 % faster with them (16384 x 8192: 0.699 ->
// 0.753 of 8 TB/s; 131072 x 1024: 0.749 -> 0.794; 8192 x 32000: 0.710 -> 0.734), while on inputs
// the cache holds, called back to back, they lose what it gives (8192 x 8192: 0.859 -> 0.770).
template <bool NTL = false>
__device__ __forceinline__ float4_t ld4(const float *src)
{
    float4_u v;
    if constexpr (NTL)
        v = __builtin_nontemporal_load(reinterpret_cast<const float4_u *>(src));
    else
        v = *reinterpret_cast<const float4_u *>(src);
    return float4_t{v[0], v[1], v[2], v[3]};
}

// e^d for d <= 0 (or -inf).  t = d*log2(e) rounded to FP32; c = d*log2(e) - t from two FMAs (the
// product's exact rounding error plus the part of log2(e) that FP32 drops); e^d = 2^t * 2^c, with
// 2^t from v_exp_f32 (1 ulp) and 2^c ~ 1 + c*ln 2 (|c| < 2^-17).  Within 3 * 2^-24 relative of e^d
// wherever e^d is a normal FP32 number; below that the result is 0 or subnormal (under 2^-126).
__device__ __forceinline__ float exp_nonpos(float d)
{
    constexpr float kLog2e = 1.44269502162933349609375f;   // log2(e) rounded to FP32
    constexpr float kLog2eLo = 1.925963033500011e-08f;     // log2(e) - kLog2e
    constexpr float kLn2 = 0.693147182464599609375f;       // ln 2 rounded to FP32
    d = fmaxf(d, -160.0f);                                 // -inf (a masked column) gives 0, not NaN
    const float t = d * kLog2e;
    const float c = fmaf(d, kLog2eLo, fmaf(d, kLog2e, -t));
    const float r = __builtin_amdgcn_exp2f(t);
    return fmaf(r, c * kLn2, r);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Element e (0 <= e < 4*VPL) of a lane: element e%4 of its piece e/4, i.e. column
// ((e/4)*64 + lane)*4 + e%4.
template <int VPL, bool NTL>
__global__ void __launch_bounds__(256) softmax_reg_kernel(int M, int N, const float *X, int64_t ldx, float *Y,
                                                          int64_t ldy)
{
    constexpr int E = 4 * VPL;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kRowsPerBlock + (int)(threadIdx.x >> 6);
    if (row >= M) return;   // the whole wave leaves; no barriers follow
    const float *x = X + (int64_t)row * ldx;
    float *y = Y + (int64_t)row * ldy;

    float v[E];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = (i * 64 + lane) * 4;
        if (c + 4 <= N) {
            const float4_t t = ld4<NTL>(x + c);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * i + e] = t[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * i + e] = (c + e < N) ? x[c + e] : -INFINITY;
        }
    }
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < E; ++e) m = fmaxf(m, v[e]);
    m = wave_max(m);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        v[e] = exp_nonpos(v[e] - m);   // columns past N hold -inf and give 0
        s += v[e];
    }
    const float inv = 1.0f / wave_sum(s);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = (i * 64 + lane) * 4;
        if (c + 4 <= N) {
            store_out(y + c, float4_t{v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv});
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c + e < N) y[c + e] = v[4 * i + e] * inv;
        }
    }
}

// ---------------------------------------------------------------- one workgroup per row
// Long rows: the four waves of a workgroup share one row, so a row keeps four times the
// parallelism and up to four times the registers of a single wave.  Each wave reduces its part
// with the butterflies above; the four wave results meet in LDS and every thread combines them in
// wave order (fixed, so results stay deterministic).
constexpr int kBlock = 256;

// W waves' results combined in wave order (0, 1, .., W-1), the same order in every thread.
template <int W>
__device__ __forceinline__ float block_max(float v, float *red)
{
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r = fmaxf(r, red[w]);
    __syncthreads();   // red is written again by the next reduction
    return r;
}

template <int W>
__device__ __forceinline__ float block_sum(float v, float *red)
{
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) r += red[w];
    __syncthreads();
    return r;
}

// Rows of up to 4*VPT*BLOCK elements held in registers: one read and one write per element.
// Element e of a thread: element e%4 of piece (e/4)*BLOCK + t, i.e. column ((e/4)*BLOCK + t)*4 +
// e%4, and the row's last N%4 elements one each in threads 0-2.  BLOCK = 1024 (sixteen waves)
// holds rows of up to 65536 elements at 64 values per thread.
template <int VPT, int BLOCK, bool NTL>
__global__ void __launch_bounds__(BLOCK) softmax_block_kernel(int M, int N, const float *X, int64_t ldx, float *Y,
                                                              int64_t ldy)
{
    constexpr int W = BLOCK / 64;
    __shared__ float red[W];
    constexpr int E = 4 * VPT;
    const int t = threadIdx.x;
    const float *x = X + (int64_t)blockIdx.x * ldx;
    float *y = Y + (int64_t)blockIdx.x * ldy;
    float v[E];
    // Every load is issued unconditionally -- pieces past the row's whole ones are read from
    // piece 0 and masked, the tail from element 0 -- so that no branch makes the compiler wait
    // for all loads before the first is used.
    const int nf = N >> 2, ntail = N & 3;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int p = i * BLOCK + t;
        const float4_t q = ld4<NTL>(x + 4 * (p < nf ? p : 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * i + e] = q[e];
        __builtin_amdgcn_sched_barrier(0);   // loads issued in piece order, the order of use
    }
    float tv = x[t < ntail ? 4 * nf + t : 0];
    __builtin_amdgcn_sched_barrier(0);   // all loads issued before any use (the masks below)
    tv = t < ntail ? tv : -INFINITY;
    // With at least 8 pieces per thread, each group of GS pieces is reduced against its own
    // maximum as soon as it has arrived, while the later groups are still on their way (loads
    // complete in issue order); the row's maximum then only rescales the groups' sums and, at
    // the output, their stored e^(x - m_group) by e^(m_group - max) / sum.  With fewer, the
    // row's maximum comes first and every exponential is taken against it.
    constexpr bool GROUPED = VPT >= 8;
    constexpr int GS = GROUPED ? (VPT % 4 == 0 ? 4 : 2) : VPT, NG = VPT / GS;
    float mg[NG], sg[NG];
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        mg[g] = -INFINITY;
#pragma unroll
        for (int e = 4 * GS * g; e < 4 * GS * (g + 1); ++e) {
            v[e] = (e / 4) * BLOCK + t < nf ? v[e] : -INFINITY;   // pieces past the row's whole ones
            mg[g] = fmaxf(mg[g], v[e]);
        }
        m = fmaxf(m, mg[g]);
        sg[g] = 0.0f;
        if constexpr (GROUPED) {
            const float ref = mg[g] == -INFINITY ? 0.0f : mg[g];   // a group of only -inf: all 0
#pragma unroll
            for (int e = 4 * GS * g; e < 4 * GS * (g + 1); ++e) {
                v[e] = exp_nonpos(v[e] - ref);
                sg[g] += v[e];
            }
            asm volatile("" ::"v"(sg[g]));   // here, not sunk past the reductions below
            __builtin_amdgcn_sched_barrier(0);   // and group by group, in the order of arrival
        }
    }
    m = block_max<W>(fmaxf(m, tv), red);   // the tail last: its load was issued last
    float s = exp_nonpos(tv - m);          // 0 without a tail element
    if constexpr (GROUPED) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            mg[g] = exp_nonpos(mg[g] - m);   // the group's scale; 0 for a group of only -inf
            s += sg[g] * mg[g];
        }
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            v[e] = exp_nonpos(v[e] - m);   // pieces past the row hold -inf and give 0
            s += v[e];
        }
    }
    const float inv = 1.0f / block_sum<W>(s, red);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const float f = GROUPED ? mg[i / GS] * inv : inv;
        const int p = i * BLOCK + t;
        if (p < nf)
            store_out(y + 4 * p, float4_t{v[4 * i] * f, v[4 * i + 1] * f, v[4 * i + 2] * f, v[4 * i + 3] * f});
    }
    if (t < ntail) y[4 * nf + t] = exp_nonpos(tv - m) * inv;
}

// ---------------------------------------------------------------- rows longer than the registers
// Rows of more than 65536 elements, one workgroup of sixteen waves per row (BLOCK = 1024; also,
// with BLOCK = 512 and half the LDS, 257-2047 16-byte aligned rows of 32769-65536 elements, two to
// a CU).  The row is cut
// into float4 pieces (16 bytes); piece p of the row's first N/4, with R1 = VPT*BLOCK:
//   region 1, p < R1: registers, piece i*BLOCK + t in thread t (VPT pieces, 4*VPT values each);
//   region 2 (LDS = true: 16-byte aligned rows, which the direct-to-LDS load is used for only, as
//     in the GEMM), the next up to LF4 pieces (10112 = 158 KiB, nearly all of the CU's LDS, or
//     5056 for two rows per CU): LDS, piece R1 + k*BLOCK + t at part[k*BLOCK + t], loaded
//     straight into LDS (global_load_lds_dwordx4), so
//     it needs no registers in flight, and each thread only ever touches its own pieces, which its
//     own wave loaded (no barrier: the wave's own load counter orders them);
//   region 3, the rest: read twice, in chunks of C pieces per thread (what the registers left
//     beside region 1 hold);
//   the last N%4 elements: one each in threads 0-2.
// HBM sees one read of regions 1 and 2, two of region 3, and one write.  VPT = 16, C = 6 from
// 65537 elements; VPT = 20, C = 4 (every register of a thread taken) where region 1 fills and
// region 3 fits one chunk, 81921-138752 elements: at 131072, 2.07 passes against 2.19 with 16.
// Each thread first reduces its own values against its own maxima (one per region), so the
// exponentials of regions 1 and 2 are taken while region 3 is still on its way, and each is taken
// once: an output is its stored e^(x - m_region) times e^(m_region - max) / sum.  Region 3 keeps a
// running maximum and sum, rescaled once per chunk.  All loads of a step are issued before any is
// used (addresses past a region's end are redirected to the row's first piece and the values
// masked), so each thread keeps VPT (region 1), then C (region 3) 16-byte loads in flight.
constexpr int kHybridLdsF4 = 10112;  // region 2: float4 pieces per row in LDS (158 waves' loads)

// One direct-to-LDS load: 16 bytes per lane from base + off into LDS [lds + lds_off + 16*lane].
// Inline assembly, as in the GEMM kernels, so that M0 (the instruction's LDS base) is written only
// here; the add that forms it writes SCC, which is declared clobbered.  The compiler does not see
// the load: the kernel below waits for it explicitly.
__device__ __forceinline__ void dma16(const float *base, uint32_t off, uint32_t lds, uint32_t lds_off)
{
    asm volatile("s_add_u32 m0, %2, %3\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds), "s"(lds_off)
                 : "memory", "scc");
}

template <int VPT, int C, bool LDS, int BLOCK, int LF4>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4, 4)))
softmax_hybrid_kernel(int M, int N, const float *X, int64_t ldx, float *Y, int64_t ldy)
{
    constexpr int W = BLOCK / 64, R1 = VPT * BLOCK;   // N > 4 * R1: region 1 is whole
    constexpr int K2 = (LF4 + BLOCK - 1) / BLOCK;     // LDS rounds; round k, wave w loads if k*W + w < LF4/64
    static_assert(LF4 % 64 == 0, "region 2 is whole waves' loads");
    __shared__ float4_t part[LDS ? LF4 : 1];
    __shared__ float red[W];
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const float *x = X + (int64_t)blockIdx.x * ldx;
    float *y = Y + (int64_t)blockIdx.x * ldy;
    const int nf = N >> 2;                                                // whole pieces (>= R1)
    const int n2 = !LDS ? 0 : nf - R1 < LF4 ? nf - R1 : LF4;
    const int s3 = R1 + n2;                                               // first piece of region 3
    const int ntail = N & 3;
    // Byte offsets within a row fit 32 bits (N <= 2^30).  An access to piece u + v, with u the same
    // in every lane, takes the address as (row + 16u) in scalar registers plus 16v per lane, so
    // region 1's loads and stores share one offset register.
    const char *xb = reinterpret_cast<const char *>(x);
    char *yb = reinterpret_cast<char *>(y);
    // Ordinary loads throughout: non-temporal ones for regions 1 and 2 of inputs beyond the cache
    // measured within 3 % either way (600 x 131072, 4096 x 128256).
    const auto piece = [&](int u, int v) {
        return ld4(reinterpret_cast<const float *>((xb + (uint32_t)u * 16u) + (uint32_t)v * 16u));
    };
    const auto put = [&](int u, int v, float4_t val) {
        store_out(reinterpret_cast<float *>((yb + (uint32_t)u * 16u) + (uint32_t)v * 16u), val);
    };

    // Issue, in this order (loads complete in order): region 2 into LDS, region 1 into registers,
    // region 3's first chunk, the tail element.
    const uint32_t lds = (uint32_t)(uintptr_t)part;
#pragma unroll
    for (int k = 0; k < (LDS ? K2 : 0); ++k) {
        if (k * W + wave < LF4 / 64) {
            const int i = k * BLOCK + t;
            dma16(x, (uint32_t)(i < n2 ? R1 + i : 0) * 16u, lds, (uint32_t)((k * BLOCK + wave * 64) * 16));
        }
    }
    float4_t q[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) q[i] = piece(i * BLOCK, t);
    __builtin_amdgcn_sched_barrier(0);   // region 1's loads all go before region 3's
    float4_t r[C];
    const auto load_chunk = [&](int b) {
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int p = b + j * BLOCK + t;
            r[j] = piece(0, p < nf ? p : 0);
        }
    };
    load_chunk(s3);   // unconditionally (all to piece 0 if region 3 is empty): the wait below counts on it
    float tv = -INFINITY;
    if (t < ntail) tv = x[4 * nf + t];
    __builtin_amdgcn_sched_barrier(0);   // every load above is issued before any work starts

    // Region 2 first, while regions 1 and 3 are on their way: this wave's LDS loads are older than
    // the VPT + C loads after them (and the tail load, in wave 0 only).
    if constexpr (LDS) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VPT + C) : "memory");
    const int k2 = wave * 64 < n2 ? (n2 - wave * 64 + BLOCK - 1) / BLOCK : 0;   // rounds holding this wave's pieces
    float m2 = -INFINITY;
#pragma unroll 1
    for (int k = 0; k < k2; ++k) {
        const int i = k * BLOCK + t;
        const float4_t v = part[i];
        if (i < n2) m2 = fmaxf(m2, fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    }
    const float ref2 = m2 == -INFINITY ? 0.0f : m2;
    float s2 = 0.0f;
#pragma unroll 1
    for (int k = 0; k < k2; ++k) {
        const int i = k * BLOCK + t;
        float4_t v = part[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = exp_nonpos(v[e] - ref2);
        if (i < n2) {
            s2 += (v[0] + v[1]) + (v[2] + v[3]);
            part[i] = v;
        }
    }

    asm volatile("" ::"v"(s2));   // keep region 2's work here (the compiler would sink it past region 3)

    // Region 1 against its own maximum, while region 3's first chunk is on its way.
    float m1 = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPT; ++i) m1 = fmaxf(m1, fmaxf(fmaxf(q[i][0], q[i][1]), fmaxf(q[i][2], q[i][3])));
    const float ref1 = m1 == -INFINITY ? 0.0f : m1;   // a row part of only -inf: its exponentials are 0
    float s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            q[i][e] = exp_nonpos(q[i][e] - ref1);
            s1 += q[i][e];
        }
    asm volatile("" ::"v"(s1));

    // Region 3: running maximum and sum, one rescale per chunk, the next chunk loaded after each.
    float m3 = -INFINITY, s3sum = 0.0f;
    for (int b = s3; b < nf; b += C * BLOCK) {
        float cm = -INFINITY;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            if (b + j * BLOCK + t >= nf) r[j] = float4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            cm = fmaxf(cm, fmaxf(fmaxf(r[j][0], r[j][1]), fmaxf(r[j][2], r[j][3])));
        }
        const float nm = fmaxf(m3, cm);
        const float ref = nm == -INFINITY ? 0.0f : nm;
        float cs = 0.0f;
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) cs += exp_nonpos(r[j][e] - ref);
        s3sum = s3sum * exp_nonpos(m3 - ref) + cs;
        m3 = nm;
        if (b + C * BLOCK < nf) load_chunk(b + C * BLOCK);
    }

    // The row: maximum, then each thread's sums brought to it, in a fixed order.
    const float mx = block_max<W>(fmaxf(fmaxf(m1, m2), fmaxf(m3, tv)), red);
    const float st = s1 * exp_nonpos(m1 - mx) + s2 * exp_nonpos(m2 - mx) + s3sum * exp_nonpos(m3 - mx) +
                     exp_nonpos(tv - mx);
    const float inv = 1.0f / block_sum<W>(st, red);

    // Outputs: regions 1 and 2 from their stored exponentials, region 3 read again, then the tail.
    // (Reading region 3's first chunk again before writing region 2 measured slower.)
    const float f1 = exp_nonpos(m1 - mx) * inv, f2 = exp_nonpos(m2 - mx) * inv;
#pragma unroll
    for (int i = 0; i < VPT; ++i) put(i * BLOCK, t, q[i] * f1);
#pragma unroll 1
    for (int k = 0; k < k2; ++k) {
        const int i = k * BLOCK + t;
        if (i < n2) put(R1 + k * BLOCK, t, part[i] * f2);
    }
    for (int b = s3; b < nf; b += C * BLOCK) {
        load_chunk(b);
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int p = b + j * BLOCK + t;
            if (p < nf)
                put(0, p, float4_t{exp_nonpos(r[j][0] - mx) * inv, exp_nonpos(r[j][1] - mx) * inv,
                                   exp_nonpos(r[j][2] - mx) * inv, exp_nonpos(r[j][3] - mx) * inv});
        }
    }
    if (t < ntail) y[4 * nf + t] = exp_nonpos(tv - mx) * inv;
}

template <class Kernel>
hipError_t launch_block(Kernel kernel, int M, int N, const float *X, int64_t ldx, float *Y, int64_t ldy, hipStream_t s,
                        int block = kBlock)
{
    void *args[] = {(void *)&M, (void *)&N, (void *)&X, (void *)&ldx, (void *)&Y, (void *)&ldy};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)M), dim3(block), args, 0, s);
}

template <class Kernel>
hipError_t launch_one(Kernel kernel, int M, int N, const float *X, int64_t ldx, float *Y, int64_t ldy, hipStream_t s)
{
    void *args[] = {(void *)&M, (void *)&N, (void *)&X, (void *)&ldx, (void *)&Y, (void *)&ldy};
    const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(64 * kRowsPerBlock);
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, s);
}

// a16: rows 16-byte aligned (X, Y and both strides), which the hybrid kernel's LDS region needs.
template <bool NTL>
hipError_t launch_softmax(int M, int N, const float *X, int64_t ldx, float *Y, int64_t ldy, hipStream_t s, bool a16)
{
    if (N <= 256) return launch_one(&softmax_reg_kernel<1, NTL>, M, N, X, ldx, Y, ldy, s);
    if (N <= 512) return launch_one(&softmax_reg_kernel<2, NTL>, M, N, X, ldx, Y, ldy, s);
    if (N <= 1024) return launch_one(&softmax_reg_kernel<4, NTL>, M, N, X, ldx, Y, ldy, s);
    if (N <= 2048) return launch_one(&softmax_reg_kernel<8, NTL>, M, N, X, ldx, Y, ldy, s);
    // Longer rows: a workgroup per row (measured faster than a wave per row from 4096 elements),
    // in registers up to 65536 elements.
    if (N <= 4096) return launch_block(&softmax_block_kernel<4, kBlock, NTL>, M, N, X, ldx, Y, ldy, s);
    if (N <= 8192) return launch_block(&softmax_block_kernel<8, kBlock, NTL>, M, N, X, ldx, Y, ldy, s);
    // 8193-32768 elements: eight waves per row at up to 64 values per thread, so two workgroups
    // (two rows) share a CU with sixteen waves between them.  Four waves per row (up to 128 values
    // per thread, two rows per CU, eight waves) measured up to 10 % slower (1024 x 32768: 48.4
    // against 44.2 us); sixteen (one row per CU) up to 15 % slower with many rows and within
    // 1.5 % with few.
    if (N <= 12288) return launch_block(&softmax_block_kernel<6, 512, NTL>, M, N, X, ldx, Y, ldy, s, 512);
    if (N <= 16384) return launch_block(&softmax_block_kernel<8, 512, NTL>, M, N, X, ldx, Y, ldy, s, 512);
    if (N <= 20480) return launch_block(&softmax_block_kernel<10, 512, NTL>, M, N, X, ldx, Y, ldy, s, 512);
    if (N <= 24576) return launch_block(&softmax_block_kernel<12, 512, NTL>, M, N, X, ldx, Y, ldy, s, 512);
    if (N <= 32768) return launch_block(&softmax_block_kernel<16, 512, NTL>, M, N, X, ldx, Y, ldy, s, 512);
    // 32769-65536 elements, 16-byte aligned, 257-2047 rows: eight waves per row, 32768 (to 45056
    // elements) or 45056 elements in registers (64 or 88 per thread) and the rest in 79 KiB of
    // LDS, so that two rows share a CU and one computes while the other loads.  With 45056 in
    // registers, measured 1-18 % faster than a row per CU from 300 to 1536 rows (300 x 49152:
    // 20.4 against 24.3 us; 1024 x 65536: 88.3 against 91.1), the same at 2048, slower with one
    // row per CU (256 x 65536: 27.2 against 25.5) and with many (4096 x 46080: 274.6 against
    // 267.0).  Otherwise sixteen waves per row keep up to 64 values per thread in registers.
    const bool two_per_cu = a16 && M > 256 && M < 2048;
    if (two_per_cu && N <= 45056)
        return launch_block(&softmax_hybrid_kernel<16, 1, true, 512, 5056>, M, N, X, ldx, Y, ldy, s, 512);
    if (two_per_cu && N <= 65536)
        return launch_block(&softmax_hybrid_kernel<22, 1, true, 512, 5056>, M, N, X, ldx, Y, ldy, s, 512);
    if (N <= 49152) return launch_block(&softmax_block_kernel<12, 1024, NTL>, M, N, X, ldx, Y, ldy, s, 1024);
    if (N <= 65536) return launch_block(&softmax_block_kernel<16, 1024, NTL>, M, N, X, ldx, Y, ldy, s, 1024);
    // Longer: 65536 or 81920 elements in registers, 40448 in LDS if the rows are 16-byte aligned,
    // the rest read twice.
    constexpr int L = kHybridLdsF4;
    const bool r20 = N > 81920 && N <= 138752;
    if (a16)
        return r20 ? launch_block(&softmax_hybrid_kernel<20, 4, true, 1024, L>, M, N, X, ldx, Y, ldy, s, 1024)
                   : launch_block(&softmax_hybrid_kernel<16, 6, true, 1024, L>, M, N, X, ldx, Y, ldy, s, 1024);
    return r20 ? launch_block(&softmax_hybrid_kernel<20, 4, false, 1024, L>, M, N, X, ldx, Y, ldy, s, 1024)
               : launch_block(&softmax_hybrid_kernel<16, 6, false, 1024, L>, M, N, X, ldx, Y, ldy, s, 1024);
}

}  // namespace

extern "C" int softmax_rows_f32(int64_t M, int64_t N, const float *X, int64_t ldx, float *Y, int64_t ldy,
                                void *stream)
{
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return GEMM_F16_ERR_DIM;
    if (M == 0 || N == 0) return GEMM_F16_OK;
    if (ldx < N || ldy < N || ldx > kMaxDim || ldy > kMaxDim) return GEMM_F16_ERR_LD;
    if (X == nullptr || Y == nullptr) return GEMM_F16_ERR_NULL;
    if ((uintptr_t)X % 4 != 0 || (uintptr_t)Y % 4 != 0) return GEMM_F16_ERR_ALIGN;
    const bool a16 = (uintptr_t)X % 16 == 0 && (uintptr_t)Y % 16 == 0 && ldx % 4 == 0 && ldy % 4 == 0;
    const bool ntl = M * N * 4 > (int64_t(256) << 20);   // X larger than the memory-attached cache
    hipStream_t s = static_cast<hipStream_t>(stream);
    // A launch counts its work-items along x in 32 bits, so rows go in chunks that keep
    // workgroups x threads below 2^32: 2^25 rows of up to 2048 elements (a wave per row, 2^31
    // threads), 2^21 longer rows (a workgroup of up to 1024 threads per row, 2^31 threads).
    const int64_t chunk = N <= 2048 ? (int64_t(1) << 25) : (int64_t(1) << 21);
    for (int64_t r0 = 0; r0 < M; r0 += chunk) {
        const int m = (int)(M - r0 < chunk ? M - r0 : chunk);
        const float *x = X + r0 * ldx;
        float *y = Y + r0 * ldy;
        const hipError_t err = ntl ? launch_softmax<true>(m, (int)N, x, ldx, y, ldy, s, a16)
                                   : launch_softmax<false>(m, (int)N, x, ldx, y, ldy, s, a16);
        if (err != hipSuccess) return GEMM_F16_ERR_LAUNCH;
    }
    return GEMM_F16_OK;
}
