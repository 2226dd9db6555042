// Measurement only (not on the product path): two microbenchmarks behind the design choices of the
// product kernel, compiled into the measurement library with the matrix-core ceiling.
//
// 1. LDS fragment reads (lds_read_probe).  Four waves of a workgroup read LDS in the patterns the
//    product's 256x256 tile uses -- the fragment of a 32-wide block for one k16 step -- with each
//    candidate XOR swizzle, and time the reads with s_memtime.  The reads are issued back to back,
//    so the figure is LDS throughput per wave with four waves contending (the product's situation:
//    one wave per SIMD).  The XOR swizzle exists to keep these reads conflict-free (04_tensor_cores.py,
//    CS349E lecture 10, "Tensor Core kernels", demo 2: 8-way / 4-way conflicts without it); this
//    measures what each key costs on gfx950.
//
// 2. Direct-to-LDS load latency (dma_latency_probe).  One wave per workgroup issues a
//    global_load_lds_dwordx4 (1 KiB: 64 lanes x 16 bytes, the product's load), waits for it, and
//    repeats; cycles and 100 MHz reference ticks per load give the latency of a load that hits L2
//    (a 1 MiB region per workgroup, re-read after a warming pass: too large for the vector L1, small
//    enough for the 4 MB L2 of its XCD) or that goes to HBM (a fresh 1 KiB window every time, 64 KiB
//    apart, in a buffer larger than the 256 MB memory-attached cache).  The pages size the number
//    of pipeline stages by Little's law from this latency and the time one stage takes to compute
//    (04_tensor_cores.py, demo 4).
//
// 3. LDS traffic mix (lds_mix_probe).  Four waves per workgroup, each round writing D KiB into LDS
//    (direct-to-LDS loads of 1 KiB from a region that its XCD's L2 holds, with up to three rounds in
//    flight; or ds_write_b128 from registers, with or without the global loads that fill them) and
//    issuing a set of fragment reads in the product's patterns; no matrix instructions.  A round with
//    D = 8 and the product's read set is what one wave of the 256x256 tile moves through LDS per K
//    slice, so comparing the round time with the main loop's time per slice shows whether LDS
//    traffic alone sets the loop's pace, and what staging through registers would change.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

// Read patterns (mode):
//  0..2  K-contiguous panel with 64-byte rows ([256][32] FP16), ds_read_b128; lane l reads row
//        d + l%32, chunk 2s + l/32 of step s.  Keys: 0 none, 1 (r>>1)&3, 2 (r ^ r>>2)&3.
//  3..4  K-contiguous panel with 128-byte rows ([256][64], two slices per row), ds_read_b128,
//        steps 0..3.  Keys: 3 none, 4 (r ^ r>>3)&7.
//  5     reference: 16 contiguous 1 KiB reads (lane l at 16 l), ds_read_b128.
//  6..7  K-row panel ([32][256] FP16, 512-byte rows), two ds_read_b64_tr_b16 per fragment: group
//        lane i of a 16-lane group addresses n = d + 16q + 4(i&3), k row 16s + 8(l/32) + i/4 + 4h.
//        Keys: 6 none, 7 2(r&3).
//  8     reference: 16 contiguous 512-byte ds_read_b64_tr_b16 (lane l at 8 l).
constexpr int kModes = 9;
constexpr int kReadsPerRound = 16;
constexpr int kLdsBytes = 96 * 1024;   // one workgroup per CU (two would need 192 KiB)

__device__ __forceinline__ int key_of(int mode, int r)
{
    switch (mode) {
    case 1: return (r >> 1) & 3;
    case 2: return (r ^ (r >> 2)) & 3;
    case 4: return (r ^ (r >> 3)) & 7;
    case 7: return 2 * (r & 3);
    default: return 0;
    }
}

// Byte address of read j (0..15) of a round for this lane.
__device__ __forceinline__ int read_address(int mode, int j, int wave, int lane)
{
    const int wm = wave >> 1, wn = wave & 1;
    if (mode <= 2) {                       // 4 blocks x 2 steps x (one b128) = 8 reads, twice
        const int jj = j & 7;
        const int row = wm * 128 + (jj >> 1) * 32 + (lane & 31);
        const int c = 2 * (jj & 1) + (lane >> 5);
        return row * 64 + ((c ^ key_of(mode, row)) * 16);
    }
    if (mode <= 4) {                       // 4 blocks x 4 steps
        const int row = wm * 128 + (j >> 2) * 32 + (lane & 31);
        const int c = 2 * (j & 3) + (lane >> 5);
        return row * 128 + ((c ^ key_of(mode, row)) * 16);
    }
    if (mode == 5) return j * 1024 + lane * 16;
    if (mode <= 7) {                       // 4 blocks x 2 steps x 2 halves
        const int blk = j >> 2, s = (j >> 1) & 1, h = j & 1;
        const int gi = lane & 15, q = (lane >> 4) & 1;
        const int n = wn * 128 + blk * 32 + 16 * q + 4 * (gi & 3);
        const int krow = 16 * s + 8 * (lane >> 5) + (gi >> 2) + 4 * h;
        return krow * 512 + (((n >> 3) ^ key_of(mode, krow)) * 16) + (n & 7) * 2;
    }
    return j * 512 + lane * 8;             // mode 8
}

// out[(block*4 + wave)*2 + {0,1}] = {shader cycles of the timed rounds, a value that keeps the reads live}
__global__ void __launch_bounds__(256) lds_read_probe_kernel(unsigned long long *out, int mode, int rounds)
{
    __shared__ __attribute__((aligned(1024))) char lds_raw[kLdsBytes];
    LDS_AS char *lds = (LDS_AS char *)lds_raw;
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    for (int o = t * 16; o < kLdsBytes; o += 256 * 16)
        *(LDS_AS u32x4 *)(lds + o) = u32x4{(uint32_t)o, (uint32_t)o * 3u + 1u, (uint32_t)o ^ 0x5a5au, 7u};
    int addr[kReadsPerRound];
#pragma unroll
    for (int j = 0; j < kReadsPerRound; ++j) addr[j] = read_address(mode, j, wave, lane);
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    short4_t acc2 = {0, 0, 0, 0};
    const bool tr = mode >= 6;
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    // Each round: two batches of 8 reads into distinct registers, issued before any is used (the
    // scheduling barrier keeps the compiler from interleaving the uses), so every wave keeps 8 reads
    // in flight -- the LDS pipe, not a wave's latency, sets the rate.
    for (int it = 0; it < rounds; ++it) {
        int off = 0;
        asm volatile("" : "+v"(off));      // opaque: the reads are issued again every round
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (tr) {
                short4_t v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    v[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t *)(lds + addr[half * 8 + j] + off));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc2 ^= v[j];
            } else {
                u32x4 v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = *(const LDS_AS u32x4 *)(lds + addr[half * 8 + j] + off);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 8; ++j) acc ^= v[j];
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint32_t keep = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ (uint16_t)acc2[0] ^ (uint16_t)acc2[1] ^
                          (uint16_t)acc2[2] ^ (uint16_t)acc2[3];
    if (lane == 0) {
        unsigned long long *d = out + ((size_t)blockIdx.x * 4 + wave) * 2;
        d[0] = t1 - t0;
        d[1] = keep;
    }
}

// Latency of one direct-to-LDS load: offset(i) = blockIdx.x * group_stride + (i % windows) * stride.
// With `warm`, one untimed pass over the windows first.  out[block*3 + {0,1,2}] = {shader cycles,
// reference ticks, loads timed}.
__global__ void __launch_bounds__(64) dma_latency_probe_kernel(const char *src, uint64_t bytes,
                                                               unsigned long long *out, int iters, int windows,
                                                               uint64_t stride, uint64_t group_stride, int warm)
{
    __shared__ __attribute__((aligned(1024))) char win[1024];
    const uint32_t lds = (uint32_t)(uintptr_t)(LDS_AS char *)win;
    const uint32_t lane_off = (uint32_t)(threadIdx.x & 63) * 16u;
    const uint64_t base = (uint64_t)blockIdx.x * group_stride;
    auto load = [&](int i) {
        const uint64_t o = base + (uint64_t)(i % windows) * stride;
        if (o + 1024 > bytes) return;      // the host checks this never happens; kept as a guard
        const char *p = src + o;
        asm volatile("s_mov_b32 m0, %2\n\t"
                     "s_nop 0\n\t"
                     "global_load_lds_dwordx4 %0, %1\n\t"
                     "s_waitcnt vmcnt(0)"
                     :
                     : "v"(lane_off), "s"(p), "s"(lds)
                     : "memory");
    };
    if (warm)
        for (int i = 0; i < windows; ++i) load(i);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < iters; ++i) load(i);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
        unsigned long long *d = out + (size_t)blockIdx.x * 3;
        d[0] = t1 - t0;
        d[1] = r1 - r0;
        d[2] = (unsigned long long)iters;
    }
}

// Read sets of the mix probe (per wave per round):
//  0  none;
//  1  16 ds_read_b128 of the paired K-contiguous panel (pattern 4 above): 16 KiB;
//  2  8 ds_read_b128 (pattern 4) + 16 ds_read_b64_tr_b16 of the K-row panel (pattern 7): 16 KiB, the
//     256x256 tile's fragments for one BK = 32 slice in the NN layout;
//  3  4 ds_read_b128 + 8 ds_read_b64_tr_b16: 8 KiB, the K-split tile's fragments for one BK = 64 slice.
constexpr int kMixKinds = 4;
constexpr int kMixLds = 96 * 1024;       // read panels in the first 48 KiB; 8 KiB of load windows per wave at 64 KiB
constexpr int kMixTrBase = 32 * 1024;    // the K-row panel ([32][256] FP16) after the [256][64] one
constexpr int kMixDmaBase = 64 * 1024;

template <int N>
__device__ __forceinline__ void kc_batch(const LDS_AS char *lds, const int *addr, int off, u32x4 &acc)
{
    u32x4 v[N];
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = *(const LDS_AS u32x4 *)(lds + addr[j] + off);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < N; ++j) acc ^= v[j];
}

__device__ __forceinline__ void tr_batch(LDS_AS char *lds, const int *addr, int off, short4_t &acc)
{
    short4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t *)(lds + addr[j] + off));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc ^= v[j];
}

// Load window i of this workgroup's region lies at src + blockIdx.x * region + (i % (region / 1024)) * 1024;
// the host checks grid * region <= bytes.  out[(block*4 + wave)*2 + {0,1}] = {shader cycles of the
// timed rounds, a value that keeps the reads live}.
// WRITER 0: the D KiB per round arrive by direct-to-LDS loads; 1: by ds_write_b128 from registers
// (no memory traffic: the LDS side of register staging alone); 2: by global_load_dwordx4 into
// registers, written with ds_write_b128 one round later (register staging, two register sets);
// 3: half each way (one operand staged through registers, the other loaded direct-to-LDS).
template <int D, int WRITER>
__global__ void __launch_bounds__(256) lds_mix_probe_kernel(const char *src, uint64_t bytes, uint64_t region,
                                                            unsigned long long *out, int kind, int rounds)
{
    __shared__ __attribute__((aligned(1024))) char lds_raw[kMixLds];
    LDS_AS char *lds = (LDS_AS char *)lds_raw;
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    for (int o = t * 16; o < kMixLds; o += 256 * 16)
        *(LDS_AS u32x4 *)(lds + o) = u32x4{(uint32_t)o, (uint32_t)o * 3u + 1u, (uint32_t)o ^ 0x5a5au, 7u};
    int a_kc[16], a_tr[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        a_kc[j] = read_address(4, j, wave, lane);
        a_tr[j] = kMixTrBase + read_address(7, j, wave, lane);
    }
    const uint32_t dma0 = (uint32_t)(uintptr_t)(lds + kMixDmaBase + wave * 8192);
    const uint32_t lane_off = (uint32_t)lane * 16u;
    // The host guarantees grid * region <= bytes; a workgroup past it would read the first region
    // (a branch-free guard, so the compiler's load counting stays exact).
    const uint64_t base = (uint64_t)blockIdx.x * region + region <= bytes ? (uint64_t)blockIdx.x * region : 0;
    const int windows = (int)(region / 1024);
    __syncthreads();
    u32x4 acc = {0u, 0u, 0u, 0u};
    short4_t acc2 = {0, 0, 0, 0};
    int w = 0;
    LDS_AS char *wbase = lds + kMixDmaBase + wave * 8192 + lane * 16;   // this lane's 16 bytes of window 0
    constexpr int DR = D > 0 ? D : 1;
    u32x4 set0[DR], set1[DR];              // WRITER 1: values to write; WRITER 2: two register sets
#pragma unroll
    for (int j = 0; j < DR; ++j) set0[j] = set1[j] = u32x4{(uint32_t)j, (uint32_t)lane, 3u, 5u};
    constexpr int RS = WRITER == 3 ? D / 2 : D;   // KiB per round staged through registers (WRITER 2, 3)
    constexpr int DL = WRITER == 3 ? D / 2 : D;   // KiB per round loaded direct-to-LDS (WRITER 0, 3)
    constexpr int DOFF = WRITER == 3 ? D / 2 : 0; // their first window after the staged ones
    auto load_set = [&](u32x4 *dst) {
#pragma unroll
        for (int j = 0; j < RS; ++j) {
            dst[j] = *(const u32x4 *)(src + base + (uint64_t)w * 1024 + lane_off);
            w = w + 1 == windows ? 0 : w + 1;
        }
    };
    // One round: its D KiB of LDS writes and its fragment reads.  WRITER 2 loads `next` and writes
    // `cur`, which the previous round loaded (the two sets alternate, so no register is copied and
    // a round waits only for the loads issued a round earlier).
    auto round = [&](int it, u32x4 *cur, u32x4 *next) {
        int off = 0;
        asm volatile("" : "+v"(off));      // opaque: the reads are issued again every round
        if constexpr (WRITER == 1) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                u32x4 v = cur[j];
                v[0] += (uint32_t)it;
                *(LDS_AS u32x4 *)(wbase + (((it * D + j) & 7) * 1024)) = v;
            }
        }
        if constexpr (WRITER >= 2) load_set(next);
        if constexpr (WRITER == 0 || WRITER == 3) {
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                const char *p = src + base + (uint64_t)w * 1024;
                w = w + 1 == windows ? 0 : w + 1;
                const uint32_t dst = dma0 + (uint32_t)(((it * D + DOFF + j) & 7) * 1024);
                asm volatile("s_mov_b32 m0, %2\n\t"
                             "s_nop 0\n\t"
                             "global_load_lds_dwordx4 %0, %1"
                             :
                             : "v"(lane_off), "s"(p), "s"(dst)
                             : "memory");
            }
        }
        if (kind == 1) {
            kc_batch<8>(lds, a_kc, off, acc);
            kc_batch<8>(lds, a_kc + 8, off, acc);
        } else if (kind == 2) {
            kc_batch<8>(lds, a_kc, off, acc);
            tr_batch(lds, a_tr, off, acc2);
            tr_batch(lds, a_tr + 8, off, acc2);
        } else if (kind == 3) {
            kc_batch<4>(lds, a_kc, off, acc);
            tr_batch(lds, a_tr, off, acc2);
        }
        if constexpr (WRITER == 0) {
            // At most three rounds of loads in flight: wait for the one issued two rounds ago.
            if constexpr (D == 2) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
            if constexpr (D == 4) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            if constexpr (D == 8) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
            if constexpr (D == 16) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
        }
        if constexpr (WRITER >= 2) {
            // (WRITER 3: the compiler does not count the direct-to-LDS loads, so its waits here are
            // stricter than they need to be, never looser.)
#pragma unroll
            for (int j = 0; j < RS; ++j) *(LDS_AS u32x4 *)(wbase + (((it * D + j) & 7) * 1024)) = cur[j];
        }
    };
    if constexpr (WRITER >= 2) load_set(set0);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < rounds; it += 2) {   // rounds is even (checked on the host)
        round(it, set0, set1);
        round(it + 1, set1, set0);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    uint32_t keep = acc[0] ^ acc[1] ^ acc[2] ^ acc[3] ^ (uint16_t)acc2[0] ^ (uint16_t)acc2[1] ^
                    (uint16_t)acc2[2] ^ (uint16_t)acc2[3];
#pragma unroll
    for (int j = 0; j < DR; ++j) keep ^= set0[j][0] ^ set1[j][3];
    if (lane == 0) {
        unsigned long long *d = out + ((size_t)blockIdx.x * 4 + wave) * 2;
        d[0] = t1 - t0;
        d[1] = keep;
    }
}

// 4. Vector-memory load patterns (vmem_pattern_probe): four waves per workgroup, each round issuing 8
//    global_load_dwordx4 into registers (two register sets, so a round waits only for the loads of
//    the round before) from a 64 KiB region per workgroup viewed as 512 rows of 128 bytes, in one of
//    five patterns: 0 contiguous 1 KiB (8 whole cache lines per load); 1 the A fragment of a
//    16x16x32 MFMA (16 rows x 64 bytes per load, the two halves of each row's line in consecutive
//    loads); 2 the A fragment of a 32x32x16 MFMA (32 rows x 32 bytes per load, a line's four
//    quarters in four consecutive loads); 3 and 4 contiguous 1 KiB starting 2 and 4 bytes past a
//    16-byte boundary (the 16-byte loads of rows whose stride is odd, or a multiple of 2 elements but
//    not of 8); 5 one 2-byte load per lane at 16-byte spacing (the last element of each lane's chunk);
//    6 a realigned chunk: 16 bytes from the 4-byte boundary below a chunk that starts 2 bytes past
//    one, plus the chunk's last element as a 2-byte load.  It measures what the load path charges for
//    fragments read straight from memory, and for misaligned 16-byte loads and their realignment,
//    against whole aligned lines.
constexpr int kPatternRows = 512;         // rows of 128 bytes: 64 KiB per workgroup

template <int P>
__device__ __forceinline__ uint32_t pattern_offset(int it, int j, int lane)
{
    if (P == 0) return (uint32_t)(((it * 8 + j) & 63) * 1024 + lane * 16);
    if (P == 3) return (uint32_t)(((it * 8 + j) & 63) * 1024 + lane * 16 + 2);
    if (P == 4) return (uint32_t)(((it * 8 + j) & 63) * 1024 + lane * 16 + 4);
    if (P == 1) {
        const int row = (((it * 4 + (j >> 1)) & (kPatternRows / 16 - 1)) * 16) + (lane & 15);
        return (uint32_t)(row * 128 + (j & 1) * 64 + (lane >> 4) * 16);
    }
    const int row = (((it * 2 + (j >> 2)) & (kPatternRows / 32 - 1)) * 32) + (lane & 31);
    return (uint32_t)(row * 128 + (j & 3) * 32 + (lane >> 5) * 16);
}

template <int P>
__global__ void __launch_bounds__(256) vmem_pattern_probe_kernel(const char *src, uint64_t bytes,
                                                                 unsigned long long *out, int rounds)
{
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    const uint64_t region = (uint64_t)kPatternRows * 128;
    // The host guarantees grid * region + 64 <= bytes; past it a workgroup reads the first region.
    const char *base = src + ((uint64_t)(blockIdx.x + 1) * region + 64 <= bytes ? (uint64_t)blockIdx.x * region : 0);
    typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));   // 16 bytes at any 2-byte alignment
    u32x4 set0[8], set1[8];
    u32x4 acc = {0u, 0u, 0u, 0u};
    typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
    auto load = [&](int it, u32x4 *dst) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t o = (uint32_t)(((it * 8 + j) & 63) * 1024 + lane * 16);
            if constexpr (P == 5) {
                const uint32_t h = *(const uint16_t *)(base + o + 14);
                dst[j] = u32x4{h, 0u, 0u, 0u};
            } else if constexpr (P == 6) {
                const u32x4_a4 w = *(const u32x4_a4 *)(base + o);   // the chunk starts at o + 2
                const uint32_t h = *(const uint16_t *)(base + o + 2 + 14);
                dst[j] = u32x4{__builtin_amdgcn_alignbyte(w[1], w[0], 2u), __builtin_amdgcn_alignbyte(w[2], w[1], 2u),
                               __builtin_amdgcn_alignbyte(w[3], w[2], 2u), __builtin_amdgcn_alignbyte(h, w[3], 2u)};
            } else {
                const u32x4_a2 v = *(const u32x4_a2 *)(base + pattern_offset<P>(it, j, lane));
                dst[j] = u32x4{v[0], v[1], v[2], v[3]};
            }
        }
    };
    auto use = [&](const u32x4 *v) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc ^= v[j];
    };
    load(0, set0);
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int it = 1; it < rounds; it += 2) {   // rounds is odd (checked on the host)
        load(it, set1);
        use(set0);
        load(it + 1, set0);
        use(set1);
    }
    use(set0);
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) {
        unsigned long long *d = out + ((size_t)blockIdx.x * 4 + wave) * 2;
        d[0] = t1 - t0;
        d[1] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    }
}

}  // namespace

extern "C" {

// `grid` workgroups of 4 waves, each wave issuing rounds x 16 LDS reads in pattern `mode`
// (0 .. 8).  out: grid*4*2 u64 device buffer.  Returns 0, -1 for bad arguments, -6 if the launch
// failed.
int gemm_f16_lds_read_probe(void *out, int grid, int mode, int rounds, void *stream)
{
    if (out == nullptr || grid <= 0 || grid > 65536 || mode < 0 || mode >= kModes || rounds <= 0 ||
        rounds > 1000000)
        return -1;
    void *args[] = {(void *)&out, (void *)&mode, (void *)&rounds};
    return hipLaunchKernel(reinterpret_cast<const void *>(&lds_read_probe_kernel), dim3((unsigned)grid), dim3(256),
                           args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : -6;
}

// `grid` one-wave workgroups, each timing `iters` dependent 1 KiB direct-to-LDS loads from
// src + blockIdx.x * group_stride + (i % windows) * stride (after one warming pass when `warm`).
// Every load must lie inside [src, src + bytes): returns -1 otherwise (nothing launched).
// out: grid*3 u64 device buffer.  Returns 0, -1 for bad arguments, -6 if the launch failed.
int gemm_f16_dma_latency_probe(const void *src, uint64_t bytes, void *out, int grid, int iters, int windows,
                               uint64_t stride, uint64_t group_stride, int warm, void *stream)
{
    if (src == nullptr || out == nullptr || grid <= 0 || grid > 65536 || iters <= 0 || iters > 1000000 ||
        windows <= 0 || (uintptr_t)src % 16 != 0 || stride % 16 != 0 || group_stride % 16 != 0)
        return -1;
    const uint64_t last = (uint64_t)(grid - 1) * group_stride + (uint64_t)(windows - 1) * stride + 1024;
    if (last > bytes) return -1;
    const char *s = static_cast<const char *>(src);
    void *args[] = {(void *)&s, (void *)&bytes, (void *)&out, (void *)&iters, (void *)&windows,
                    (void *)&stride, (void *)&group_stride, (void *)&warm};
    return hipLaunchKernel(reinterpret_cast<const void *>(&dma_latency_probe_kernel), dim3((unsigned)grid), dim3(64),
                           args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : -6;
}

// `grid` workgroups of 4 waves, each wave running `rounds` (even) rounds of `writes_per_round` (0, 2,
// 4, 8, or 16 with writer 0) KiB written into LDS by `writer` (0 direct-to-LDS loads, 1 ds_write_b128
// from registers, 2 global loads staged through registers, 3 half by each of 0 and 2) from its
// workgroup's `region` bytes of src, and read set `kind` (0 .. 3).  region: a multiple of 1024 bytes,
// grid * region <= bytes.  out: grid*4*2 u64 device buffer.  Returns 0, -1 for bad arguments (nothing
// launched), -6 if the launch failed.
int gemm_f16_lds_mix_probe(const void *src, uint64_t bytes, uint64_t region, void *out, int grid,
                           int writes_per_round, int writer, int kind, int rounds, void *stream)
{
    if (src == nullptr || out == nullptr || grid <= 0 || grid > 65536 || kind < 0 || kind >= kMixKinds ||
        rounds <= 0 || rounds > 1000000 || (uintptr_t)src % 16 != 0 || region < 1024 || region % 1024 != 0 ||
        region > (1ull << 30) || (uint64_t)grid * region > bytes || writer < 0 || writer > 3 || rounds % 2 != 0)
        return -1;
    const void *fn = nullptr;
#define MIX_CASE(D)                                                                                      \
    case D:                                                                                              \
        fn = writer == 0   ? reinterpret_cast<const void *>(&lds_mix_probe_kernel<D, 0>)                 \
             : writer == 1 ? reinterpret_cast<const void *>(&lds_mix_probe_kernel<D, 1>)                 \
             : writer == 2 ? reinterpret_cast<const void *>(&lds_mix_probe_kernel<D, 2>)                 \
                           : reinterpret_cast<const void *>(&lds_mix_probe_kernel<D, 3>);                \
        break;
    switch (writes_per_round) {
    case 0: fn = reinterpret_cast<const void *>(&lds_mix_probe_kernel<0, 0>); break;
    MIX_CASE(2)
    MIX_CASE(4)
    MIX_CASE(8)
    case 16:
        if (writer != 0) return -1;
        fn = reinterpret_cast<const void *>(&lds_mix_probe_kernel<16, 0>);
        break;
    default: return -1;
    }
#undef MIX_CASE
    const char *s = static_cast<const char *>(src);
    void *args[] = {(void *)&s, (void *)&bytes, (void *)&region, (void *)&out, (void *)&kind, (void *)&rounds};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : -6;
}

// `grid` workgroups of 4 waves, each wave issuing `rounds` (odd) rounds of 8 global_load_dwordx4 in
// pattern `pattern` (0 .. 6) over its workgroup's 64 KiB of src; grid * 64 KiB + 64 <= bytes (the
// misaligned patterns read up to 4 bytes past a workgroup's 64 KiB).  out: grid*4*2 u64 device
// buffer.  Returns 0, -1 for bad arguments (nothing launched), -6 if the launch failed.
int gemm_f16_vmem_pattern_probe(const void *src, uint64_t bytes, void *out, int grid, int pattern, int rounds,
                                void *stream)
{
    if (src == nullptr || out == nullptr || grid <= 0 || grid > 65536 || pattern < 0 || pattern > 6 ||
        rounds <= 0 || rounds > 1000000 || rounds % 2 != 1 || (uintptr_t)src % 16 != 0 ||
        (uint64_t)grid * kPatternRows * 128 + 64 > bytes)
        return -1;
    const void *fn = pattern == 0   ? reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<0>)
                     : pattern == 1 ? reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<1>)
                     : pattern == 2 ? reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<2>)
                     : pattern == 3 ? reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<3>)
                     : pattern == 4 ? reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<4>)
                     : pattern == 5 ? reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<5>)
                                    : reinterpret_cast<const void *>(&vmem_pattern_probe_kernel<6>);
    const char *s = static_cast<const char *>(src);
    void *args[] = {(void *)&s, (void *)&bytes, (void *)&out, (void *)&rounds};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(256), args, 0, static_cast<hipStream_t>(stream)) == hipSuccess
               ? 0
               : -6;
}

}  // extern "C"
