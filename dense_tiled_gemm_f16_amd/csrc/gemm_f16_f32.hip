// gfx950 (MI355X, CDNA4) FP16-input, FP32-accumulate block-tiled matrix product: the kernels and
// their launchers (argument checks, plans and the C ABI are in gemm_api.hip).
//
// C <- op(A).op(B) + beta.C, A and B binary16 (each as given or transposed), C binary32,
// row-major with leading dimensions.
//
// The method is the block-tiled product the pages describe (04_tensor_cores.py, CS349E
// lecture 10, "Tensor Core kernels": one workgroup per BM x BN output tile, K streamed in BK
// slices through on-chip shared memory into matrix-instruction fragments, an XOR swizzle
// against bank conflicts, several stages in flight sized by Little's law; 06_triton_style.py,
// "block programming": grouped launch order and masks for ragged edges), re-designed for gfx950:
//
//  * Matrix instruction: v_mfma_f32_32x32x16_f16 on 64-lane waves.  For D = X.Y + D with X
//    32 x 16 and Y 16 x 32, lane l supplies row l%32 of X and column l%32 of Y, each as 8 k
//    values (k = 8*(l/32) .. +7), and holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator
//    register r.  The kernel feeds the B fragment as X and the A fragment as Y, so the
//    accumulator holds a block of C^T: lane l owns row l%32 of the C block and, for each group
//    g of four registers, the four consecutive columns 8g + 4*(l/32) .. +3 (one 16-byte store).
//  * Global -> LDS: interior tiles use the direct-to-LDS load (global_load_lds_dwordx4): each
//    instruction moves 1 KiB, lane l's 16 bytes landing at LDS offset 16*l of the instruction's
//    window.  No registers and no ALU work are spent on staging.  The XOR swizzle is therefore
//    applied on the global side: lane l fetches the logical chunk that belongs at its position.
//  * Each operand's panel is kept in LDS the way it lies in memory.  A K-contiguous panel (A as
//    given, B transposed) is [rows][k]; the fragment is one ds_read_b128 per lane.  Chunk c of
//    row r sits at chunk c ^ key(r): key = (r ^ r>>3) & 7 for 8-chunk rows, (r ^ r>>2) & 3 for
//    4-chunk rows.  Both make a fragment read (32 consecutive rows at one logical chunk) run at
//    the rate of a contiguous 1 KiB read; with (r >> 1) & 3 the 4-chunk case measures 2-way
//    conflicted.  With BK = 32 such a panel is loaded two slices at a time as 128-byte rows
//    (the paired layout below): a load then touches whole cache lines.
//  * A K-row panel (B as given, A transposed) is [k][outer]; the fragment (8 consecutive k of
//    one column per lane) comes from two ds_read_b64_tr_b16.  That instruction works on groups
//    of 16 lanes: group lane i receives, as element e, element i%4 of the 8 bytes that group
//    lane 4e + i/4 addressed.  So lanes addressing a 4 (k) x 16 (n) block, four lanes per k row,
//    receive one column's 4 k values each.  Chunk c of k row r sits at chunk c ^ 2*(r & 3);
//    measured, this read pattern then runs as fast as a contiguous 512-byte read, while the
//    unswizzled layout (every k row starting on the same banks) takes 1.6x as long.
//  * LDS ring, one barrier per K slice, placed before the slice's last k16 step: every wave has
//    waited for its own loads of the next slice, and the buffer read so far may be refilled.
//    Loads are slotted one at a time between MFMAs; waits and barriers are explicit (s_waitcnt
//    with the count of loads still allowed in flight), not fences that would drain every load.
//  * Edge tiles (crossing M or N) stay on the direct path with clamped sources; operands whose
//    rows are not 16-byte aligned are staged through registers into the same LDS layout; the
//    last partial K slice takes a masked path whose out-of-range elements read as 0.
//  * Launch order: grouped order, optionally after an XCD renumbering (tile_order.h).
//  * Split-K (the launch's y dimension) moves the operands' K origin and writes a slice of the
//    caller's workspace; the second pass is in splitk_reduce.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "gemm_f16.h"
#include "gemm_launch.h"

#ifndef GEMM_F16_STAGGER_LOADS
#define GEMM_F16_STAGGER_LOADS 1
#endif
#ifndef GEMM_F16_DMA_CLAMP
#define GEMM_F16_DMA_CLAMP 1
#endif
#ifndef GEMM_F16_C_PREFETCH
#define GEMM_F16_C_PREFETCH 1
#endif
#ifndef GEMM_F16_REG_PAIRED
#define GEMM_F16_REG_PAIRED 1
#endif
// 0: every LDS panel row keeps its chunks in order (no XOR swizzle).  A variant of the library built
// this way computes the same bits with a different LDS address map; it exists for measurement and
// tests only.
#ifndef GEMM_F16_SWIZZLE
#define GEMM_F16_SWIZZLE 1
#endif
// The operand layout whose kernels this translation unit instantiates: the library is built from
// four objects of this file, (GEMM_F16_TA, GEMM_F16_TB) = (0,0), (0,1), (1,0), (1,1), compiled in
// parallel; gemm_api.hip dispatches a call to the launcher of its layout.
// 1 in a measurement build only (never the product library): thread 0 of every workgroup stamps
// the shader clock at the phase boundaries of its tile into a buffer set through
// gemm_f16_phase_buffer_<layout> (see phase_mark).
#ifndef GEMM_F16_PHASES
#define GEMM_F16_PHASES 0
#endif
#ifndef GEMM_F16_TA
#define GEMM_F16_TA 0
#endif
#ifndef GEMM_F16_TB
#define GEMM_F16_TB 0
#endif
#include "tile_order.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float float4_a4 __attribute__((ext_vector_type(4), aligned(4)));  // C rows at 4-byte alignment

#define LDS_AS __attribute__((address_space(3)))

using gemm_f16::Params;
using gemm_f16::TileInfo;

// KS > 1: KS groups of WGM x WGN waves split each K slice: group g computes its output block over
// the k16 steps s with s % KS == g, and the groups' partial sums are added in the epilogue.
//
// TA / TB: A is given transposed (stored K x M) / B is given transposed (stored N x K).  Each
// operand's slice is kept in LDS the way it lies in memory: a K-contiguous operand (A as given, B
// transposed) as a [D][BK] panel read with ds_read_b128, the other kind (B as given, A transposed)
// as a [BK][D] panel read with transposing reads; D is BM for A and BN for B.
template <int BM_, int BN_, int BK_, int S_, int WGM_, int WGN_, int WPE_ = 1, int KS_ = 1, bool TA_ = false,
          bool TB_ = false>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_;
    static constexpr int WPE = WPE_;                      // waves per SIMD the kernel is built for
    static constexpr int WGM = WGM_, WGN = WGN_, KS = KS_;
    static constexpr bool TA = TA_, TB = TB_;
    static constexpr bool A_KC = !TA, B_KC = TB;          // K-contiguous panels
    static constexpr int W = WGM * WGN * KS;              // waves per workgroup
    static constexpr int T = 64 * W;                      // threads per workgroup
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // per-wave output tile
    static constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA blocks per wave
    static constexpr int A_ROWS = A_KC ? BM : BK, B_ROWS = B_KC ? BN : BK;   // LDS panel rows
    static constexpr int A_ROW = (A_KC ? BK : BM) * 2, B_ROW = (B_KC ? BK : BN) * 2;  // row bytes
    static constexpr int A_CH = A_ROW / 16, B_CH = B_ROW / 16;  // 16-byte chunks per panel row
    static constexpr int A_BYTES = A_ROWS * A_ROW, B_BYTES = B_ROWS * B_ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = S * STAGE;
    static constexpr int A_DMA_W = A_BYTES / 1024 / W;    // direct-to-LDS A loads per wave per slice
    static constexpr int A_PER_T = A_ROWS * A_CH / T;     // masked path: chunks per thread
    static constexpr int B_PER_T = B_ROWS * B_CH / T;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BK == 32 || BK == 64, "BK must be 32 or 64");
    static_assert(A_KC || A_CH >= 8, "K-row panels need at least 8 chunks per row for the swizzle");
    static_assert(B_KC || B_CH >= 8, "K-row panels need at least 8 chunks per row for the swizzle");
    static_assert(A_PER_T >= 1 && A_PER_T * T == A_ROWS * A_CH, "masked A chunks must split evenly");
    static_assert(B_PER_T >= 1 && B_PER_T * T == B_ROWS * B_CH, "masked B chunks must split evenly");
    static_assert(S >= 2, "at least two LDS stages");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((BK / 16) % KS == 0, "each K group takes the same number of k16 steps");
};

template <class TL, bool TA, bool TB>
using WithLayout = Tile<TL::BM, TL::BN, TL::BK, TL::S, TL::WGM, TL::WGN, TL::WPE, TL::KS, TA, TB>;

// ---------------------------------------------------------------- phase stamps (measurement builds)
// Record k of a workgroup's eight: 0 entry, 1 main-loop prologue done (first ring barrier passed),
// 2 main loop done, 3 masked K tail done, 4 epilogue done (shader clock, s_memtime); 5 and 6 the
// 100 MHz reference clock at entry and at the end; 7 the hardware id (XCC in the high half, HW_ID
// in the low half), which names the CU.
#if GEMM_F16_PHASES
__device__ unsigned long long *phase_times;
#endif

__device__ __forceinline__ void phase_mark(int k)
{
#if GEMM_F16_PHASES
    if (threadIdx.x == 0 && phase_times != nullptr) {
        unsigned long long *rec = phase_times + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 8;
        if (k == 0) {
            uint32_t hw, xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            rec[7] = ((unsigned long long)xcc << 32) | hw;
            rec[5] = __builtin_amdgcn_s_memrealtime();
        }
        rec[k] = __builtin_amdgcn_s_memtime();
        if (k == 4) rec[6] = __builtin_amdgcn_s_memrealtime();
    }
#else
    (void)k;
#endif
}

// ---------------------------------------------------------------- small device helpers
template <int A_CH>
__device__ __forceinline__ int a_key(int row)
{
    if (!GEMM_F16_SWIZZLE) return 0;
    return A_CH == 8 ? ((row ^ (row >> 3)) & 7) : ((row ^ (row >> 2)) & 3);
}

template <int B_CH>
__device__ __forceinline__ int b_key(int krow)  // B_CH >= 8
{
    if (!GEMM_F16_SWIZZLE) return 0;
    return 2 * (krow & 3);
}

// Swizzle of a panel row: K-contiguous panels (4 or 8 chunks per row) use a_key, K-row panels
// (at least 8 chunks per row) b_key.
template <int CH, bool KC>
__device__ __forceinline__ int panel_key(int row)
{
    if constexpr (KC)
        return a_key<CH>(row);
    else
        return b_key<CH>(row);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroup barrier without a memory fence: the waits that make data visible are explicit.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// ---------------------------------------------------------------- direct-to-LDS staging
// One direct-to-LDS load: 16 bytes per lane from base + off into LDS [lds + lds_off + 16*lane].
// Issued as inline assembly so that the compiler neither orders it against LDS reads of other
// buffers nor inserts waits for it; the ring's explicit vmcnt waits and barriers order it.  M0
// (the instruction's LDS base) is written directly: nothing else in this library uses M0 (a
// host test checks the compiled code for that), so it is neither saved nor restored, which keeps
// each load at three instructions -- with one wave per SIMD, issue slots between MFMAs are the
// scarce resource.  One wait state separates the M0 write from the load.  The add that forms M0
// writes SCC, which is declared clobbered: otherwise the compiler may keep a carry in SCC across
// the block (the low and high halves of a 64-bit address add on either side of it), and the
// address comes out 2^32 bytes off.
__device__ __forceinline__ void dma16(const char *base, uint32_t off, uint32_t lds, uint32_t lds_off)
{
    asm volatile("s_add_u32 m0, %2, %3\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds), "s"(lds_off)
                 : "memory", "scc");
}

// A stage is split into 1 KiB windows; NW waves issue them, wave w taking windows
// w*PER .. w*PER + PER-1 of A and of B.  Lane l fills bytes 16l .. 16l+15 of a window, so
// it fetches the logical chunk the swizzle places there.
template <class TL, int NW>
struct DmaPlan {
    static constexpr int A = TL::A_BYTES / 1024 / NW;
    static constexpr int B = TL::B_BYTES / 1024 / NW;
    static constexpr int COUNT = A + B;   // loads per wave per slice
    static_assert(A >= 1 && A * 1024 * NW == TL::A_BYTES, "A stage must split into 1 KiB per wave");
    static_assert(B >= 1 && B * 1024 * NW == TL::B_BYTES, "B stage must split into 1 KiB per wave");
};

// Byte offset, from the operand's base at this slice, of the chunk lane `lane` fills in window w of
// a panel.  vd: the tile's valid extent along the operand's outer dimension (rows of M for A,
// columns of N for B).
//  * K-contiguous panel: panel row = outer index; rows at or past vd re-read row vd-1.  They only
//    feed C elements that are never stored, and every address stays inside the operand.
//  * K-row panel: panel row = k row; chunks starting at or past vd re-read the last chunk that
//    starts inside the matrix.  That chunk may extend up to 7 elements past the matrix edge, which
//    stays inside the operand for every k row but the last (the caller keeps the slice holding
//    k row K-1 off this path in tiles that cross that edge).
template <int ROW_BYTES, int CH, bool KC>
__device__ __forceinline__ uint32_t panel_dma_offset(int64_t ld, int w, int lane, int vd)
{
    const int byte = w * 1024 + lane * 16;
    const int row = byte / ROW_BYTES;
    const int c = ((byte % ROW_BYTES) / 16) ^ panel_key<CH, KC>(row);
    if constexpr (KC) {
        const int src = row < vd ? row : vd - 1;
        return (uint32_t)((src * ld + c * 8) * 2);
    } else {
        const int src = c * 8 < vd ? c : (vd - 1) / 8;
        return (uint32_t)((row * ld + src * 8) * 2);
    }
}

template <class TL>
__device__ __forceinline__ uint32_t a_dma_offset(const Params &p, int w, int lane, int rows)
{
    return panel_dma_offset<TL::A_ROW, TL::A_CH, TL::A_KC>(p.lda, w, lane, rows);
}

template <class TL>
__device__ __forceinline__ uint32_t b_dma_offset(const Params &p, int w, int lane, int cols)
{
    return panel_dma_offset<TL::B_ROW, TL::B_CH, TL::B_KC>(p.ldb, w, lane, cols);
}

// Where each operand's panel of slice 0 starts, and the byte step from one slice to the next.
template <class TL>
struct PanelBases {
    const char *abase, *bbase;
    int64_t a_step, b_step;
    __device__ __forceinline__ PanelBases(const Params &p, int m0, int n0)
    {
        abase = (const char *)(TL::A_KC ? p.A + (int64_t)m0 * p.lda : p.A + m0);
        bbase = (const char *)(TL::B_KC ? p.B + (int64_t)n0 * p.ldb : p.B + n0);
        a_step = TL::A_KC ? (int64_t)TL::BK * 2 : (int64_t)TL::BK * p.lda * 2;
        b_step = TL::B_KC ? (int64_t)TL::BK * 2 : (int64_t)TL::BK * p.ldb * 2;
    }
};

// Per-lane global offsets and per-wave LDS offsets of this wave's loads of a slice, A windows first.
template <class TL>
__device__ __forceinline__ void dma_lane_offsets(const Params &p, int wave, int lane, int rows, int cols,
                                                 uint32_t (&off)[DmaPlan<TL, TL::W>::COUNT],
                                                 uint32_t (&dst)[DmaPlan<TL, TL::W>::COUNT])
{
    using D = DmaPlan<TL, TL::W>;
#pragma unroll
    for (int d = 0; d < D::COUNT; ++d) {
        if (d < D::A) {
            const int w = wave * D::A + d;
            off[d] = a_dma_offset<TL>(p, w, lane, rows);
            dst[d] = (uint32_t)(w * 1024);
        } else {
            const int w = wave * D::B + (d - D::A);
            off[d] = b_dma_offset<TL>(p, w, lane, cols);
            dst[d] = (uint32_t)(TL::A_BYTES + w * 1024);
        }
    }
}

// ---------------------------------------------------------------- masked staging
// A chunk q = t + i*T: row q / A_CH, k chunk q % A_CH.  B chunk q: k row q / B_CH, n chunk q % B_CH.
template <class TL>
struct Regs {
    u32x4 a[TL::A_PER_T];
    u32x4 b[TL::B_PER_T];
};

// 16 bytes of FP16 at any 2-byte alignment: rows whose stride is not a multiple of 8 elements are
// still read one 16-byte load per chunk (the target allows unaligned multi-dword global accesses,
// and the compiler emits global_load_dwordx4 for this type).
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));

__device__ __forceinline__ u32x4 masked_chunk(const uint16_t *row_ptr, int col, int limit, bool row_ok)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row_ok && col < limit) {
        if (col + 8 <= limit) {
            const u32x4_a2 w = *reinterpret_cast<const u32x4_a2 *>(row_ptr + col);
            v = u32x4{w[0], w[1], w[2], w[3]};
        } else {
            // The chunk that crosses the limit: element by element.  Combining the halves needs
            // the loaded values at once, so this waits for every load in flight; only chunks at
            // the end of K (and, for B, the last k row of a tile that crosses N) come here.
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = (col + e < limit) ? (uint32_t)row_ptr[col + e] : 0u;
            v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
    }
    return v;
}

// One operand's chunks of one slice into registers.  Chunk q = t + i*T: panel row q / CH, chunk
// q % CH.  X: the operand; d0, D: the tile's first index and the matrix extent along the
// operand's outer dimension; k0: the slice's first k.
//  * K-contiguous panel (A as given, B transposed): row = outer index, chunk along K; rows past D
//    and columns past K read as zeros.
//  * K-row panel (B as given, A transposed): row = k row, chunk along the outer dimension.  Columns
//    at or past D only feed C elements that are never stored, so a chunk that crosses D is read
//    whole (it ends at most 7 elements past the edge, inside the next k row) and chunks past D read
//    as zeros.  Only the last k row keeps the element-wise read.
template <int CH, bool KC, int T, int PER_T>
__device__ __forceinline__ void panel_masked_load(const uint16_t *X, int64_t ld, int d0, int D, int k0, int K,
                                                  u32x4 (&out)[PER_T])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int q = t + i * T;
        const int row = q / CH;
        const int c = q % CH;
        if constexpr (KC) {
            const int outer = d0 + row;
            const bool ok = outer < D;
            out[i] = masked_chunk(X + (int64_t)(ok ? outer : 0) * ld, k0 + c * 8, K, ok);
        } else {
            const int krow = k0 + row;
            const int col = d0 + c * 8;
            const bool ok = krow < K;
            const uint16_t *row_ptr = X + (int64_t)(ok ? krow : 0) * ld;
            if (ok && col < D && col + 8 > D && krow + 1 < K && ld >= 8) {
                const u32x4_a2 w = *reinterpret_cast<const u32x4_a2 *>(row_ptr + col);
                out[i] = u32x4{w[0], w[1], w[2], w[3]};
            } else {
                out[i] = masked_chunk(row_ptr, col, D, ok);
            }
        }
    }
}

template <class TL>
__device__ __forceinline__ void masked_load(const Params &p, int m0, int n0, int k0, Regs<TL> &r)
{
    panel_masked_load<TL::A_CH, TL::A_KC, TL::T, TL::A_PER_T>(p.A, p.lda, m0, p.M, k0, p.K, r.a);
    panel_masked_load<TL::B_CH, TL::B_KC, TL::T, TL::B_PER_T>(p.B, p.ldb, n0, p.N, k0, p.K, r.b);
}

// One operand's chunks of one full K slice: every chunk is one 16-byte load, with no branch, so
// the compiler can count the loads in flight and wait for exactly the slice it stores (a load
// under a data-dependent branch makes it wait for all of them).  Rows (K-contiguous panel) or
// chunks (K-row panel) past the outer edge D are clamped to the last valid row or column; their
// values only reach outputs that are never stored.  The caller guarantees that the slice's k range
// lies inside K and, for a K-row panel in a tile that crosses D, that the slice does not hold k
// row K-1 and ld >= 8, so a chunk that crosses D ends inside the next k row.
template <int CH, bool KC, int T, int PER_T>
__device__ __forceinline__ void panel_plain_load(const uint16_t *X, int64_t ld, int d0, int D, int k0,
                                                 u32x4 (&out)[PER_T])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int q = t + i * T;
        const int row = q / CH;
        const int c = q % CH;
        const uint16_t *src;
        if constexpr (KC) {
            const int outer = d0 + row < D ? d0 + row : D - 1;
            src = X + (int64_t)outer * ld + k0 + c * 8;
        } else {
            const int col = d0 + c * 8 < D ? d0 + c * 8 : D - 1;
            src = X + (int64_t)(k0 + row) * ld + col;
        }
        const u32x4_a2 w = *reinterpret_cast<const u32x4_a2 *>(src);
        out[i] = u32x4{w[0], w[1], w[2], w[3]};
    }
}

template <class TL>
__device__ __forceinline__ void plain_load(const Params &p, int m0, int n0, int k0, Regs<TL> &r)
{
    panel_plain_load<TL::A_CH, TL::A_KC, TL::T, TL::A_PER_T>(p.A, p.lda, m0, p.M, k0, r.a);
    panel_plain_load<TL::B_CH, TL::B_KC, TL::T, TL::B_PER_T>(p.B, p.ldb, n0, p.N, k0, r.b);
}

template <int ROW_BYTES, int CH, bool KC, int T, int PER_T>
__device__ __forceinline__ void panel_masked_store(LDS_AS char *panel, const u32x4 (&in)[PER_T])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
        const int q = t + i * T;
        const int row = q / CH;
        const int c = q % CH;
        *(LDS_AS u32x4 *)(panel + row * ROW_BYTES + ((c ^ panel_key<CH, KC>(row)) * 16)) = in[i];
    }
}

template <class TL>
__device__ __forceinline__ void masked_store(LDS_AS char *stage, const Regs<TL> &r)
{
    panel_masked_store<TL::A_ROW, TL::A_CH, TL::A_KC, TL::T, TL::A_PER_T>(stage, r.a);
    panel_masked_store<TL::B_ROW, TL::B_CH, TL::B_KC, TL::T, TL::B_PER_T>(stage + TL::A_BYTES, r.b);
}

// ---------------------------------------------------------------- LDS -> MFMA
// The fragment of a 32-wide block (32 rows of A or 32 columns of B) for one k16 step gives lane l
// outer index l%32 and the 8 consecutive k values 8*(l/32) .. +7 of the step.  From a K-contiguous
// panel that is one ds_read_b128; from a K-row panel, two transposing reads (k rows 8h + 0..3 and
// 8h + 4..7 of the step, h = l/32).  Fragments are kept as two 4-element halves either way.
template <class TL>
struct Frags {
    short4_t a[TL::TM][2];
    short4_t b[TL::TN][2];
};

template <class TL>
struct Reads {
    static constexpr int RA = TL::A_KC ? 1 : 2;   // LDS reads per A fragment
    static constexpr int RB = TL::B_KC ? 1 : 2;   // LDS reads per B fragment
    static constexpr int PER_STEP = TL::TM * RA + TL::TN * RB;
};

// K-contiguous panel: the whole fragment of the block whose first outer index is d.
template <int ROW_BYTES, int CH>
__device__ __forceinline__ void read_kc(const LDS_AS char *panel, int d, int s, int lane, short4_t (&f)[2])
{
    const int row = d + (lane & 31);
    const int c = 2 * s + (lane >> 5);
    const short8_t v = *(const LDS_AS short8_t *)(panel + row * ROW_BYTES + ((c ^ panel_key<CH, true>(row)) * 16));
    f[0] = __builtin_shufflevector(v, v, 0, 1, 2, 3);
    f[1] = __builtin_shufflevector(v, v, 4, 5, 6, 7);
}

// K-row panel: half r2 of that fragment.  ds_read_b64_tr_b16 works on groups of 16 lanes: group
// lane i receives, as element e, element i%4 of the 8 bytes group lane 4e + i/4 addressed; lanes
// addressing a 4 (k) x 16 (outer) block, four lanes per k row, therefore each receive one outer
// index's 4 k values.
template <int ROW_BYTES, int CH>
__device__ __forceinline__ short4_t read_kr(const LDS_AS char *panel, int d, int s, int lane, int r2)
{
    const int gi = lane & 15;         // lane within its 16-lane group
    const int q = (lane >> 4) & 1;    // which 16 outer indices of the 32-wide block
    const int n = d + 16 * q + 4 * (gi & 3);
    const int krow = 16 * s + 8 * (lane >> 5) + (gi >> 2) + 4 * r2;
    const LDS_AS char *addr =
        panel + krow * ROW_BYTES + (((n >> 3) ^ panel_key<CH, false>(krow)) * 16) + (n & 7) * 2;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS short4_t *)addr);
}

template <class TL>
__device__ __forceinline__ void read_a_part(const LDS_AS char *stage, int s, int wm, int lane, int mi, int part,
                                            Frags<TL> &f)
{
    const int d = wm * TL::WTM + mi * 32;
    if constexpr (TL::A_KC)
        read_kc<TL::A_ROW, TL::A_CH>(stage, d, s, lane, f.a[mi]);
    else
        f.a[mi][part] = read_kr<TL::A_ROW, TL::A_CH>(stage, d, s, lane, part);
}

template <class TL>
__device__ __forceinline__ void read_b_part(const LDS_AS char *stage, int s, int wn, int lane, int ni, int part,
                                            Frags<TL> &f)
{
    const int d = wn * TL::WTN + ni * 32;
    if constexpr (TL::B_KC)
        read_kc<TL::B_ROW, TL::B_CH>(stage + TL::A_BYTES, d, s, lane, f.b[ni]);
    else
        f.b[ni][part] = read_kr<TL::B_ROW, TL::B_CH>(stage + TL::A_BYTES, d, s, lane, part);
}

// Read number r of a step, in the order the MFMAs of the step consume them: B block 0, all A
// blocks, then the remaining B blocks.
template <class TL>
__device__ __forceinline__ void read_op(const LDS_AS char *stage, int s, int wm, int wn, int lane, int r, Frags<TL> &f)
{
    using R = Reads<TL>;
    if (r < R::RB) {
        read_b_part<TL>(stage, s, wn, lane, 0, r, f);
    } else if (r < R::RB + TL::TM * R::RA) {
        const int j = r - R::RB;
        read_a_part<TL>(stage, s, wm, lane, j / R::RA, j % R::RA, f);
    } else {
        const int j = r - R::RB - TL::TM * R::RA;
        read_b_part<TL>(stage, s, wn, lane, 1 + j / R::RB, j % R::RB, f);
    }
}

template <class TL>
__device__ __forceinline__ void load_frags(const LDS_AS char *stage, int s, int wm, int wn, int lane, Frags<TL> &f)
{
#pragma unroll
    for (int r = 0; r < Reads<TL>::PER_STEP; ++r) read_op<TL>(stage, s, wm, wn, lane, r, f);
}

// MFMA number i of a step: A block i % TM against B block i / TM (the order reads arrive in).  The
// B fragment is the instruction's first operand, so the accumulator holds a block of C^T.
template <class TL>
__device__ __forceinline__ void mfma_op(const Frags<TL> &f, int i, floatx16 (&acc)[TL::TM][TL::TN])
{
    const int mi = i % TL::TM, ni = i / TL::TM;
    const half8_t b = __builtin_bit_cast(half8_t, __builtin_shufflevector(f.b[ni][0], f.b[ni][1], 0, 1, 2, 3, 4, 5, 6, 7));
    const half8_t a = __builtin_bit_cast(half8_t, __builtin_shufflevector(f.a[mi][0], f.a[mi][1], 0, 1, 2, 3, 4, 5, 6, 7));
    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc[mi][ni], 0, 0, 0);
}

template <class TL>
__device__ __forceinline__ void mfma_step(const Frags<TL> &f, floatx16 (&acc)[TL::TM][TL::TN])
{
#pragma unroll
    for (int i = 0; i < TL::TM * TL::TN; ++i) mfma_op<TL>(f, i, acc);
}

// Interleave the MFMAs of one k16 step with the LDS reads that fetch the next step's fragments:
// one MFMA, then one read, while reads remain; then the remaining MFMAs.
template <class TL>
__device__ __forceinline__ void interleave_pattern()
{
    constexpr int READS = Reads<TL>::PER_STEP;   // LDS reads per step
    constexpr int MFMAS = TL::TM * TL::TN;       // MFMAs per step
    constexpr int PAIRS = READS < MFMAS ? READS : MFMAS;
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (MFMAS > PAIRS) __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - PAIRS, 0);
    if (READS > PAIRS) __builtin_amdgcn_sched_group_barrier(0x100, READS - PAIRS, 0);
}

// One K slice from one LDS stage (masked path).  Fragments are double-buffered: the reads of
// step s+1 are issued between the MFMAs of step s, so LDS latency hides behind the matrix pipe.
template <class TL>
__device__ __forceinline__ void compute_stage(const LDS_AS char *stage, int wm, int wn, int wk, int lane,
                                              floatx16 (&acc)[TL::TM][TL::TN])
{
    constexpr int NS = TL::BK / 16;
    if constexpr (TL::KS > 1) {
        // this K group's steps only: wk, wk + KS, ...
        Frags<TL> f;
#pragma unroll
        for (int j = 0; j < NS / TL::KS; ++j) {
            load_frags<TL>(stage, wk + j * TL::KS, wm, wn, lane, f);
            mfma_step<TL>(f, acc);
        }
        return;
    }
    Frags<TL> f[2];
    load_frags<TL>(stage, 0, wm, wn, lane, f[0]);
    __builtin_amdgcn_sched_barrier(0);   // step 0's reads stay ahead of the interleaved region
#pragma unroll
    for (int s = 0; s + 1 < NS; ++s) {
        load_frags<TL>(stage, s + 1, wm, wn, lane, f[(s + 1) & 1]);
        mfma_step<TL>(f[s & 1], acc);
        interleave_pattern<TL>();
        __builtin_amdgcn_sched_barrier(0);
    }
    mfma_step<TL>(f[(NS - 1) & 1], acc);
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------- main loops
// Interior tile, full K slices [0, nk): direct-to-LDS S-stage ring, one wave per SIMD.
//
// Issue is in order within a wave, so a burst of direct-to-LDS loads (which the CU's load path
// accepts only every ~16 cycles) would hold up the MFMAs queued behind it.  The loads of a slice
// are therefore slotted one at a time between MFMAs, a few per k16 step.
//
// Iteration kt: steps 0 .. NS-2 of slice kt (each step's MFMAs interleaved with the reads of the
// next step and the first half of the loads of slice kt+S-1); then the barrier; then step NS-1
// (interleaved with the reads of step 0 of slice kt+1 and the second half of those loads).
// Before the barrier every wave has its step NS-1 fragments in registers and waits until slice
// kt+1 has landed (later slices stay in flight).  After it, buffer kt%S is no longer read and
// slice kt+S-1 may refill it... which already happened: that slice goes to buffer (kt-1)%S,
// released by the barrier of iteration kt-1.  A slice has about S-2 iterations to land.
template <class TL, int NDMA, int PH>
__device__ __forceinline__ void step_interleaved(const LDS_AS char *next_stage, int s_next, int wm, int wn, int lane,
                                                 const Frags<TL> &cur, Frags<TL> &nxt,
                                                 floatx16 (&acc)[TL::TM][TL::TN], bool dma_on, const char *abase,
                                                 const char *bbase, uint32_t dma_stage, int d0, const uint32_t *off,
                                                 const uint32_t *dst)
{
    constexpr int MFMAS = TL::TM * TL::TN;
    constexpr int READS = Reads<TL>::PER_STEP;
    constexpr int GAP = NDMA > 0 ? MFMAS / NDMA : MFMAS;
    static_assert(NDMA == 0 || GAP >= 1, "more loads than MFMAs in a step");
#pragma unroll
    for (int i = 0; i < MFMAS; ++i) {
        mfma_op<TL>(cur, i, acc);
        if (i < READS) read_op<TL>(next_stage, s_next, wm, wn, lane, i, nxt);
        if (NDMA > 0 && i % GAP == PH % GAP && i / GAP < NDMA) {
            const int d = d0 + i / GAP;   // index into the slice's loads: A windows first
            if (dma_on) dma16(d < TL::A_DMA_W ? abase : bbase, off[d], dma_stage, dst[d]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = MFMAS; r < READS; ++r) read_op<TL>(next_stage, s_next, wm, wn, lane, r, nxt);
}

template <class TL, int PH>
__device__ __forceinline__ void fast_loop(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wave,
                                          int wm, int wn, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    const int rows = p.M - m0 < TL::BM ? p.M - m0 : TL::BM;   // valid rows and columns of the tile
    const int cols = p.N - n0 < TL::BN ? p.N - n0 : TL::BN;
    constexpr int NS = TL::BK / 16;
    using D = DmaPlan<TL, TL::W>;
    constexpr int COUNT = D::COUNT;
    constexpr int H1 = COUNT / 2;                 // loads issued before the barrier
    constexpr int H2 = COUNT - H1;                // loads issued after it
    constexpr int PER_EARLY = H1 / (NS - 1);      // spread over steps 0 .. NS-2
    static_assert(TL::S >= 3, "a slice needs at least one iteration to land");
    static_assert(NS >= 2 && NS % 2 == 0, "fragment double-buffer parity");
    static_assert(PER_EARLY * (NS - 1) == H1, "loads must split evenly over the early steps");
    static_assert(TL::A_DMA_W == D::A, "tile load split");
    static_assert((TL::S - 1) * COUNT <= 63, "vmcnt limit");
    if (nk <= 0) return;

    uint32_t off[COUNT], dst[COUNT];
    dma_lane_offsets<TL>(p, wave, lane, rows, cols, off, dst);
    const PanelBases<TL> pb(p, m0, n0);
    const char *abase = pb.abase;
    const char *bbase = pb.bbase;
    const int64_t a_step = pb.a_step;
    const int64_t b_step = pb.b_step;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // Prologue: slices 0 .. S-2 in flight; wait for slice 0.
#pragma unroll
    for (int sl = 0; sl + 1 < TL::S; ++sl)
        if (sl < nk)
#pragma unroll
            for (int d = 0; d < COUNT; ++d)
                dma16(d < D::A ? abase + sl * a_step : bbase + sl * b_step, off[d], lds0 + sl * TL::STAGE, dst[d]);
    if (TL::S - 1 <= nk)
        wait_vmcnt<(TL::S - 2) * COUNT>();
    else
        wait_vmcnt<0>();
    barrier();
    phase_mark(1);

    Frags<TL> f[2];
    load_frags<TL>(smem, 0, wm, wn, lane, f[0]);
    __builtin_amdgcn_sched_barrier(0);

    for (int kt = 0; kt < nk; ++kt) {
        const LDS_AS char *stage = smem + (kt % TL::S) * TL::STAGE;
        const int ds = kt + TL::S - 1;            // slice whose loads this iteration issues
#if GEMM_F16_DMA_CLAMP
        // Past the last slice the loads re-read slice nk-1 into the free buffer (never read), so
        // the loop body has no branches; they are drained before the ring is reused.
        constexpr bool dma_on = true;
        const int dsrc = ds < nk ? ds : nk - 1;
#else
        const bool dma_on = ds < nk;
        const int dsrc = ds;
#endif
        const char *da = abase + dsrc * a_step;
        const char *db = bbase + dsrc * b_step;
        const uint32_t dstage = lds0 + (uint32_t)((ds % TL::S) * TL::STAGE);
#pragma unroll
        for (int s = 0; s + 1 < NS; ++s)
            step_interleaved<TL, PER_EARLY, PH>(stage, s + 1, wm, wn, lane, f[s & 1], f[(s + 1) & 1], acc, dma_on, da, db,
                                            dstage, s * PER_EARLY, off, dst);
        wait_lgkmcnt0();
        if (kt + 1 < nk) {
            if (dma_on)
                wait_vmcnt<(TL::S - 3) * COUNT + H1>();
            else
                wait_vmcnt<0>();
        }
        barrier();
        // Last step of slice kt; its reads fetch step 0 of slice kt+1 (unused after the last
        // slice, where they read a buffer no load is writing).
        step_interleaved<TL, H2, PH>(smem + ((kt + 1) % TL::S) * TL::STAGE, 0, wm, wn, lane, f[(NS - 1) & 1], f[NS & 1],
                                 acc, dma_on, da, db, dstage, H1, off, dst);
    }
#if GEMM_F16_DMA_CLAMP
    wait_vmcnt<0>();   // the re-reads past the last slice must land before the ring is reused
#endif
}

// ---------------------------------------------------------------- paired slices
// With BK = 32 a K-contiguous panel (A as given, B transposed) has 64-byte rows, so each 1 KiB
// direct-to-LDS load of it touches 16 half-used cache lines where a load of a K-row panel's 256-
// or 512-byte rows touches 8 full ones, and the load path's cost follows the lines.  The paired
// layout (every tile but the K-split one) loads one K-contiguous operand X two slices at a time as
// 128-byte rows: three X double stages (rows x 2BK) and four stages of the other operand Y,
// 160 KiB at most.  X is A when A is K-contiguous (NN, NT), else B (TT); only one operand fits.
//
// Iteration kt computes slice kt (X: double stage (kt/2) % 3, steps 2(kt%2) and 2(kt%2)+1 of its
// four k16 steps; Y: stage kt % 4).  Before the barrier it issues half of the X loads of the pair
// starting at slice 2(kt/2) + 4, into the double stage that held slices 2(kt/2) - 2 and
// 2(kt/2) - 1 (released by the barrier of iteration 2(kt/2) - 1); after it, the Y loads of slice
// kt+3 into stage (kt-1) % 4 (released by the barrier of iteration kt-1).  Every load a slice
// needs is issued by the end of iteration kt-2, so the wait before barrier kt allows one
// iteration plus this iteration's X loads in flight, as in the single-slice ring.
template <class TL>
struct UsePaired {
    static constexpr bool value = (TL::A_KC || TL::B_KC) && TL::KS == 1 && TL::BK == 32 && TL::S == 4 &&
                                  ((TL::BM == 256 && (TL::BN == 256 || TL::BN == 128)) ||
                                   (TL::BM == TL::BN && TL::BM <= 128));
    static constexpr bool pb = !TL::A_KC;   // B is the paired operand
};

template <class TL>
struct Paired {
    static constexpr bool PB = UsePaired<TL>::pb;
    static constexpr int X_ROW2 = (PB ? TL::B_ROW : TL::A_ROW) * 2;   // bytes per row of a double stage
    static constexpr int X_CH2 = (PB ? TL::B_CH : TL::A_CH) * 2;
    static constexpr int X_STAGE2 = (PB ? TL::BN : TL::BM) * X_ROW2;  // one double stage
    static constexpr int X_REGION = 3 * X_STAGE2;
    static constexpr int Y_STAGE = PB ? TL::A_BYTES : TL::B_BYTES;
    static constexpr int LDS_BYTES = X_REGION + 4 * Y_STAGE;
    static constexpr int XW = X_STAGE2 / 1024 / TL::W;   // X windows per wave per double stage
    static constexpr int YW = Y_STAGE / 1024 / TL::W;    // Y windows per wave per slice
    static constexpr int XH = XW / 2;                    // X windows per wave per iteration
    static_assert((PB ? TL::B_KC : TL::A_KC), "the paired operand is K-contiguous");
    static_assert(XW * 1024 * TL::W == X_STAGE2 && YW * 1024 * TL::W == Y_STAGE, "windows must split evenly");
    static_assert(XH * 2 == XW, "a pair's loads split over two iterations");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// LDS the main loop's ring takes.
template <class TL, bool PAIRED = UsePaired<TL>::value>
struct RingBytes {
    static constexpr int value = TL::LDS_BYTES;
};
template <class TL>
struct RingBytes<TL, true> {
    static constexpr int value = Paired<TL>::LDS_BYTES;
};

// Read r of a step from the paired layout: X from `xp` (double stage, step sx of four), Y from
// `yp` (stage, step sy of two); same order as read_op.
template <class TL>
__device__ __forceinline__ void read_op_paired(const LDS_AS char *xp, int sx, const LDS_AS char *yp, int sy, int wm,
                                               int wn, int lane, int r, Frags<TL> &f)
{
    using R = Reads<TL>;
    using P = Paired<TL>;
    auto read_a = [&](int mi, int part) {
        const int d = wm * TL::WTM + mi * 32;
        if constexpr (!P::PB)
            read_kc<P::X_ROW2, P::X_CH2>(xp, d, sx, lane, f.a[mi]);
        else if constexpr (TL::A_KC)
            read_kc<TL::A_ROW, TL::A_CH>(yp, d, sy, lane, f.a[mi]);
        else
            f.a[mi][part] = read_kr<TL::A_ROW, TL::A_CH>(yp, d, sy, lane, part);
    };
    auto read_b = [&](int ni, int part) {
        const int d = wn * TL::WTN + ni * 32;
        if constexpr (P::PB)
            read_kc<P::X_ROW2, P::X_CH2>(xp, d, sx, lane, f.b[ni]);
        else if constexpr (TL::B_KC)
            read_kc<TL::B_ROW, TL::B_CH>(yp, d, sy, lane, f.b[ni]);
        else
            f.b[ni][part] = read_kr<TL::B_ROW, TL::B_CH>(yp, d, sy, lane, part);
    };
    if (r < R::RB) {
        read_b(0, r);
    } else if (r < R::RB + TL::TM * R::RA) {
        const int j = r - R::RB;
        read_a(j / R::RA, j % R::RA);
    } else {
        const int j = r - R::RB - TL::TM * R::RA;
        read_b(1 + j / R::RB, j % R::RB);
    }
}

// One k16 step of the paired loop: MFMAs of `cur`, the reads of the next step, and NSLOT loads.
template <class TL, int NSLOT, int PH, class Load>
__device__ __forceinline__ void step_paired(const LDS_AS char *xp, int sx, const LDS_AS char *yp, int sy, int wm,
                                            int wn, int lane, const Frags<TL> &cur, Frags<TL> &nxt,
                                            floatx16 (&acc)[TL::TM][TL::TN], Load load)
{
    constexpr int MFMAS = TL::TM * TL::TN;
    constexpr int READS = Reads<TL>::PER_STEP;
    constexpr int GAP = NSLOT > 0 ? MFMAS / NSLOT : MFMAS;
#pragma unroll
    for (int i = 0; i < MFMAS; ++i) {
        mfma_op<TL>(cur, i, acc);
        if (i < READS) read_op_paired<TL>(xp, sx, yp, sy, wm, wn, lane, i, nxt);
        if (NSLOT > 0 && i % GAP == PH % GAP && i / GAP < NSLOT) load(i / GAP);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = MFMAS; r < READS; ++r) read_op_paired<TL>(xp, sx, yp, sy, wm, wn, lane, r, nxt);
}

// Full K slices [0, nk), nk even, of an interior-path tile in the paired layout.
template <class TL, int PH>
__device__ __forceinline__ void fast_loop_paired(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wave,
                                                 int wm, int wn, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    using P = Paired<TL>;
    constexpr bool PB = P::PB;
    constexpr int COUNT = P::XH + P::YW;   // loads per wave per iteration
    static_assert(3 * P::XW + 3 * P::YW <= 63, "vmcnt limit");
    if (nk <= 0) return;
    const int rows = p.M - m0 < TL::BM ? p.M - m0 : TL::BM;
    const int cols = p.N - n0 < TL::BN ? p.N - n0 : TL::BN;
    uint32_t offx[P::XW], offy[P::YW];
#pragma unroll
    for (int j = 0; j < P::XW; ++j)
        offx[j] = panel_dma_offset<P::X_ROW2, P::X_CH2, true>(PB ? p.ldb : p.lda, wave * P::XW + j, lane,
                                                              PB ? cols : rows);
#pragma unroll
    for (int j = 0; j < P::YW; ++j)
        offy[j] = PB ? a_dma_offset<TL>(p, wave * P::YW + j, lane, rows) : b_dma_offset<TL>(p, wave * P::YW + j, lane, cols);
    const PanelBases<TL> pb(p, m0, n0);
    const char *xbase = PB ? pb.bbase : pb.abase;
    const char *ybase = PB ? pb.abase : pb.bbase;
    const int64_t x_step = PB ? pb.b_step : pb.a_step;   // bytes per slice along K
    const int64_t y_step = PB ? pb.a_step : pb.b_step;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t ldsy = lds0 + P::X_REGION;
    auto pair_src = [&](int first) { return xbase + (first + 2 <= nk ? first : nk - 2) * x_step; };
    auto y_src = [&](int sl) { return ybase + (sl < nk ? sl : nk - 1) * y_step; };

    // Prologue: X pair 0, Y slices 0..2, X pair 1; wait for X pair 0 and Y slice 0.
#pragma unroll
    for (int j = 0; j < P::XW; ++j) dma16(pair_src(0), offx[j], lds0, (uint32_t)((wave * P::XW + j) * 1024));
#pragma unroll
    for (int sl = 0; sl < 3; ++sl)
#pragma unroll
        for (int j = 0; j < P::YW; ++j)
            dma16(y_src(sl), offy[j], ldsy + sl * P::Y_STAGE, (uint32_t)((wave * P::YW + j) * 1024));
#pragma unroll
    for (int j = 0; j < P::XW; ++j)
        dma16(pair_src(2), offx[j], lds0 + P::X_STAGE2, (uint32_t)((wave * P::XW + j) * 1024));
    wait_vmcnt<2 * P::YW + P::XW>();
    barrier();
    phase_mark(1);

    Frags<TL> f[2];
#pragma unroll
    for (int r = 0; r < Reads<TL>::PER_STEP; ++r)
        read_op_paired<TL>(smem, 0, smem + P::X_REGION, 0, wm, wn, lane, r, f[0]);
    __builtin_amdgcn_sched_barrier(0);

    // One trip per pair of slices (kt, kt+1); the step within the pair is static in each half, so
    // the swizzled X read addresses are fixed and only the stage bases move.
    int dx = 0;   // double stage of this pair; the next pair is in dx+1, the X loads fill dx+2 (mod 3)
    for (int kt = 0; kt < nk; kt += 2) {
        const int dn = dx == 2 ? 0 : dx + 1;
        const int dl = dx == 0 ? 2 : dx - 1;
        const LDS_AS char *xp = smem + dx * P::X_STAGE2;
        const LDS_AS char *xpn = smem + dn * P::X_STAGE2;
        const char *xsrc = pair_src(kt + 4);
        const uint32_t xdst = lds0 + (uint32_t)(dl * P::X_STAGE2);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kt + h;
            const LDS_AS char *yp = smem + P::X_REGION + (k & 3) * P::Y_STAGE;
            step_paired<TL, P::XH, PH>(xp, 2 * h + 1, yp, 1, wm, wn, lane, f[0], f[1], acc, [&](int j) {
                dma16(xsrc, offx[h * P::XH + j], xdst, (uint32_t)((wave * P::XW + h * P::XH + j) * 1024));
            });
            wait_lgkmcnt0();
            if (h == 0 || k + 1 < nk) wait_vmcnt<COUNT + P::XH>();
            barrier();
            // Y loads of slice k+3; the reads fetch step 0 of slice k+1
            const char *ysrc = y_src(k + 3);
            const uint32_t ydst = ldsy + (uint32_t)(((k + 3) & 3) * P::Y_STAGE);
            step_paired<TL, P::YW, PH>(h == 0 ? xp : xpn, h == 0 ? 2 : 0, smem + P::X_REGION + ((k + 1) & 3) * P::Y_STAGE,
                                       0, wm, wn, lane, f[1], f[0], acc, [&](int j) {
                                           dma16(ysrc, offy[j], ydst, (uint32_t)((wave * P::YW + j) * 1024));
                                       });
        }
        dx = dn;
    }
    wait_vmcnt<0>();   // the re-reads past the last slice must land before LDS is reused
}

// ---------------------------------------------------------------- NT: both operands in pairs
// With B given transposed both operands are K-contiguous.  In the paired layout above only A fits
// three double stages; B^T would then be loaded one slice at a time, as 64-byte rows, and each of
// its 1 KiB direct-to-LDS loads would touch 16 half-used cache lines where a 128-byte-row load
// touches 8 whole ones (the load path's cost follows the lines).  Here B^T is paired too, in two
// double stages: 3 x BM + 2 x BN rows of 128 bytes (160 KiB at 256 x 256, the same as the paired
// layout).
//
// Iteration kt computes slice kt from A double stage (kt/2) % 3 and B double stage (kt/2) % 2,
// steps 2(kt%2) and 2(kt%2)+1 of each.  Before each barrier it issues half of A's loads of the pair
// starting at slice 2(kt/2)+4, into the A double stage of the pair before this one (free since the
// barrier of the previous iteration).  After the barrier of a pair's second iteration, when every
// wave has read all of this pair's B, it issues B's loads of the pair after next into this pair's
// B double stage.  A load therefore has at least two iterations to land; the wait before the
// barrier that precedes a pair's first reads (a pair's second iteration) lets only the A loads
// issued since that pair's B loads stay in flight.
template <class TL>
struct PairedNT {
    static constexpr int ROW2 = TL::BK * 2 * 2;            // a row of two slices: 128 bytes
    static constexpr int CH2 = ROW2 / 16;
    static constexpr int A_STAGE2 = TL::BM * ROW2;
    static constexpr int B_STAGE2 = TL::BN * ROW2;
    static constexpr int A_REGION = 3 * A_STAGE2;
    static constexpr int LDS_BYTES = A_REGION + 2 * B_STAGE2;
    static constexpr int AW = A_STAGE2 / 1024 / TL::W;     // A windows per wave per pair
    static constexpr int AH = AW / 2;                      // per iteration
    static constexpr int BW = B_STAGE2 / 1024 / TL::W;     // B windows per wave per pair
    static_assert(AW * 1024 * TL::W == A_STAGE2 && BW * 1024 * TL::W == B_STAGE2, "windows must split evenly");
    static_assert(AH * 2 == AW, "a pair's A loads split over two iterations");
    static_assert(LDS_BYTES == RingBytes<TL>::value, "same LDS as the paired layout");
    static_assert(AW + BW + AH <= 63, "vmcnt limit");
};

// The tiles whose steps have an MFMA per B load (every paired tile but 64 x 64) take it in NT.
// GEMM_F16_PAIR_NT=0 builds the single-slice B^T ring instead (for measurement).
#ifndef GEMM_F16_PAIR_NT
#define GEMM_F16_PAIR_NT 1
#endif
template <class TL>
struct UsePairedNT {
    static constexpr bool value = GEMM_F16_PAIR_NT && UsePaired<TL>::value && TL::A_KC && TL::B_KC &&
                                  TL::TM * TL::TN >= TL::BN * TL::BK * 4 / 1024 / TL::W;
};

// Read r of a step: A from double stage `ap` (step sa of four), B from `bp` (step sb); the order of
// read_op.
template <class TL>
__device__ __forceinline__ void read_op_paired_nt(const LDS_AS char *ap, int sa, const LDS_AS char *bp, int sb, int wm,
                                                  int wn, int lane, int r, Frags<TL> &f)
{
    using P = PairedNT<TL>;
    if (r < 1) {
        read_kc<P::ROW2, P::CH2>(bp, wn * TL::WTN, sb, lane, f.b[0]);
    } else if (r < 1 + TL::TM) {
        const int mi = r - 1;
        read_kc<P::ROW2, P::CH2>(ap, wm * TL::WTM + mi * 32, sa, lane, f.a[mi]);
    } else {
        const int ni = 1 + (r - 1 - TL::TM);
        read_kc<P::ROW2, P::CH2>(bp, wn * TL::WTN + ni * 32, sb, lane, f.b[ni]);
    }
}

// One k16 step: the MFMAs of `cur`, the reads of the next step, and NSLOT loads.
template <class TL, int NSLOT, int PH, class Load>
__device__ __forceinline__ void step_paired_nt(const LDS_AS char *ap, int sa, const LDS_AS char *bp, int sb, int wm,
                                               int wn, int lane, const Frags<TL> &cur, Frags<TL> &nxt,
                                               floatx16 (&acc)[TL::TM][TL::TN], Load load)
{
    constexpr int MFMAS = TL::TM * TL::TN;
    constexpr int READS = Reads<TL>::PER_STEP;
    constexpr int GAP = NSLOT > 0 ? MFMAS / NSLOT : MFMAS;
    static_assert(GAP >= 1, "an MFMA per load");
#pragma unroll
    for (int i = 0; i < MFMAS; ++i) {
        mfma_op<TL>(cur, i, acc);
        if (i < READS) read_op_paired_nt<TL>(ap, sa, bp, sb, wm, wn, lane, i, nxt);
        if (NSLOT > 0 && i % GAP == PH % GAP && i / GAP < NSLOT) load(i / GAP);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = MFMAS; r < READS; ++r) read_op_paired_nt<TL>(ap, sa, bp, sb, wm, wn, lane, r, nxt);
}

// Full K slices [0, nk), nk even, of an interior-path NT tile with both operands paired.
template <class TL, int PH>
__device__ __forceinline__ void fast_loop_paired_nt(const Params &p, LDS_AS char *smem, int m0, int n0, int nk,
                                                    int wave, int wm, int wn, int lane,
                                                    floatx16 (&acc)[TL::TM][TL::TN])
{
    using P = PairedNT<TL>;
    if (nk <= 0) return;
    const int rows = p.M - m0 < TL::BM ? p.M - m0 : TL::BM;
    const int cols = p.N - n0 < TL::BN ? p.N - n0 : TL::BN;
    uint32_t offa[P::AW], offb[P::BW];
#pragma unroll
    for (int j = 0; j < P::AW; ++j)
        offa[j] = panel_dma_offset<P::ROW2, P::CH2, true>(p.lda, wave * P::AW + j, lane, rows);
#pragma unroll
    for (int j = 0; j < P::BW; ++j)
        offb[j] = panel_dma_offset<P::ROW2, P::CH2, true>(p.ldb, wave * P::BW + j, lane, cols);
    const PanelBases<TL> pb(p, m0, n0);
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const uint32_t ldsb = lds0 + P::A_REGION;
    // pairs past the last one re-read it (into double stages nobody reads again)
    auto a_src = [&](int first) { return pb.abase + (first + 2 <= nk ? first : nk - 2) * pb.a_step; };
    auto b_src = [&](int first) { return pb.bbase + (first + 2 <= nk ? first : nk - 2) * pb.b_step; };
    auto load_a = [&](const char *src, int stage, int j) {
        dma16(src, offa[j], lds0 + (uint32_t)(stage * P::A_STAGE2), (uint32_t)((wave * P::AW + j) * 1024));
    };
    auto load_b = [&](const char *src, int stage, int j) {
        dma16(src, offb[j], ldsb + (uint32_t)(stage * P::B_STAGE2), (uint32_t)((wave * P::BW + j) * 1024));
    };

    // Prologue: A pair 0, B pair 0, A pair 1, B pair 1; wait for the first two.
#pragma unroll
    for (int j = 0; j < P::AW; ++j) load_a(a_src(0), 0, j);
#pragma unroll
    for (int j = 0; j < P::BW; ++j) load_b(b_src(0), 0, j);
#pragma unroll
    for (int j = 0; j < P::AW; ++j) load_a(a_src(2), 1, j);
#pragma unroll
    for (int j = 0; j < P::BW; ++j) load_b(b_src(2), 1, j);
    wait_vmcnt<P::AW + P::BW>();
    barrier();
    phase_mark(1);

    Frags<TL> f[2];
#pragma unroll
    for (int r = 0; r < Reads<TL>::PER_STEP; ++r)
        read_op_paired_nt<TL>(smem, 0, smem + P::A_REGION, 0, wm, wn, lane, r, f[0]);
    __builtin_amdgcn_sched_barrier(0);

    int da = 0;   // A double stage of this pair; the next pair is in da+1, A's loads fill da+2 (mod 3)
    int db = 0;   // B double stage of this pair; the next pair is in the other one
    for (int kt = 0; kt < nk; kt += 2) {
        const int dan = da == 2 ? 0 : da + 1;
        const int dal = da == 0 ? 2 : da - 1;
        const LDS_AS char *ap = smem + da * P::A_STAGE2;
        const LDS_AS char *apn = smem + dan * P::A_STAGE2;
        const LDS_AS char *bp = smem + P::A_REGION + db * P::B_STAGE2;
        const LDS_AS char *bpn = smem + P::A_REGION + (db ^ 1) * P::B_STAGE2;
        const char *asrc = a_src(kt + 4);
        const char *bsrc = b_src(kt + 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kt + h;
            step_paired_nt<TL, P::AH, PH>(ap, 2 * h + 1, bp, 2 * h + 1, wm, wn, lane, f[0], f[1], acc,
                                          [&](int j) { load_a(asrc, dal, h * P::AH + j); });
            wait_lgkmcnt0();
            if (h == 0)
                wait_vmcnt<P::AW + P::BW + P::AH>();   // nothing new is read before the next barrier
            else if (k + 1 < nk)
                wait_vmcnt<P::AW>();                   // the next pair has landed: only its successor's A may fly
            barrier();
            // the reads fetch step 0 of slice k+1; after the pair's second barrier, B of the pair
            // after next goes into this pair's B double stage
            if (h == 0)
                step_paired_nt<TL, 0, PH>(ap, 2, bp, 2, wm, wn, lane, f[1], f[0], acc, [&](int) {});
            else
                step_paired_nt<TL, P::BW, PH>(apn, 0, bpn, 0, wm, wn, lane, f[1], f[0], acc,
                                              [&](int j) { load_b(bsrc, db, j); });
        }
        da = dan;
        db ^= 1;
    }
    wait_vmcnt<0>();   // the re-reads past the last slice must land before LDS is reused
}

// The waves of a workgroup run the same instruction sequence nearly in lockstep.  Each wave
// therefore takes its own load slot within a gap of MFMAs (wave w: slot w % gap), so the CU's
// load path receives one wave's load at a time instead of all four at once.
template <class TL>
struct LoadSlots {
    static constexpr int NS = TL::BK / 16;
    static constexpr int H1 = DmaPlan<TL, TL::W>::COUNT / 2;
    static constexpr int GAP = TL::TM * TL::TN / (H1 / (NS - 1));
};

template <class TL, int PH = 0>
__device__ __forceinline__ void fast_loop_slotted(const Params &p, LDS_AS char *smem, int m0, int n0, int nk,
                                                  int wave, int wm, int wn, int lane,
                                                  floatx16 (&acc)[TL::TM][TL::TN])
{
#if GEMM_F16_STAGGER_LOADS
    constexpr int G = LoadSlots<TL>::GAP;
    if constexpr (PH + 1 < G) {
        if (wave % G != PH) {
            fast_loop_slotted<TL, PH + 1>(p, smem, m0, n0, nk, wave, wm, wn, lane, acc);
            return;
        }
    }
    if constexpr (UsePairedNT<TL>::value)
        fast_loop_paired_nt<TL, PH>(p, smem, m0, n0, nk, wave, wm, wn, lane, acc);
    else if constexpr (UsePaired<TL>::value)
        fast_loop_paired<TL, PH>(p, smem, m0, n0, nk, wave, wm, wn, lane, acc);
    else
        fast_loop<TL, PH>(p, smem, m0, n0, nk, wave, wm, wn, lane, acc);
#else
    fast_loop<TL, LoadSlots<TL>::GAP / 2>(p, smem, m0, n0, nk, wave, wm, wn, lane, acc);
#endif
}

// Full K slices [0, nk) of a tile whose K groups split every slice (one k16 step per group per
// slice, one wave per group).  Iteration kt: wait until slice kt+1 has landed, barrier (slice kt+1
// is visible to every wave, and every wave is done with buffer (kt-1)%S, which this iteration
// refills); then this wave's 16 MFMAs of slice kt, interleaved with the reads of its fragments of
// slice kt+1 and with its loads of slice kt+S-1.  Each slice has S-2 iterations to land.
template <class TL, int PH>
__device__ __forceinline__ void ksplit_iteration(const Params &p, LDS_AS char *smem, int nk, int kt, int wk, int lane,
                                                 const Frags<TL> &cur, Frags<TL> &nxt,
                                                 floatx16 (&acc)[TL::TM][TL::TN], const char *abase,
                                                 const char *bbase, int64_t a_step, int64_t b_step, uint32_t lds0,
                                                 const uint32_t *off, const uint32_t *dst)
{
    constexpr int COUNT = DmaPlan<TL, TL::W>::COUNT;
    if (kt + 1 < nk) wait_vmcnt<(TL::S - 3) * COUNT>();
    barrier();
    const int ds = kt + TL::S - 1;
    const int dsrc = ds < nk ? ds : nk - 1;   // past the last slice: re-read it into the free buffer
    step_interleaved<TL, COUNT, PH>(smem + ((kt + 1) % TL::S) * TL::STAGE, wk, 0, 0, lane, cur, nxt, acc, true,
                                    abase + dsrc * a_step, bbase + dsrc * b_step,
                                    lds0 + (uint32_t)((ds % TL::S) * TL::STAGE), 0, off, dst);
}

template <class TL, int PH>
__device__ __forceinline__ void fast_loop_ksplit_ph(const Params &p, LDS_AS char *smem, int m0, int n0, int nk,
                                                    int wave, int wk, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    using D = DmaPlan<TL, TL::W>;
    constexpr int COUNT = D::COUNT;
    static_assert(TL::BK / 16 == TL::KS && TL::WGM == 1 && TL::WGN == 1, "one k16 step per wave per slice");
    static_assert(TL::S >= 3, "a slice needs at least one iteration to land");
    static_assert((TL::S - 1) * COUNT <= 63, "vmcnt limit");
    if (nk <= 0) return;
    const int rows = p.M - m0 < TL::BM ? p.M - m0 : TL::BM;
    const int cols = p.N - n0 < TL::BN ? p.N - n0 : TL::BN;
    uint32_t off[COUNT], dst[COUNT];
    dma_lane_offsets<TL>(p, wave, lane, rows, cols, off, dst);
    const PanelBases<TL> pb(p, m0, n0);
    const char *abase = pb.abase;
    const char *bbase = pb.bbase;
    const int64_t a_step = pb.a_step;
    const int64_t b_step = pb.b_step;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

#pragma unroll
    for (int sl = 0; sl + 1 < TL::S; ++sl)
        if (sl < nk)
#pragma unroll
            for (int d = 0; d < COUNT; ++d)
                dma16(d < D::A ? abase + sl * a_step : bbase + sl * b_step, off[d], lds0 + sl * TL::STAGE, dst[d]);
    if (TL::S - 1 <= nk)
        wait_vmcnt<(TL::S - 2) * COUNT>();
    else
        wait_vmcnt<0>();
    barrier();
    phase_mark(1);

    Frags<TL> f[2];
    load_frags<TL>(smem, wk, 0, 0, lane, f[0]);
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < nk; kt += 2) {   // two slices per trip keep the fragment buffers static
        ksplit_iteration<TL, PH>(p, smem, nk, kt, wk, lane, f[0], f[1], acc, abase, bbase, a_step, b_step, lds0, off,
                                 dst);
        if (kt + 1 < nk)
            ksplit_iteration<TL, PH>(p, smem, nk, kt + 1, wk, lane, f[1], f[0], acc, abase, bbase, a_step, b_step,
                                     lds0, off, dst);
    }
    wait_vmcnt<0>();   // the re-reads past the last slice must land before the ring is reused
}

template <class TL>
__device__ __forceinline__ void fast_loop_ksplit(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wave,
                                                 int wk, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    // The four waves issue their loads in alternating MFMA slots (one load per two MFMAs).
    if (wave & 1)
        fast_loop_ksplit_ph<TL, 1>(p, smem, m0, n0, nk, wave, wk, lane, acc);
    else
        fast_loop_ksplit_ph<TL, 0>(p, smem, m0, n0, nk, wave, wk, lane, acc);
}

// Masked slices [kb, nk): register-staged through two LDS buffers, one barrier per slice.  Slice
// s is loaded into register set (s - kb) % D and stored to LDS one iteration before it is
// computed, so each load has D iterations to land (D register sets are in flight).
template <class TL>
struct MaskedDepth {
    static constexpr int CHUNKS = TL::A_PER_T + TL::B_PER_T;   // 16-byte chunks per thread per slice
    static constexpr int D = CHUNKS <= 4 ? 4 : 2;
};

template <class TL>
__device__ __forceinline__ void masked_loop(const Params &p, LDS_AS char *smem, int m0, int n0, int kb, int nk,
                                            int wm, int wn, int wk, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    constexpr int D = MaskedDepth<TL>::D;
    if (kb >= nk) return;
    Regs<TL> r[D];
#pragma unroll
    for (int u = 0; u < D; ++u)
        if (kb + u < nk) masked_load<TL>(p, m0, n0, (kb + u) * TL::BK, r[u]);
    masked_store<TL>(smem, r[0]);
    if (kb + D < nk) masked_load<TL>(p, m0, n0, (kb + D) * TL::BK, r[0]);
    wait_lgkmcnt0();
    barrier();
    for (int kt = kb; kt < nk; kt += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int k = kt + u;
            if (k >= nk) break;
            const int cur = (k - kb) & 1;
            compute_stage<TL>(smem + cur * TL::STAGE, wm, wn, wk, lane, acc);
            if (k + 1 < nk) {
                masked_store<TL>(smem + (cur ^ 1) * TL::STAGE, r[(u + 1) % D]);   // slice k+1
                if (k + 1 + D < nk) masked_load<TL>(p, m0, n0, (k + 1 + D) * TL::BK, r[(u + 1) % D]);
            }
            wait_lgkmcnt0();
            barrier();
        }
    }
}

// Full K slices [0, nk) through registers (operands whose rows are not 16-byte aligned, or the
// forced register path): the masked loop's schedule with branch-free loads.  Past the last slice
// the loads re-read slice nk-1 and the stores fill the idle buffer, so every step issues the same
// loads and the wait before a store covers exactly the D-1 slices loaded after it.
template <class TL>
__device__ __forceinline__ void reg_loop(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wm, int wn,
                                         int wk, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    constexpr int D = MaskedDepth<TL>::D;
    if (nk <= 0) return;
    Regs<TL> r[D];
#pragma unroll
    for (int u = 0; u < D; ++u) plain_load<TL>(p, m0, n0, (u < nk ? u : nk - 1) * TL::BK, r[u]);
    masked_store<TL>(smem, r[0]);
    plain_load<TL>(p, m0, n0, (D < nk ? D : nk - 1) * TL::BK, r[0]);
    wait_lgkmcnt0();
    barrier();
    for (int kt = 0; kt < nk; kt += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int k = kt + u;
            if (k >= nk) break;
            const int cur = k & 1;
            compute_stage<TL>(smem + cur * TL::STAGE, wm, wn, wk, lane, acc);
            masked_store<TL>(smem + (cur ^ 1) * TL::STAGE, r[(u + 1) % D]);   // slice k+1
            const int nx = k + 1 + D;
            plain_load<TL>(p, m0, n0, (nx < nk ? nx : nk - 1) * TL::BK, r[(u + 1) % D]);
            wait_lgkmcnt0();
            barrier();
        }
    }
}

// Register-staged S-stage ring for tiles whose waves do not split K (full K slices only) and that
// have no paired layout (both operands K-row: A transposed, B as given).
//
// The direct-to-LDS loop's schedule with each load slot doing two things for one 16-byte chunk
// of this thread: store the chunk of slice kt+S-1 from registers into its ring buffer, then load
// the same chunk of slice kt+S-1+NSET into the registers just freed.  With two register sets
// (iterations unrolled in pairs) a chunk has two iterations to arrive before its store; a tile
// whose accumulators leave room for only one set gives it one.
// Every load is one branch-free 16-byte load (panel_plain_load's clamping), so the compiler waits
// for exactly the chunk a store needs.  Past the last slice the loads re-read slice nk-1 and the
// stores fill buffers that are never read.
template <class TL>
struct RegRing {
    static constexpr int CH = TL::A_PER_T + TL::B_PER_T;   // chunks per thread per slice
    static constexpr int NS = TL::BK / 16;
    static constexpr int H1 = CH / 2;                       // slots before the barrier
    static constexpr int H2 = CH - H1;                      // slots after it
    static constexpr int PER_EARLY = H1 / (NS - 1);
    static constexpr int GAP = TL::TM * TL::TN / (PER_EARLY > 0 ? PER_EARLY : 1);
    static_assert(NS >= 2 && NS % 2 == 0 && PER_EARLY * (NS - 1) == H1, "slots must split evenly");
    static_assert(PER_EARLY >= 1 && GAP >= 1 && H2 * GAP <= TL::TM * TL::TN, "slots must fit the MFMAs");

    const char *src[CH];   // chunk address in slice 0
    uint32_t lds[CH];      // byte offset of the chunk in a stage
    int64_t a_step, b_step;

    __device__ __forceinline__ RegRing(const Params &p, int m0, int n0)
    {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < TL::A_PER_T; ++i) {
            const int q = t + i * TL::T, row = q / TL::A_CH, c = q % TL::A_CH;
            int64_t e;
            if constexpr (TL::A_KC)
                e = (int64_t)(m0 + row < p.M ? m0 + row : p.M - 1) * p.lda + c * 8;
            else
                e = (int64_t)row * p.lda + (m0 + c * 8 < p.M ? m0 + c * 8 : p.M - 1);
            src[i] = reinterpret_cast<const char *>(p.A + e);
            lds[i] = (uint32_t)(row * TL::A_ROW + ((c ^ panel_key<TL::A_CH, TL::A_KC>(row)) * 16));
        }
#pragma unroll
        for (int i = 0; i < TL::B_PER_T; ++i) {
            const int q = t + i * TL::T, row = q / TL::B_CH, c = q % TL::B_CH;
            int64_t e;
            if constexpr (TL::B_KC)
                e = (int64_t)(n0 + row < p.N ? n0 + row : p.N - 1) * p.ldb + c * 8;
            else
                e = (int64_t)row * p.ldb + (n0 + c * 8 < p.N ? n0 + c * 8 : p.N - 1);
            src[TL::A_PER_T + i] = reinterpret_cast<const char *>(p.B + e);
            lds[TL::A_PER_T + i] =
                (uint32_t)(TL::A_BYTES + row * TL::B_ROW + ((c ^ panel_key<TL::B_CH, TL::B_KC>(row)) * 16));
        }
        a_step = TL::A_KC ? (int64_t)TL::BK * 2 : (int64_t)TL::BK * p.lda * 2;
        b_step = TL::B_KC ? (int64_t)TL::BK * 2 : (int64_t)TL::BK * p.ldb * 2;
    }

    __device__ __forceinline__ u32x4 load(int d, int slice) const
    {
        const u32x4_a2 w =
            *reinterpret_cast<const u32x4_a2 *>(src[d] + (int64_t)slice * (d < TL::A_PER_T ? a_step : b_step));
        return u32x4{w[0], w[1], w[2], w[3]};
    }
};

// One k16 step: MFMAs of `cur`, reads of step s_next into `nxt`, and NSLOT store/load slots
// (chunks d0 ..) spread over the MFMAs at phase PH.
template <class TL, int NSLOT, int PH>
__device__ __forceinline__ void step_reg(const LDS_AS char *next_stage, int s_next, int wm, int wn, int lane,
                                         const Frags<TL> &cur, Frags<TL> &nxt, floatx16 (&acc)[TL::TM][TL::TN],
                                         const RegRing<TL> &rr, u32x4 (&R)[RegRing<TL>::CH], LDS_AS char *dst_stage,
                                         int load_slice, int d0)
{
    constexpr int MFMAS = TL::TM * TL::TN;
    constexpr int READS = Reads<TL>::PER_STEP;
    constexpr int GAP = NSLOT > 0 ? MFMAS / NSLOT : MFMAS;
    static_assert(NSLOT == 0 || GAP >= 1, "more slots than MFMAs in a step");
#pragma unroll
    for (int i = 0; i < MFMAS; ++i) {
        mfma_op<TL>(cur, i, acc);
        if (i < READS) read_op<TL>(next_stage, s_next, wm, wn, lane, i, nxt);
        if (NSLOT > 0 && i % GAP == PH % GAP && i / GAP < NSLOT) {
            const int d = d0 + i / GAP;
            *(LDS_AS u32x4 *)(dst_stage + rr.lds[d]) = R[d];
            R[d] = rr.load(d, load_slice);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = MFMAS; r < READS; ++r) read_op<TL>(next_stage, s_next, wm, wn, lane, r, nxt);
}

// Iteration kt of the register ring with register set R (holding slice kt+S-1).
template <class TL, int PH, int NSET>
__device__ __forceinline__ void reg_ring_iteration(LDS_AS char *smem, int nk, int kt, int wm, int wn, int lane,
                                                   Frags<TL> (&f)[2], floatx16 (&acc)[TL::TM][TL::TN],
                                                   const RegRing<TL> &rr, u32x4 (&R)[RegRing<TL>::CH])
{
    using G = RegRing<TL>;
    constexpr int NS = G::NS;
    const LDS_AS char *stage = smem + (kt % TL::S) * TL::STAGE;
    LDS_AS char *dst = smem + ((kt + TL::S - 1) % TL::S) * TL::STAGE;   // slice kt+S-1, buffer (kt-1)%S
    const int ls = kt + TL::S - 1 + NSET < nk ? kt + TL::S - 1 + NSET : nk - 1;   // slice this set loads next
#pragma unroll
    for (int s = 0; s + 1 < NS; ++s)
        step_reg<TL, G::PER_EARLY, PH>(stage, s + 1, wm, wn, lane, f[s & 1], f[(s + 1) & 1], acc, rr, R, dst, ls,
                                       s * G::PER_EARLY);
    wait_lgkmcnt0();   // this slice's fragment reads and this wave's stores so far are complete
    barrier();         // slice kt+1 is in LDS for every wave; buffer kt%S is no longer read
    step_reg<TL, G::H2, PH>(smem + ((kt + 1) % TL::S) * TL::STAGE, 0, wm, wn, lane, f[(NS - 1) & 1], f[NS & 1], acc,
                            rr, R, dst, ls, G::H1);
}

template <class TL, int PH, int NSET>
__device__ __forceinline__ void reg_ring_loop(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wm,
                                              int wn, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    using G = RegRing<TL>;
    static_assert(TL::KS == 1, "waves must not split K");
    static_assert(TL::S >= 3, "a slice needs at least one iteration in flight");
    static_assert(NSET == 1 || NSET == 2, "one or two register sets");
    if (nk <= 0) return;
    const G rr(p, m0, n0);
    u32x4 R[NSET][G::CH];
    // Prologue: slices 0 .. S-2 stored; slices S-1 .. S-2+NSET in the register sets (slice j in
    // set j % NSET).
#pragma unroll
    for (int u = 0; u < NSET; ++u)
#pragma unroll
        for (int d = 0; d < G::CH; ++d) R[u][d] = rr.load(d, u < nk ? u : nk - 1);
#pragma unroll
    for (int j = 0; j + 1 < TL::S; ++j) {
        const int nx = j + NSET < nk ? j + NSET : nk - 1;
#pragma unroll
        for (int d = 0; d < G::CH; ++d) {
            *(LDS_AS u32x4 *)(smem + j * TL::STAGE + rr.lds[d]) = R[j % NSET][d];
            R[j % NSET][d] = rr.load(d, nx);
        }
    }
    wait_lgkmcnt0();
    barrier();
    phase_mark(1);

    Frags<TL> f[2];
    load_frags<TL>(smem, 0, wm, wn, lane, f[0]);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int X = (TL::S - 1) % NSET;   // register set of slice kt+S-1 for even kt
    for (int kt = 0; kt < nk; kt += NSET) {
        reg_ring_iteration<TL, PH, NSET>(smem, nk, kt, wm, wn, lane, f, acc, rr, R[X]);
        if constexpr (NSET == 2) {
            if (kt + 1 >= nk) break;
            reg_ring_iteration<TL, PH, NSET>(smem, nk, kt + 1, wm, wn, lane, f, acc, rr, R[X ^ 1]);
        }
    }
    // The last iteration's stores (into buffers nothing reads) must be done before whatever
    // reuses this LDS (the masked K tail, the epilogue) passes its barrier.
    wait_lgkmcnt0();
}

// Register-staged ring in the paired layout, for the tiles that take the paired layout on the
// direct-to-LDS path: the K-contiguous operand X travels in 128-byte rows (two slices per row), so
// its loads touch whole cache lines, as there.
//
// Iteration kt stores, before its barrier, half of this thread's chunks of X pair kt/2 + 2 into the
// double stage that the barrier of iteration 2(kt/2) - 1 freed, and after its barrier this thread's
// chunks of Y slice kt+3 into the stage that the barrier of iteration kt-1 freed.  Each slot then
// reloads the register it just stored with the chunk NSET iterations further along the same
// stream (X: the pairs' chunks in order; Y: the slices' chunks in order), so a load has NSET
// iterations to arrive.  The loads clamp rows and columns as RegRing's do; past the last pair or
// slice they re-read the last one and the stores fill buffers that are never read.
template <class TL>
struct RegPaired {
    using P = Paired<TL>;
    static constexpr bool PB = P::PB;
    static constexpr int XC = P::X_STAGE2 / 16 / TL::T;   // X chunks per thread per pair
    static constexpr int XH = XC / 2;                      // X chunks per thread per iteration
    static constexpr int YC = P::Y_STAGE / 16 / TL::T;    // Y chunks per thread per slice
    static constexpr int Y_ROW = PB ? TL::A_ROW : TL::B_ROW;
    static constexpr int Y_CH = PB ? TL::A_CH : TL::B_CH;
    static constexpr bool Y_KC = PB ? TL::A_KC : TL::B_KC;
    static constexpr int MFMAS = TL::TM * TL::TN;
    static constexpr int GAP = MFMAS / (XH > YC ? XH : YC);
    static_assert(XC * 16 * TL::T == P::X_STAGE2 && XH * 2 == XC, "X chunks must split evenly over two iterations");
    static_assert(YC * 16 * TL::T == P::Y_STAGE, "Y chunks must split evenly");
    static_assert(TL::BK / 16 == 2 && TL::S == 4, "one step on each side of the barrier, four Y stages");
    static_assert(GAP >= 1, "slots must fit the MFMAs");

    const char *xsrc[XC];   // chunk address in pair 0
    uint32_t xlds[XC];      // byte offset in a double stage
    const char *ysrc[YC];   // chunk address in slice 0
    uint32_t ylds[YC];      // byte offset in a Y stage
    int64_t x_step, y_step; // bytes per slice along K

    __device__ __forceinline__ RegPaired(const Params &p, int m0, int n0)
    {
        const int t = threadIdx.x;
        const char *xb = reinterpret_cast<const char *>(PB ? p.B : p.A);
        const int64_t xld = PB ? p.ldb : p.lda;
        const int xo = PB ? n0 : m0, xn = PB ? p.N : p.M;
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int q = t + i * TL::T, row = q / P::X_CH2, c = q % P::X_CH2;
            xsrc[i] = xb + ((int64_t)(xo + row < xn ? xo + row : xn - 1) * xld + c * 8) * 2;
            xlds[i] = (uint32_t)(row * P::X_ROW2 + ((c ^ panel_key<P::X_CH2, true>(row)) * 16));
        }
        const char *yb = reinterpret_cast<const char *>(PB ? p.A : p.B);
        const int64_t yld = PB ? p.lda : p.ldb;
        const int yo = PB ? m0 : n0, yn = PB ? p.M : p.N;
#pragma unroll
        for (int i = 0; i < YC; ++i) {
            const int q = t + i * TL::T, row = q / Y_CH, c = q % Y_CH;
            int64_t e;
            if constexpr (Y_KC)
                e = (int64_t)(yo + row < yn ? yo + row : yn - 1) * yld + c * 8;
            else
                e = (int64_t)row * yld + (yo + c * 8 < yn ? yo + c * 8 : yn - 1);
            ysrc[i] = yb + e * 2;
            ylds[i] = (uint32_t)(row * Y_ROW + ((c ^ panel_key<Y_CH, Y_KC>(row)) * 16));
        }
        x_step = (int64_t)TL::BK * 2;
        y_step = Y_KC ? (int64_t)TL::BK * 2 : (int64_t)TL::BK * yld * 2;
    }

    __device__ __forceinline__ u32x4 load_x(int i, int first) const
    {
        const u32x4_a2 w = *reinterpret_cast<const u32x4_a2 *>(xsrc[i] + (int64_t)first * x_step);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
    __device__ __forceinline__ u32x4 load_y(int i, int slice) const
    {
        const u32x4_a2 w = *reinterpret_cast<const u32x4_a2 *>(ysrc[i] + (int64_t)slice * y_step);
        return u32x4{w[0], w[1], w[2], w[3]};
    }
};

// Full K slices [0, nk), nk even, through RegPaired's ring.
template <class TL, int PH, int NSET>
__device__ __forceinline__ void reg_ring_paired(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wm,
                                                int wn, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    using G = RegPaired<TL>;
    using P = Paired<TL>;
    constexpr int XC = G::XC, XH = G::XH, YC = G::YC;
    constexpr int XR = XH * NSET;   // X registers (chunks): stream chunk j lives in register j % XR
    static_assert(NSET == 1 || NSET == 2, "one or two register sets");
    if (nk <= 0) return;
    const G rr(p, m0, n0);
    auto pair_first = [&](int first) { return first + 2 <= nk ? first : nk - 2; };
    auto y_slice = [&](int sl) { return sl < nk ? sl : nk - 1; };
    LDS_AS char *ybase = smem + P::X_REGION;

    // Prologue: X pairs 0 and 1 and Y slices 0 .. 2 stored, all loads in flight at once; then the
    // registers take X pair 2 (stream chunks 2*XC .. 2*XC + XR - 1) and Y slices 3 .. 2 + NSET.
    {
        u32x4 tx[2][XC], ty[3][YC];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < XC; ++i) tx[u][i] = rr.load_x(i, pair_first(2 * u));
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int i = 0; i < YC; ++i) ty[u][i] = rr.load_y(i, y_slice(u));
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < XC; ++i) *(LDS_AS u32x4 *)(smem + u * P::X_STAGE2 + rr.xlds[i]) = tx[u][i];
#pragma unroll
        for (int u = 0; u < 3; ++u)
#pragma unroll
            for (int i = 0; i < YC; ++i) *(LDS_AS u32x4 *)(ybase + u * P::Y_STAGE + rr.ylds[i]) = ty[u][i];
    }
    u32x4 RX[XR], RY[NSET][YC];
#pragma unroll
    for (int r = 0; r < XR; ++r) RX[r] = rr.load_x(r, pair_first(4));
#pragma unroll
    for (int s = 3; s < 3 + NSET; ++s)
#pragma unroll
        for (int i = 0; i < YC; ++i) RY[s % NSET][i] = rr.load_y(i, y_slice(s));
    wait_lgkmcnt0();
    barrier();
    phase_mark(1);

    Frags<TL> f[2];
#pragma unroll
    for (int r = 0; r < Reads<TL>::PER_STEP; ++r) read_op_paired<TL>(smem, 0, ybase, 0, wm, wn, lane, r, f[0]);
    __builtin_amdgcn_sched_barrier(0);

    int dx = 0;   // double stage of this pair; the next pair is in dx+1, the X stores fill dx+2 (mod 3)
    for (int kt = 0; kt < nk; kt += 2) {
        const int dn = dx == 2 ? 0 : dx + 1;
        const int dl = dx == 0 ? 2 : dx - 1;
        const LDS_AS char *xp = smem + dx * P::X_STAGE2;
        const LDS_AS char *xpn = smem + dn * P::X_STAGE2;
        LDS_AS char *xdst = smem + dl * P::X_STAGE2;
        const int pj = kt / 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int k = kt + h;
            step_paired<TL, XH, PH>(xp, 2 * h + 1, ybase + (k & 3) * P::Y_STAGE, 1, wm, wn, lane, f[0], f[1], acc,
                                    [&](int j) {
                                        const int ci = h * XH + j;   // chunk of pair pj+2 stored here
                                        const int cn = ci + XR;      // stream chunk the register takes next
                                        *(LDS_AS u32x4 *)(xdst + rr.xlds[ci]) = RX[ci % XR];
                                        RX[ci % XR] = rr.load_x(cn % XC, pair_first(2 * (pj + 2 + cn / XC)));
                                    });
            wait_lgkmcnt0();
            barrier();
            // Y slice k+3 from set (k+3) % NSET; the reads fetch step 0 of slice k+1.
            LDS_AS char *ydst = ybase + ((k + 3) & 3) * P::Y_STAGE;
            const int yl = y_slice(k + 3 + NSET);
            step_paired<TL, YC, PH>(h == 0 ? xp : xpn, h == 0 ? 2 : 0, ybase + ((k + 1) & 3) * P::Y_STAGE, 0, wm, wn,
                                    lane, f[1], f[0], acc, [&](int j) {
                                        u32x4(&ry)[YC] = RY[(h + 3) % NSET];
                                        *(LDS_AS u32x4 *)(ydst + rr.ylds[j]) = ry[j];
                                        ry[j] = rr.load_y(j, yl);
                                    });
        }
        dx = dn;
    }
    // The last stores (into buffers nothing reads) must be done before whatever reuses this LDS
    // (the masked K tail, the epilogue) passes its barrier.
    wait_lgkmcnt0();
}

// Slot phases of the register-staged ring, per layout.
template <class TL, bool PAIRED = UsePaired<TL>::value>
struct RegGap {
    static constexpr int value = RegRing<TL>::GAP;
};
template <class TL>
struct RegGap<TL, true> {
    static constexpr int value = RegPaired<TL>::GAP;
};

// Each wave takes its own store/load slot phase, as in the direct-to-LDS loop.  Tiles with the
// paired layout take the paired ring (nk even), the others the single-slice ring.
template <class TL, int PH = 0>
__device__ __forceinline__ void reg_ring_slotted(const Params &p, LDS_AS char *smem, int m0, int n0, int nk, int wave,
                                                 int wm, int wn, int lane, floatx16 (&acc)[TL::TM][TL::TN])
{
    constexpr int G = RegGap<TL>::value;
    if constexpr (PH + 1 < G) {
        if (wave % G != PH) {
            reg_ring_slotted<TL, PH + 1>(p, smem, m0, n0, nk, wave, wm, wn, lane, acc);
            return;
        }
    }
    constexpr int NSET = TL::WTM * TL::WTN >= 128 * 128 ? 1 : 2;
#if GEMM_F16_REG_PAIRED
    if constexpr (UsePaired<TL>::value)
        reg_ring_paired<TL, PH, NSET>(p, smem, m0, n0, nk, wm, wn, lane, acc);
    else
#endif
        reg_ring_loop<TL, PH, NSET>(p, smem, m0, n0, nk, wm, wn, lane, acc);
}

// ---------------------------------------------------------------- epilogue
// C <- acc + beta*C through LDS.  In the accumulators, lane l holds row l%32 of each 32x32 block
// and, for each group g of four registers, columns 8g + 4*(l/32) .. +3.  The tile is written to
// LDS in 32-row bands (the K ring is idle by then), then every thread reads the band back
// row-major, 16 bytes at a time, so each wave reads C (when beta != 0) and writes C in whole 1 KiB
// row segments.  The accumulators only ever feed memory instructions, never ALU operations.
// Band rows are padded by 16 bytes so the 32 rows one accumulator write touches spread over the
// banks.
template <class TL>
struct Epi {
    static constexpr int ROWS = 32;                          // one band = one mi block row of each wave
    static constexpr int ROW_BYTES = TL::BN * 4 + 16;
    static constexpr int REGION = ROWS * TL::WGM * ROW_BYTES; // one band of every wave row
    static constexpr int BYTES = REGION * TL::KS;            // one region per K group
    static constexpr int CHUNKS = ROWS * TL::WGM * TL::BN / 4;  // 16-byte pieces per band pass
    static constexpr int PER_T = CHUNKS / TL::T;
    static_assert(PER_T * TL::T == CHUNKS, "band must split evenly over the threads");
};

// Band mi of the accumulators into LDS: rows wm*WTM + mi*32 + 0..31 of every wave row wm, stacked
// as band rows wm*32 + r; K group wk writes its partial sums into region wk.
template <class TL>
__device__ __forceinline__ void band_to_lds(LDS_AS char *smem, int mi, int wm, int wn, int wk, int lane,
                                            const floatx16 (&acc)[TL::TM][TL::TN])
{
    using E = Epi<TL>;
    barrier();   // the previous band (or the K ring) is no longer read
    LDS_AS char *wrow = smem + wk * E::REGION + (wm * E::ROWS + (lane & 31)) * E::ROW_BYTES +
                        (wn * TL::WTN + 4 * (lane >> 5)) * 4;
#pragma unroll
    for (int ni = 0; ni < TL::TN; ++ni)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(LDS_AS float4_t *)(wrow + (ni * 32 + 8 * g) * 4) =
                float4_t{acc[mi][ni][4 * g + 0], acc[mi][ni][4 * g + 1], acc[mi][ni][4 * g + 2], acc[mi][ni][4 * g + 3]};
    wait_lgkmcnt0();
    barrier();
}

// 16 bytes of band row br, column piece c4: the sum of the K groups' partial sums, in group order.
template <class TL>
__device__ __forceinline__ float4_t band_piece(const LDS_AS char *smem, int br, int c4)
{
    using E = Epi<TL>;
    float4_t v = *(const LDS_AS float4_t *)(smem + br * E::ROW_BYTES + c4 * 16);
#pragma unroll
    for (int g = 1; g < TL::KS; ++g) {
        const float4_t w = *(const LDS_AS float4_t *)(smem + g * E::REGION + br * E::ROW_BYTES + c4 * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += w[e];
    }
    return v;
}

// C is read and written once per call.  When later rounds of tiles still stream A and B through
// the caches (NT), C's accesses are non-temporal so they do not evict those lines; with a single
// round they are ordinary (measured faster there).
template <bool NT>
__device__ __forceinline__ float4_t c_load(const float *src)
{
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const float4_t *>(src));
    else
        return *reinterpret_cast<const float4_t *>(src);
}

template <bool NT>
__device__ __forceinline__ void c_store(float *dst, float4_t v)
{
    if constexpr (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<float4_t *>(dst));
    else
        *reinterpret_cast<float4_t *>(dst) = v;
}

// Global row of band piece q (q = thread + i*T) of band mi, and its first column.
template <class TL>
__device__ __forceinline__ int band_row(int m0, int mi, int q)
{
    using E = Epi<TL>;
    const int br = q / (TL::BN / 4);
    return m0 + (br / E::ROWS) * TL::WTM + mi * 32 + (br % E::ROWS);
}

// Full tile, 16-byte aligned C, beta != 0: C of band mi+1 is loaded while band mi is combined and
// stored, so the reads of C keep the memory pipe busy instead of each band waiting its own latency.
template <class TL, bool NT>
__device__ __forceinline__ void epilogue_accum_vec(const Params &p, LDS_AS char *smem, int m0, int n0, int wm, int wn,
                                                   int wk, int lane, const floatx16 (&acc)[TL::TM][TL::TN])
{
    using E = Epi<TL>;
    constexpr int COLS4 = TL::BN / 4;
    const float beta = p.beta;
    float4_t old[2][E::PER_T];
    auto load_band = [&](int mi, float4_t(&dst)[E::PER_T]) {
#pragma unroll
        for (int i = 0; i < E::PER_T; ++i) {
            const int q = threadIdx.x + i * TL::T;
            const float *src = p.C + (int64_t)band_row<TL>(m0, mi, q) * p.ldc + n0 + (q % COLS4) * 4;
            dst[i] = c_load<NT>(src);
        }
    };
    load_band(0, old[0]);
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) {
        band_to_lds<TL>(smem, mi, wm, wn, wk, lane, acc);
        if (mi + 1 < TL::TM) load_band(mi + 1, old[(mi + 1) & 1]);
#pragma unroll
        for (int i = 0; i < E::PER_T; ++i) {
            const int q = threadIdx.x + i * TL::T;
            const int br = q / COLS4;
            const int c4 = q % COLS4;
            float4_t v = band_piece<TL>(smem, br, c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(beta, old[mi & 1][i][e], v[e]);
            c_store<NT>(p.C + (int64_t)band_row<TL>(m0, mi, q) * p.ldc + n0 + c4 * 4, v);
        }
    }
}

template <class TL, bool NT>
__device__ __forceinline__ void epilogue(const Params &p, LDS_AS char *smem, int m0, int n0, int wm, int wn, int wk,
                                         int lane, const floatx16 (&acc)[TL::TM][TL::TN])
{
    using E = Epi<TL>;
    const float beta = p.beta;
    const bool full = (m0 + TL::BM <= p.M) && (n0 + TL::BN <= p.N);
    const bool vec = full && p.c_vec;
    constexpr int COLS4 = TL::BN / 4;   // 16-byte pieces per C row of the tile
#if GEMM_F16_C_PREFETCH
    if (vec && beta != 0.0f) {
        epilogue_accum_vec<TL, NT>(p, smem, m0, n0, wm, wn, wk, lane, acc);
        return;
    }
#endif
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi) {
        band_to_lds<TL>(smem, mi, wm, wn, wk, lane, acc);
#pragma unroll
        for (int i = 0; i < E::PER_T; ++i) {
            const int q = threadIdx.x + i * TL::T;
            const int br = q / COLS4;                 // band row: wave row br / 32, row br % 32
            const int c4 = q % COLS4;
            const int row = m0 + (br / E::ROWS) * TL::WTM + mi * 32 + (br % E::ROWS);
            const int col = n0 + c4 * 4;
            float4_t v = band_piece<TL>(smem, br, c4);
            float *dst = p.C + (int64_t)row * p.ldc + col;
            if (vec) {
                if (beta != 0.0f) {
                    const float4_t old = c_load<NT>(dst);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(beta, old[e], v[e]);
                }
                c_store<NT>(dst, v);
            } else if (row < p.M && col + 4 <= p.N) {
                // whole chunk in range, C rows only 4-byte aligned: one unaligned 16-byte access
                if (beta != 0.0f) {
                    const float4_a4 old = *reinterpret_cast<const float4_a4 *>(dst);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(beta, old[e], v[e]);
                }
                *reinterpret_cast<float4_a4 *>(dst) = float4_a4{v[0], v[1], v[2], v[3]};
            } else if (row < p.M) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (col + e < p.N) {
                        float x = v[e];
                        if (beta != 0.0f) x = __builtin_fmaf(beta, dst[e], x);
                        dst[e] = x;
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- the kernel
template <class TL>
__global__ void __launch_bounds__(TL::T) __attribute__((amdgpu_waves_per_eu(TL::WPE, TL::WPE)))
gemm_f16_f32_kernel(Params p)
{
    constexpr int LDS_RING = RingBytes<TL>::value;
    constexpr int LDS_USE = LDS_RING > Epi<TL>::BYTES ? LDS_RING : Epi<TL>::BYTES;
    __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_USE];
    LDS_AS char *smem = (LDS_AS char *)smem_raw;

    if (p.split_k > 0) {
        // split-K: this workgroup's K range and output slice (the slices are summed afterwards)
        const int k0 = (int)blockIdx.y * p.split_k;
        const int kl = p.K - k0 < p.split_k ? p.K - k0 : p.split_k;
        p.K = kl > 0 ? kl : 0;
        p.A += TL::A_KC ? (int64_t)k0 : (int64_t)k0 * p.lda;
        p.B += TL::B_KC ? (int64_t)k0 : (int64_t)k0 * p.ldb;
        p.C += (int64_t)blockIdx.y * p.c_split;
    }
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wk = wave / (TL::WGM * TL::WGN);              // K group (0 unless the tile splits K)
    const int wm = (wave % (TL::WGM * TL::WGN)) / TL::WGN;
    const int wn = wave % TL::WGN;
    const int lane = threadIdx.x & 63;

    int64_t pm64, pn64;
    gemm_f16::tile_of_workgroup(blockIdx.x, p.tiles_m, p.tiles_n, p.group_m, p.xcd_remap, &pm64, &pn64);
    const int m0 = (int)pm64 * TL::BM;
    const int n0 = (int)pn64 * TL::BN;
    phase_mark(0);

    floatx16 acc[TL::TM][TL::TN];
#pragma unroll
    for (int mi = 0; mi < TL::TM; ++mi)
#pragma unroll
        for (int ni = 0; ni < TL::TN; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.0f;

    const int nk = (p.K + TL::BK - 1) / TL::BK;
    if (p.a_dma && p.b_dma) {
        // Full K slices through the direct-to-LDS ring, the K tail through the masked path.  In a
        // tile that crosses the outer edge of a K-row panel (N for B as given, M for A
        // transposed) the slice holding k row K-1 goes to the masked path too: its last chunk may
        // extend past the end of the matrix.
        int nkf = p.K / TL::BK;
        const bool kr_edge = (!TL::B_KC && n0 + TL::BN > p.N) || (!TL::A_KC && m0 + TL::BM > p.M);
        if (kr_edge && nkf > 0 && nkf * TL::BK == p.K) --nkf;
        if constexpr (UsePaired<TL>::value) nkf &= ~1;   // A is loaded in pairs of slices
        if constexpr (TL::KS > 1)
            fast_loop_ksplit<TL>(p, smem, m0, n0, nkf, wave, wk, lane, acc);
        else
            fast_loop_slotted<TL>(p, smem, m0, n0, nkf, wave, wm, wn, lane, acc);
        phase_mark(2);
        if (nkf < nk) {
            barrier();   // every wave is done with the ring before the masked path reuses buffers 0/1
            masked_loop<TL>(p, smem, m0, n0, nkf, nk, wm, wn, wk, lane, acc);
        }
    } else {
        // Full K slices through branch-free register loads, the K tail element-wise.  A K-row
        // panel in a tile that crosses its outer edge reads whole chunks across that edge into the
        // next k row: the slice holding k row K-1 stays on the masked path, and so does every
        // slice when rows are shorter than a chunk.
        const bool a_cross = !TL::A_KC && m0 + TL::BM > p.M;
        const bool b_cross = !TL::B_KC && n0 + TL::BN > p.N;
        int nkr = p.K / TL::BK;
        if ((a_cross && p.lda < 8) || (b_cross && p.ldb < 8))
            nkr = 0;
        else if ((a_cross || b_cross) && nkr > 0 && nkr * TL::BK == p.K)
            --nkr;
        // A 32x32 wave tile has too few MFMAs per step to cover the ring's slots (measured slower).
        if constexpr (TL::KS > 1 || TL::WTM * TL::WTN < 64 * 64) {
            reg_loop<TL>(p, smem, m0, n0, nkr, wm, wn, wk, lane, acc);
        } else {
#if GEMM_F16_REG_PAIRED
            if constexpr (UsePaired<TL>::value) nkr &= ~1;   // X is loaded in pairs of slices
#endif
            reg_ring_slotted<TL>(p, smem, m0, n0, nkr, wave, wm, wn, lane, acc);
        }
        phase_mark(2);
        if (nkr < nk) {
            barrier();
            masked_loop<TL>(p, smem, m0, n0, nkr, nk, wm, wn, wk, lane, acc);
        }
    }
    phase_mark(3);

    if (p.c_nt)
        epilogue<TL, true>(p, smem, m0, n0, wm, wn, wk, lane, acc);
    else
        epilogue<TL, false>(p, smem, m0, n0, wm, wn, wk, lane, acc);
    phase_mark(4);
}

// ---------------------------------------------------------------- tiles and launchers
// K slice depth and ring depth of the large tile (build-time tuning knobs).
#ifndef GEMM_F16_T256_BK
#define GEMM_F16_T256_BK 32
#endif
#ifndef GEMM_F16_T256_STAGES
#define GEMM_F16_T256_STAGES 4
#endif
using Tile256 = Tile<256, 256, GEMM_F16_T256_BK, GEMM_F16_T256_STAGES, 2, 2>;
#ifndef GEMM_F16_T128_STAGES
#define GEMM_F16_T128_STAGES 4
#endif
#ifndef GEMM_F16_T64_STAGES
#define GEMM_F16_T64_STAGES 4
#endif
using Tile128 = Tile<128, 128, 32, GEMM_F16_T128_STAGES, 2, 2>;
using Tile64 = Tile<64, 64, 32, GEMM_F16_T64_STAGES, 2, 2>;
using Tile256x128 = Tile<256, 128, 32, 4, 2, 2>;
#ifndef GEMM_F16_T128K_STAGES
#define GEMM_F16_T128K_STAGES 4
#endif
using Tile128K4 = Tile<128, 128, 64, GEMM_F16_T128K_STAGES, 1, 1, 1, 4>;


template <class TL>
constexpr TileInfo info_of()
{
    return TileInfo{TL::BM, TL::BN, TL::BK, TL::T, TL::LDS_BYTES};
}

template <class TL>
hipError_t launch(const Params &p, int64_t grid, hipStream_t stream, int splits = 1)
{
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_f16_f32_kernel<TL>),
                           dim3((unsigned)grid, (unsigned)splits), dim3(TL::T), args, 0, stream);
}

}  // namespace

namespace gemm_f16 {

#if GEMM_F16_TA == 0 && GEMM_F16_TB == 0
TileInfo tile_info(int tile)
{
    switch (tile) {
    case GEMM_F16_TILE_256x256: return info_of<Tile256>();
    case GEMM_F16_TILE_128x128: return info_of<Tile128>();
    case GEMM_F16_TILE_64x64: return info_of<Tile64>();
    case GEMM_F16_TILE_256x128: return info_of<Tile256x128>();
    case GEMM_F16_TILE_128x128_K4: return info_of<Tile128K4>();
    default: return TileInfo{0, 0, 0, 0, 0};
    }
}
#define GEMM_F16_LAUNCH_LAYOUT launch_tile_nn
#elif GEMM_F16_TA == 0 && GEMM_F16_TB == 1
#define GEMM_F16_LAUNCH_LAYOUT launch_tile_nt
#elif GEMM_F16_TA == 1 && GEMM_F16_TB == 0
#define GEMM_F16_LAUNCH_LAYOUT launch_tile_tn
#else
#define GEMM_F16_LAUNCH_LAYOUT launch_tile_tt
#endif

#if GEMM_F16_PHASES
// Measurement builds: where this layout's kernels stamp their phases (NULL: nowhere), grid x splits x 8
// u64 per launch; gemm_f16_phase_buffer_nn / _nt / _tn / _tt, one per layout object.  Returns the
// hipMemcpyToSymbol status.
#define GEMM_F16_PHASE_SETTER_(x) gemm_f16_phase_buffer_##x
#define GEMM_F16_PHASE_SETTER(x) GEMM_F16_PHASE_SETTER_(x)
#if GEMM_F16_TA == 0 && GEMM_F16_TB == 0
#define GEMM_F16_LAYOUT_TAG nn
#elif GEMM_F16_TA == 0
#define GEMM_F16_LAYOUT_TAG nt
#elif GEMM_F16_TB == 0
#define GEMM_F16_LAYOUT_TAG tn
#else
#define GEMM_F16_LAYOUT_TAG tt
#endif
extern "C" hipError_t GEMM_F16_PHASE_SETTER(GEMM_F16_LAYOUT_TAG)(void *buf)
{
    return hipMemcpyToSymbol(HIP_SYMBOL(phase_times), &buf, sizeof(buf));
}
#endif

hipError_t GEMM_F16_LAUNCH_LAYOUT(int tile, const Params &p, int64_t grid, hipStream_t s, int splits)
{
    constexpr bool TA = GEMM_F16_TA != 0, TB = GEMM_F16_TB != 0;
    switch (tile) {
    case GEMM_F16_TILE_256x256: return launch<WithLayout<Tile256, TA, TB>>(p, grid, s, splits);
    case GEMM_F16_TILE_128x128: return launch<WithLayout<Tile128, TA, TB>>(p, grid, s, splits);
    case GEMM_F16_TILE_64x64: return launch<WithLayout<Tile64, TA, TB>>(p, grid, s, splits);
    case GEMM_F16_TILE_256x128: return launch<WithLayout<Tile256x128, TA, TB>>(p, grid, s, splits);
    case GEMM_F16_TILE_128x128_K4: return launch<WithLayout<Tile128K4, TA, TB>>(p, grid, s, splits);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gemm_f16
