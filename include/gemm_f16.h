/*
 * gemm_f16.h -- C ABI of the gfx950 (MI355X) FP16-input, FP32-accumulate matrix product.
 *
 * The operation is the dense product with the accumulate form
 *
 *     C <- A.B + beta.C      A: M x K, B: K x N (binary16), C: M x N (binary32)
 *
 * as defined on the pages: 04_tensor_cores.py (CS349E lecture 10, "Tensor Core kernels"),
 * the problem statement of the block kernel (FP16 A and B, FP32 accumulation) and demo 1's
 * D = A.B + C form of one matrix instruction; 06_triton_style.py (CS349E lecture 10, "block
 * programming"), the matmul launcher of demo 1 (FP32 C, one program per output tile, masked
 * edges so that any shape is valid).  beta is the plainest reading of "+ C": beta = 1 gives
 * D = A.B + C in place, beta = 0 gives C = A.B and C is then never read.
 *
 * Every product of two binary16 values is exact in binary32, and sums are accumulated in
 * binary32; the order of the additions is the library's own (several orders are correct).
 *
 * Layout: all matrices row-major with a unit column stride.  lda, ldb, ldc are row strides in
 * ELEMENTS (not bytes): A[i][k] is at A + i*lda + k, B[k][j] at B + k*ldb + j, C[i][j] at
 * C + i*ldc + j.  Requirements: lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N).
 * Alignment: A and B must be aligned to their 2-byte elements and C to its 4-byte elements
 * (GEMM_F16_ERR_ALIGN otherwise).  Nothing more is required: 16-byte aligned base pointers with
 * lda, ldb multiples of 8 take the direct-to-LDS path; any other layout takes 16-byte register
 * loads at whatever alignment the rows have.
 *
 * Pointers: A, B and C are DEVICE pointers (HIP device memory of the current device).  The
 * caller owns every buffer; the library allocates nothing, keeps no state between calls and
 * may be called from several host threads at once.  C must not overlap A or B.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls are
 * asynchronous: a return of 0 means the kernel was enqueued; faults during execution surface
 * at the caller's next synchronisation on that stream.
 *
 * Errors: every entry point returns 0 on success or one of the negative codes below.  Nothing
 * is enqueued when a call returns an error.  No entry point aborts or throws.
 */
#ifndef GEMM_F16_H
#define GEMM_F16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM_F16_OK 0
#define GEMM_F16_ERR_DIM (-1)       /* M, N or K negative, or larger than 2^30              */
#define GEMM_F16_ERR_LD (-2)        /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N)     */
#define GEMM_F16_ERR_NULL (-3)      /* NULL pointer for an operand that is read or written  */
#define GEMM_F16_ERR_OPTS (-4)      /* an option field out of range                         */
#define GEMM_F16_ERR_TOO_LARGE (-5) /* the tile grid does not fit one launch (workgroups x  */
                                    /* threads per workgroup must stay below 2^32)          */
#define GEMM_F16_ERR_LAUNCH (-6)    /* the HIP runtime refused the launch                   */
#define GEMM_F16_ERR_ALIGN (-7)     /* A or B not 2-byte aligned, or C not 4-byte aligned   */
#define GEMM_F16_ERR_WORKSPACE (-8) /* split-K workspace missing or smaller than required   */
#define GEMM_F16_ERR_SCRATCH (-9)   /* split-K partials larger than the fixed scratch        */

/* Tile configurations (BM x BN output tile per workgroup; K streamed in slices of BK = 32 through
 * an LDS ring four slices deep: the K-contiguous operand in three stages of two slices, the other
 * in four stages of one; LDS per workgroup as listed). */
#define GEMM_F16_TILE_AUTO 0
#define GEMM_F16_TILE_256x256 1 /* 4 waves, 128 x 128 per wave, 160 KiB of LDS */
#define GEMM_F16_TILE_128x128 2 /* 4 waves,  64 x  64 per wave,  80 KiB of LDS */
#define GEMM_F16_TILE_64x64 3   /* 4 waves,  32 x  32 per wave,  40 KiB of LDS */
#define GEMM_F16_TILE_256x128 4 /* 4 waves, 128 x  64 per wave, 128 KiB of LDS */
/* 4 waves that split K: each computes the whole 128 x 128 block over every fourth k16 step of a
 * BK = 64 slice, and the partial sums are added in the epilogue; 4 x 32 KiB LDS stages (128 KiB). */
#define GEMM_F16_TILE_128x128_K4 5
#define GEMM_F16_TILE_COUNT 6

/*
 * Launch-order and tile options.  All-zero fields (and xcd_remap = -1) mean "choose".
 *   tile      GEMM_F16_TILE_* (0 = chosen from the shape)
 *   group_m   output-tile rows per group of the grouped launch order (06_triton_style.py,
 *             demo 2: programs walk GROUP_M tile-rows down before moving right); 1 = plain
 *             row-major order; 0 = chosen.  Range 0..65535.
 *   xcd_remap 1 = renumber workgroups so that each of the 8 XCDs (each with its own L2) runs
 *             a contiguous run of the launch order; 0 = hardware order; -1 = chosen.
 *   path      GEMM_F16_PATH_AUTO (0): direct-to-LDS staging wherever rows are 16-byte aligned;
 *             GEMM_F16_PATH_REGISTER (1): every tile through the register-staged masked path
 *             (the path unaligned operands take), for testing and measurement.
 */
#define GEMM_F16_PATH_AUTO 0
#define GEMM_F16_PATH_REGISTER 1
typedef struct gemm_f16_f32_opts {
    int32_t tile;
    int32_t group_m;
    int32_t xcd_remap;
    int32_t path;
} gemm_f16_f32_opts;

/* What a call with these arguments launches (filled by gemm_f16_f32_plan). */
typedef struct gemm_f16_f32_plan_t {
    int32_t tile;      /* GEMM_F16_TILE_* actually used                         */
    int32_t bm, bn, bk;
    int32_t threads;   /* per workgroup                                         */
    int32_t lds_bytes; /* per workgroup                                         */
    int32_t group_m;
    int32_t xcd_remap;
    int32_t vec_a;     /* 1 if A is staged direct-to-LDS (16-byte aligned rows)  */
    int32_t vec_b;     /* 1 if B is staged direct-to-LDS (16-byte aligned rows)  */
    int64_t tiles_m, tiles_n, grid;   /* the (first) launch's tile grid                  */
    int64_t split_at;  /* rows (split_dim 0) or columns (1) of C the first launch */
                       /* covers: M (or N) unless split                          */
    int32_t tile2;     /* 0, or the tile of a second launch over the rest        */
    int32_t split_dim; /* 0: split by rows of C, 1: by columns                   */
    int64_t grid2;     /* workgroups of the second launch (0 if none)            */
} gemm_f16_f32_plan_t;

/*
 * C <- A.B + beta.C on `stream` (FP16 A, B; FP32 accumulate and C): the block-tiled product of
 * 04_tensor_cores.py (CS349E lecture 10, "Tensor Core kernels": FP16 operands, FP32 accumulation,
 * demo 1's D = A.B + C) and 06_triton_style.py (CS349E lecture 10, "block programming", demo 1's
 * matmul launcher: FP32 C, any shape through masked edges), with beta as the plainest reading of "+ C".
 * M == 0 or N == 0: no-op (returns 0, nothing launched).  K == 0: C <- beta.C (zeros if beta == 0,
 * C not read).  beta == 0: C is write-only (NaNs in it do not propagate).
 * Arguments: sizes and strides as above; A, B, C device pointers; beta a binary32 scalar;
 * stream a hipStream_t or NULL.  The call is one kernel launch on `stream`, or two in order when
 * the planner splits the rows or columns of C against wave quantisation (gemm_f16_f32_plan
 * reports it: tile2 != 0); either way each element of C is computed by one workgroup.
 */
int gemm_f16_f32(int64_t M, int64_t N, int64_t K,
                 const void *A, int64_t lda,
                 const void *B, int64_t ldb,
                 float *C, int64_t ldc,
                 float beta, void *stream);

/* Same as gemm_f16_f32 with explicit options; opts == NULL means all automatic.  The options pick the
 * tile (the block size of 04_tensor_cores.py demo 3), GROUP_M and the XCD renumbering of the launch
 * order (06_triton_style.py demo 2) and the staging path; the result is the same product. */
int gemm_f16_f32_ex(int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    float *C, int64_t ldc,
                    float beta, void *stream,
                    const gemm_f16_f32_opts *opts);

/*
 * Host-only: validate the arguments exactly as gemm_f16_f32_ex does and describe the launch it
 * would make, without touching the GPU.  Pointers are used only for their alignment (NULL is
 * treated as aligned).  Returns 0 or the error code the call would return.
 */
int gemm_f16_f32_plan(int64_t M, int64_t N, int64_t K,
                      const void *A, int64_t lda,
                      const void *B, int64_t ldb,
                      const void *C, int64_t ldc,
                      const gemm_f16_f32_opts *opts, gemm_f16_f32_plan_t *plan);

/*
 * Host-only: the launch order.  For workgroup ids 0..count-1 of a tiles_m x tiles_n grid,
 * write the output-tile coordinates each workgroup computes (the same function the kernels
 * use).  group_m >= 1; xcd_remap 0 or 1.  Returns 0, GEMM_F16_ERR_DIM if count exceeds
 * tiles_m*tiles_n or a size is negative, GEMM_F16_ERR_OPTS for a bad group_m/xcd_remap,
 * GEMM_F16_ERR_NULL for NULL outputs (when count > 0).
 */
int gemm_f16_f32_tile_order(int64_t tiles_m, int64_t tiles_n, int32_t group_m, int32_t xcd_remap,
                            int64_t count, int64_t *pid_m, int64_t *pid_n);

/*
 * Transposed operands: C <- op(A).op(B) + beta.C with op(A) = A (trans_a = 0: A stored M x K,
 * lda >= max(1, K)) or A^T (trans_a = 1: A stored K x M, lda >= max(1, M)), and op(B) = B
 * (trans_b = 0: B stored K x N, ldb >= max(1, N)) or B^T (trans_b = 1: B stored N x K,
 * ldb >= max(1, K)).  Every layout takes the same tiles, pipeline and edge handling: an operand
 * stored with K contiguous (A as given, B transposed) is staged into LDS as rows of K and read
 * with ds_read_b128, the other kind as rows of M or N and read with transposing LDS reads.  Other
 * arguments, options and errors as gemm_f16_f32_ex (GEMM_F16_ERR_OPTS for a trans flag other than
 * 0 or 1).  gemm_f16_f32_ex is gemm_f16_f32_tt(0, 0, ...).  The pages' block kernel keeps B
 * transposed in shared memory for the same reason (04_tensor_cores.py, the block kernel's
 * structure); 06_triton_style.py's matmul takes any strides.
 */
int gemm_f16_f32_tt(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda,
                    const void *B, int64_t ldb,
                    float *C, int64_t ldc,
                    float beta, void *stream,
                    const gemm_f16_f32_opts *opts);

/* Host-only planning for gemm_f16_f32_tt, as gemm_f16_f32_plan. */
int gemm_f16_f32_plan_tt(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                         const void *A, int64_t lda,
                         const void *B, int64_t ldb,
                         const void *C, int64_t ldc,
                         const gemm_f16_f32_opts *opts, gemm_f16_f32_plan_t *plan);

/*
 * Split-K, for problems with few output tiles and a long K (the output-tile grid alone would
 * leave most compute units idle).  K is cut into at most `splits` contiguous ranges, each a
 * multiple of the tile's K slice; the workgroups of range s compute op(A)[:, range] . op(B)[range, :]
 * into slice s of `workspace` (an M x N FP32 matrix whose row stride is N rounded up to a multiple
 * of 4); a second kernel then writes C <- (sum of the slices) + beta.C.  The slices are added in an
 * order fixed by M, N and the split count alone (in slice order within each of up to 16 groups of
 * consecutive slices, then the group sums in group order), so results are deterministic; they
 * differ from the unsplit call only by rounding order.
 *   splits     1 .. 1024; 1 (or a K too short to split) is gemm_f16_f32_tt and needs no workspace.
 *   workspace  caller-owned device memory, 16-byte aligned, at least
 *              gemm_f16_f32_splitk_workspace(M, N, splits) bytes (GEMM_F16_ERR_WORKSPACE otherwise);
 *              its contents are overwritten; it must not overlap A, B or C.
 * Other arguments, options and errors as gemm_f16_f32_tt.  Both kernels run on `stream`.
 */
int gemm_f16_f32_splitk(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda,
                        const void *B, int64_t ldb,
                        float *C, int64_t ldc,
                        float beta, int splits, void *workspace, size_t workspace_bytes,
                        void *stream, const gemm_f16_f32_opts *opts);

/* Bytes of workspace gemm_f16_f32_splitk needs for these sizes (0 when splits <= 1). */
size_t gemm_f16_f32_splitk_workspace(int64_t M, int64_t N, int splits);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): gemm_f16_f32_splitk with its partial products in a
 * scratch array of GEMM_F16_SCRATCH_BYTES (32 MiB) inside the library instead of a caller
 * workspace.  The caller still passes A, B and C; arguments, results and errors are those of
 * gemm_f16_f32_splitk, and the results are bit for bit the same.
 *   - No allocation: the call makes no hipMalloc / hipFree and calls no allocating routine.  Each
 *     GPU the library runs on holds its own copy of the array from the first call on it until
 *     the process ends; that first call looks up the copy's address (hipGetSymbolAddress) with
 *     the device current.
 *   - Limit: splits * M * (N rounded up to a multiple of 4) * 4 bytes must not exceed
 *     GEMM_F16_SCRATCH_BYTES for the split count actually used; larger problems return
 *     GEMM_F16_ERR_SCRATCH before any GPU work (use gemm_f16_f32_splitk with a workspace).
 *     Calls that do not split (splits = 1, or K too short) need no scratch.
 *   - Sharing: every call on one GPU uses that GPU's one array, which keeps the last call's
 *     contents.  Nothing in it needs to start at zero (each element the second pass reads is
 *     written by the first kernel of the same call), but calls that overlap on one GPU (two
 *     streams, or two host threads without ordering) race on it; order them on one stream.
 */
#define GEMM_F16_SCRATCH_BYTES ((size_t)32 << 20)
int gemm_f16_f32_splitk_noalloc(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                                const void *A, int64_t lda,
                                const void *B, int64_t ldb,
                                float *C, int64_t ldc,
                                float beta, int splits, void *stream, const gemm_f16_f32_opts *opts);

/*
 * The split count the library's cost model expects to be fastest for an M x N x K product (1: do
 * not split), for gemm_f16_f32_splitk with default options.  The model takes the largest of three
 * bounds for the tile that call would use -- whole waves of 256 workgroups at the tile's sustained
 * matrix-core rate, each workgroup streaming its A and B panels at the rate its ring depth allows,
 * and A, B and C once from HBM -- plus the second pass's traffic and launch, keeps at least 1024 K
 * rows per range, and splits only when that is predicted at least 10 % faster than the plain call:
 * problems whose output tiles leave compute units idle (deep K) or keep too few loads in flight
 * (a few rows or columns, long K).  Pure host arithmetic, no GPU call.
 */
int gemm_f16_f32_splitk_choose(int64_t M, int64_t N, int64_t K);

/* A static, human-readable string for an error code (never NULL). */
const char *gemm_f16_f32_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_H */
