/*
 * Reference oracle for C <- A.B + beta.C with FP16 inputs.  TEST INFRASTRUCTURE ONLY:
 * only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg of bench.py
 * may load this library.  It shares no code, header or table with the GPU library.
 *
 * What it computes is the plain definition of the product, accumulated in FP64:
 *
 *     D[i][j] = ( sum_{k=0}^{K-1} A[i][k] * B[k][j] )  +  beta * Cin[i][j]
 *
 * with the sum taken over ascending k in double precision, then beta*Cin added once.
 * The pages use exactly this as their high-precision reference:
 *   - 04_tensor_cores.py (CS349E lecture 10, "Tensor Core kernels"), demo 1 and demo 2:
 *     FP16 inputs promoted to FP64 and multiplied, D = A.B + C, compared against the
 *     FP32-accumulating tensor-core result;
 *   - 06_triton_style.py (CS349E lecture 10, "block programming"), demo 1 and demo 4:
 *     the kernel under test is compared against an FP64 product of the same inputs.
 * The tiling, swizzle, launch order and pipelining described on the pages change only
 * where data sits and in which order blocks run, not the mathematical result
 * (04_tensor_cores.py, demo 2 observations: the swizzle changes physical addresses only),
 * so the oracle has none of them.
 *
 * Inputs are IEEE 754 binary16 bit patterns; they are decoded here by a decoder written
 * from the binary16 definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction
 * bits; exponent 0 = subnormal, exponent 31 = Inf/NaN).  Subnormal inputs are honoured.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC (no fast-math), so every
 * multiply and add is an individually rounded IEEE double operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* binary16 bit pattern -> double, from the format's definition. */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);              /* subnormal: frac * 2^-14 * 2^-10 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* All 65536 decodings, filled once; lookups are the same values the decoder returns. */
static double g_f16_table[65536];
static int g_f16_table_ready = 0;

static void ensure_table(void)
{
    if (g_f16_table_ready) return;
    for (int h = 0; h < 65536; ++h) g_f16_table[h] = oracle_f16_to_f64((uint16_t)h);
    g_f16_table_ready = 1;
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * D (M x N, row stride ldd, FP64) <- A.B + beta*Cin.
 *   A: M x K binary16, row-major, row stride lda (elements)
 *   B: K x N binary16, row-major, row stride ldb
 *   Cin: M x N FP32, row stride ldc; read only when beta != 0 (may be NULL otherwise)
 * Returns 0, or -1 for invalid sizes/strides, -2 for a NULL operand that is needed,
 * -3 if a work buffer cannot be allocated.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb,
                double beta, const float *Cin, int64_t ldc,
                double *D, int64_t ldd)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (lda < (K > 1 ? K : 1) || ldb < N || ldd < N) return -1;
    if (beta != 0.0 && ldc < N) return -1;
    if (D == NULL || (K > 0 && (A == NULL || B == NULL)) || (beta != 0.0 && Cin == NULL)) return -2;
    ensure_table();

    int failed = 0;
#pragma omp parallel
    {
        double *acc = (double *)malloc((size_t)N * sizeof(double));
        if (acc == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            if (acc == NULL) continue;
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            /* i-k-j order: every acc[j] still receives its K terms in ascending k. */
            for (int64_t k = 0; k < K; ++k) {
                const double a = g_f16_table[A[i * lda + k]];
                const uint16_t *brow = B + k * ldb;
                for (int64_t j = 0; j < N; ++j) acc[j] += a * g_f16_table[brow[j]];
            }
            double *drow = D + i * ldd;
            if (beta != 0.0) {
                const float *crow = Cin + i * ldc;
                for (int64_t j = 0; j < N; ++j) drow[j] = acc[j] + beta * (double)crow[j];
            } else {
                for (int64_t j = 0; j < N; ++j) drow[j] = acc[j];
            }
        }
        free(acc);
    }
    return failed ? -3 : 0;
}

/*
 * Number of pairs (x[i], y[j]) whose product, taken as an FP32 multiply of the two values
 * converted to FP32, differs from their exact product.  The exact product is the FP64 one, which
 * is exact whenever the two FP32 significands (at most 24 bits each) multiply into at most 53
 * bits -- always true for values that are already FP32, and the callers pass only such values.
 * Both the scan over every FP16 pair below and the tests' control sets (values with more than
 * 11 significant bits, whose FP32 products must round) go through this one routine, so a slip in
 * it (a product taken in double, a missed conversion) shows up as a wrong control count.
 */
static int64_t count_inexact_pairs(const double *x, int64_t nx, const double *y, int64_t ny)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad)
    for (int64_t i = 0; i < nx; ++i) {
        const float xf = (float)x[i];
        int64_t local = 0;
        for (int64_t j = 0; j < ny; ++j) {
            volatile float pf = xf * (float)y[j];   /* an FP32 multiply, rounded to FP32 */
            const double pd = x[i] * y[j];          /* exact for FP32 inputs */
            local += ((double)pf != pd);
        }
        bad += local;
    }
    return bad;
}

/*
 * The control entry point: count_inexact_pairs over caller-given values.  Returns -1 for a
 * negative count, NULL arrays with a positive count, or a value that is not exactly an FP32 number
 * (its FP64 product would then not be exact and the count would mean nothing).
 */
int64_t oracle_count_inexact_products(const double *x, int64_t nx, const double *y, int64_t ny)
{
    if (nx < 0 || ny < 0 || (nx > 0 && x == NULL) || (ny > 0 && y == NULL)) return -1;
    for (int64_t i = 0; i < nx; ++i)
        if ((double)(float)x[i] != x[i]) return -1;
    for (int64_t j = 0; j < ny; ++j)
        if ((double)(float)y[j] != y[j]) return -1;
    return count_inexact_pairs(x, nx, y, ny);
}

/*
 * The pages state that the product of two FP16 numbers is exact in FP32, because two
 * 11-bit significands multiply into at most 22 bits (04_tensor_cores.py, demo 1
 * observations).  This walks every pair of finite binary16 values and counts the pairs
 * whose FP32 product differs from the exact (FP64) product.  *checked receives the
 * number of pairs examined (63488^2 for the finite set).
 */
int64_t oracle_count_inexact_f16_products(int64_t *checked)
{
    ensure_table();
    /* finite values: exponent field != 31 */
    static double finite[65536];
    int64_t nf = 0;
    for (int h = 0; h < 65536; ++h)
        if (((h >> 10) & 0x1f) != 31) finite[nf++] = g_f16_table[h];
    if (checked) *checked = nf * nf;
    return count_inexact_pairs(finite, nf, finite, nf);
}
