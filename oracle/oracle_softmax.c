/*
 * Reference oracle for the row softmax.  TEST INFRASTRUCTURE ONLY: only tests/, the smoke check
 * in __graft_entry__.py and the cpu_baseline leg of bench.py may load it.  It shares no code,
 * header or table with the GPU library.
 *
 * What it computes is the definition the pages' fusion demo uses (06_triton_style.py, CS349E
 * lecture 10, "block programming", demo 3, both the operator-by-operator and the fused version):
 * for every row i of an M x N matrix,
 *
 *     m_i = max_j x[i][j],   e[i][j] = exp(x[i][j] - m_i),   y[i][j] = e[i][j] / sum_j e[i][j],
 *
 * here in FP64 from FP32 inputs, with the sum over ascending j.  Subtracting the row maximum
 * changes nothing mathematically and keeps exp from overflowing.
 */
#include <math.h>
#include <stdint.h>

int oracle_softmax_rows(int64_t M, int64_t N, const float *x, int64_t ldx, double *y, int64_t ldy)
{
    if (M < 0 || N < 0 || (M > 0 && N > 0 && (ldx < N || ldy < N))) return -1;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < M; ++i) {
        const float *xr = x + i * ldx;
        double *yr = y + i * ldy;
        double m = -INFINITY;
        for (int64_t j = 0; j < N; ++j)
            if ((double)xr[j] > m) m = (double)xr[j];
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            yr[j] = exp((double)xr[j] - m);
            s += yr[j];
        }
        for (int64_t j = 0; j < N; ++j) yr[j] /= s;
    }
    return 0;
}
