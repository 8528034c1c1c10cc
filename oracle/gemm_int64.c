/* Integer GEMM on INT4 codes with int64 accumulation — ORACLE, test
 * infrastructure only (the GPU library never links or calls this file).
 *
 * Method: the W4A4 product of SpinQuant (abstract; page "SpinQuant,
 * Reproduced", Q7/Q8: 4-bit weights and activations).  With per-token
 * activation codes qx[m][k] and per-output-channel weight codes qw[n][k]
 * (both int8 holding values in [-8, 7]), the integer product is
 *     acc[m][n] = sum_k qx[m][k] * qw[n][k]
 * accumulated exactly in int64.  Rows of qw are output channels, so both
 * operands are K-contiguous.  The dequantisation epilogue lives in Python.
 *
 * oracle_gemm_i64_rows computes only the rows listed in `rows` (used when the
 * full product is too slow to form on the CPU); oracle_gemm_i64 computes all.
 * Plain loops, no blocking; OpenMP splits the output rows across threads.
 */
#include <stdint.h>
#include <stddef.h>

static void row_dot(const int8_t *x, const int8_t *qw, int N, int K, int64_t *out)
{
    for (int n = 0; n < N; ++n) {
        const int8_t *w = qw + (size_t)n * (size_t)K;
        int64_t acc = 0;
        for (int k = 0; k < K; ++k)
            acc += (int64_t)x[k] * (int64_t)w[k];
        out[n] = acc;
    }
}

void oracle_gemm_i64(const int8_t *qx, const int8_t *qw, int M, int N, int K, int64_t *acc)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m)
        row_dot(qx + (size_t)m * (size_t)K, qw, N, K, acc + (size_t)m * (size_t)N);
}

void oracle_gemm_i64_rows(const int8_t *qx, const int8_t *qw, const int64_t *rows, int R,
                          int N, int K, int64_t *acc)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < R; ++i)
        row_dot(qx + (size_t)rows[i] * (size_t)K, qw, N, K, acc + (size_t)i * (size_t)N);
}

int oracle_num_threads(void)
{
    int t = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
