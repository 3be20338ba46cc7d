/*
 * Oracle for the FP32 GEMM C = A.B -- TEST INFRASTRUCTURE, not part of the product.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg load this file's
 * library.  It shares no code, header or constant with the GPU library.
 *
 * What it computes (the plain definition of the product):
 *   C64[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j]        accumulated in FP64, k ascending
 *   Bnd[i][j] = sum_{k=0}^{K-1} |A[i][k]| * |B[k][j]|      accumulated in FP64
 * for row-major A (M x K, leading dimension lda) and B (K x N, leading dimension ldb).
 *
 * Source of the definition: "Double Buffering" (metalworking glossary), opening paragraph
 * and code figure -- the K-loop walks tiles of A and B and accumulates their product; the
 * schedule (one or two staging buffers) does not change what is summed.  The LuisaCompute
 * note "Dependence-aware group synchronization on M1 Max", section "Transformation and
 * safety boundary", states that moving barriers changes neither the order of operations
 * nor their distribution, and its section "Controlled implementation comparison" checks
 * every output against an FP64 oracle.  The loops below are the textbook i-k-j triple loop;
 * there is no blocking and no reordering of the k sum.
 *
 * Products of two FP32 values are exact in FP64 (24 + 24 significant bits <= 53), so the
 * only rounding is in the FP64 running sums.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Full output.  C64 and Bnd are M x N with leading dimension ldo (FP64).  Returns 0, or -1
 * on a bad argument (negative size, leading dimension too small, null pointer). */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    double *C64, double *Bnd, int64_t ldo)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    if (M == 0 || N == 0) return 0;
    if (ldo < N || (K > 0 && (lda < K || ldb < N))) return -1;
    if (!C64 || !Bnd || (K > 0 && (!A || !B))) return -1;

    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *c = C64 + i * ldo;
        double *b = Bnd + i * ldo;
        for (int64_t j = 0; j < N; ++j) { c[j] = 0.0; b[j] = 0.0; }
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *brow = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) {
                const double p = a * (double)brow[j];
                c[j] += p;
                b[j] += fabs(p);
            }
        }
    }
    return 0;
}

/* Sampled output: the same sums, for `count` positions (rows[s], cols[s]).  Returns 0, or
 * -1 on a bad argument (including a position outside M x N). */
int oracle_gemm_f64_sampled(int64_t M, int64_t N, int64_t K,
                            const float *A, int64_t lda,
                            const float *B, int64_t ldb,
                            int64_t count, const int64_t *rows, const int64_t *cols,
                            double *c64, double *bnd)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (count == 0) return 0;
    if (!rows || !cols || !c64 || !bnd) return -1;
    if (K > 0 && (!A || !B || lda < K || ldb < N)) return -1;
    for (int64_t s = 0; s < count; ++s)
        if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N) return -1;

    int64_t s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < count; ++s) {
        const int64_t i = rows[s], j = cols[s];
        double c = 0.0, b = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = (double)A[i * lda + k] * (double)B[k * ldb + j];
            c += p;
            b += fabs(p);
        }
        c64[s] = c;
        bnd[s] = b;
    }
    return 0;
}
