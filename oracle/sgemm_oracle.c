/*
 * CPU oracle for C = alpha * A * B + beta * C on row-major fp32 matrices.
 *
 * TEST INFRASTRUCTURE ONLY. Tests, the smoke check and the benchmark's CPU
 * baseline may call it. The GPU library never links, loads or calls it, and it
 * shares no code with that library.
 *
 * What it computes (the plain definition, evaluated in IEEE binary64):
 *
 *   s_ij   = sum_{k = 0 .. K-1} a_ik * b_kj     (k ascending, one fp64 accumulator)
 *   g_ij   = sum_{k = 0 .. K-1} |a_ik * b_kj|
 *   t_ij   = beta * c_ij, or 0 when beta == 0  (C is then not read at all)
 *   ref_ij = alpha * s_ij + t_ij
 *   bound_ij = 4 * max(K, 1) * 2^-24 * (|alpha| * g_ij + |t_ij|)
 *
 * Sources on the pages:
 *  - Each entry of AB is the dot product of a row of A with a column of B;
 *    AutoMine++ #4, "Current algorithm". Summing outer products of A's columns
 *    and B's rows gives the same matrix; same page, "Matrix product by outer
 *    products of vectors".
 *  - The result form alpha*acc + beta*C, with C not read when beta is zero;
 *    "Micro_gemm_4x4 - cuBLAS micro GEMM skeleton", section "Final C write
 *    (alpha, beta)". Its "Kernel signature" section writes the formula as
 *    alpha times A plus beta times C; the final-write code multiplies the
 *    accumulated product, which is the reading taken here.
 *  - Tiled and library results differ only through the order of accumulation;
 *    "GPU Target - GPT-2 on the GPU", section "Running it". That is why the
 *    comparison is against a bound and not bitwise.
 *
 * Readings where the pages are silent:
 *  - alpha == 0 or K == 0: A and B are not read and s = g = 0 (the usual BLAS
 *    quick return), so the result is beta*C.
 *  - beta == 0: C is not read, so NaN or Inf already in C has no effect.
 *  - max(K, 1) keeps a nonzero bound for the one rounding of beta*c at K = 0.
 *
 * Why fp64 suffices: an fp32 x fp32 product has at most 48 significant bits, so
 * it is exact in binary64; the fp64 summation error, at most (K-1) * 2^-53 * g,
 * is about 2^-31 of the bound.
 *
 * Leading dimensions: a_ik = A[i*lda + k], b_kj = B[k*ldb + j], c_ij = C[i*ldc + j].
 * Offsets are computed in 64-bit integers.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of host threads the oracle runs with (OpenMP over rows of C). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static double bound_scale(int K)
{
    return 4.0 * (double)(K > 1 ? K : 1) * ldexp(1.0, -24);
}

/*
 * Full oracle. Writes ref (M x N, row stride ldr) and, when bound != NULL, the
 * per-entry bound (row stride ldbd). Returns 0, or -1 if a work array cannot be
 * allocated. C0 may be NULL when beta == 0.
 */
int oracle_sgemm_f64(int M, int N, int K, float alpha,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float beta, const float *C0, int64_t ldc,
                     double *ref, int64_t ldr,
                     double *bound, int64_t ldbd)
{
    if (M <= 0 || N <= 0)
        return 0;
    const int use_ab = (alpha != 0.0f) && (K > 0);
    const double scale = bound_scale(K);
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)calloc((size_t)N, sizeof(double));
        double *g = (double *)calloc((size_t)N, sizeof(double));
        if (s == NULL || g == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < M; ++i) {
            if (s == NULL || g == NULL)
                continue;
            for (int j = 0; j < N; ++j) {
                s[j] = 0.0;
                g[j] = 0.0;
            }
            if (use_ab) {
                /* i-k-j order: for every j the terms still arrive in ascending k. */
                for (int k = 0; k < K; ++k) {
                    const double a = (double)A[(int64_t)i * lda + k];
                    const float *brow = B + (int64_t)k * ldb;
                    if (bound != NULL) {
                        for (int j = 0; j < N; ++j) {
                            const double p = a * (double)brow[j];
                            s[j] += p;
                            g[j] += fabs(p);
                        }
                    } else {
                        for (int j = 0; j < N; ++j)
                            s[j] += a * (double)brow[j];
                    }
                }
            }
            for (int j = 0; j < N; ++j) {
                const double t = (beta == 0.0f) ? 0.0 : (double)beta * (double)C0[(int64_t)i * ldc + j];
                ref[(int64_t)i * ldr + j] = (double)alpha * s[j] + t;
                if (bound != NULL)
                    bound[(int64_t)i * ldbd + j] = scale * (fabs((double)alpha) * g[j] + fabs(t));
            }
        }
        free(s);
        free(g);
    }
    return failed ? -1 : 0;
}

/*
 * Sampled oracle: the same definition for `count` chosen entries (rows[e], cols[e]),
 * each a dot product over ascending k. Used where the full product is too large
 * to evaluate in seconds. Returns 0, or -1 if an index is out of range.
 */
int oracle_sgemm_entries_f64(int M, int N, int K, float alpha,
                             const float *A, int64_t lda,
                             const float *B, int64_t ldb,
                             float beta, const float *C0, int64_t ldc,
                             int64_t count, const int64_t *rows, const int64_t *cols,
                             double *ref, double *bound)
{
    const int use_ab = (alpha != 0.0f) && (K > 0);
    const double scale = bound_scale(K);
    for (int64_t e = 0; e < count; ++e)
        if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N)
            return -1;

#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        const int64_t i = rows[e], j = cols[e];
        double s = 0.0, g = 0.0;
        if (use_ab) {
            for (int k = 0; k < K; ++k) {
                const double p = (double)A[i * lda + k] * (double)B[(int64_t)k * ldb + j];
                s += p;
                g += fabs(p);
            }
        }
        const double t = (beta == 0.0f) ? 0.0 : (double)beta * (double)C0[i * ldc + j];
        ref[e] = (double)alpha * s + t;
        if (bound != NULL)
            bound[e] = scale * (fabs((double)alpha) * g + fabs(t));
    }
    return 0;
}
