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
 * The general entry point also takes operand transposes, a per-column bias and a
 * GELU activation (documented at oracle_gemm_f64 below).
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

/* Operand forms: op == 0 reads the matrix as stored, op == 1 reads its transpose. */
static double a_at(const float *A, int64_t lda, int opA, int64_t i, int64_t k)
{
    return (double)(opA ? A[k * lda + i] : A[i * lda + k]);
}

static double b_at(const float *B, int64_t ldb, int opB, int64_t k, int64_t j)
{
    return (double)(opB ? B[j * ldb + k] : B[k * ldb + j]);
}

/* GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). */
double oracle_gelu_tanh(double x)
{
    const double c = sqrt(2.0 / 3.14159265358979323846);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* Largest slope of the tanh-form GELU over the reals (attained near x = 2.1); the
 * bound below carries an input error through the activation with this factor. */
#define GELU_SLOPE_MAX 1.13

/* Result and bound of one entry from its fp64 sums. */
static void finish(double s, double g, double c0, int K, float alpha, float beta, const float *bias,
                   int64_t j, int act, double *ref, double *bound)
{
    const double t_c = (beta == 0.0f) ? 0.0 : (double)beta * c0;
    const double b = bias ? (double)bias[j] : 0.0;
    const double t = (double)alpha * s + t_c + b;
    const double mag = fabs((double)alpha) * g + fabs(t_c) + fabs(b);
    /* The plain product keeps the bound 4 max(K,1) u (|alpha| g + |beta c|); one more
     * rounding (the bias add) widens the factor to 4 (max(K,1) + 1). */
    double e = 4.0 * (double)((K > 1 ? K : 1) + (bias || act ? 1 : 0)) * ldexp(1.0, -24) * mag;
    double r = t;
    if (act == 1) {
        r = oracle_gelu_tanh(t);
        /* input error through the activation, plus fp32 evaluation of the formula */
        e = GELU_SLOPE_MAX * e + 8.0 * ldexp(1.0, -24) * (fabs(t) + fabs(r));
    }
    *ref = r;
    if (bound)
        *bound = e;
}

/*
 * General oracle: C = act(alpha * op(A) op(B) + beta * C + bias) for the M x N window.
 * op(A) is M x K and op(B) is K x N:
 *   opA == 0: a_ik = A[i*lda + k]      opA == 1: a_ik = A[k*lda + i]
 *   opB == 0: b_kj = B[k*ldb + j]      opB == 1: b_kj = B[j*ldb + k]
 * bias (length N, by column) may be NULL; act is 0 (none) or 1 (tanh-form GELU).
 * Operand transposes as strided views follow the GPT-2 post ("Tiled matrix
 * multiplication"); the bias add after a product, and the GELU after the first MLP
 * product, follow its traced model ("The whole model as one kernel") and its GELU
 * kernel built from a power and a tanh ("From loops to kernels").
 * Writes ref (row stride ldr) and, if bound != NULL, the bound (row stride ldbd).
 * Returns 0, -1 if a work array cannot be allocated, -2 for a bad op or act.
 */
int oracle_gemm_f64(int opA, int opB, int M, int N, int K, float alpha,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    float beta, const float *C0, int64_t ldc,
                    const float *bias, int act,
                    double *ref, int64_t ldr, double *bound, int64_t ldbd)
{
    if (opA < 0 || opA > 1 || opB < 0 || opB > 1 || act < 0 || act > 1)
        return -2;
    if (M <= 0 || N <= 0)
        return 0;
    const int use_ab = (alpha != 0.0f) && (K > 0);
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
                    const double a = a_at(A, lda, opA, i, k);
                    if (bound != NULL) {
                        for (int j = 0; j < N; ++j) {
                            const double p = a * b_at(B, ldb, opB, k, j);
                            s[j] += p;
                            g[j] += fabs(p);
                        }
                    } else {
                        for (int j = 0; j < N; ++j)
                            s[j] += a * b_at(B, ldb, opB, k, j);
                    }
                }
            }
            for (int j = 0; j < N; ++j) {
                const double c0 = (beta == 0.0f) ? 0.0 : (double)C0[(int64_t)i * ldc + j];
                finish(s[j], g[j], c0, K, alpha, beta, bias, j, act, &ref[(int64_t)i * ldr + j],
                       bound ? &bound[(int64_t)i * ldbd + j] : NULL);
            }
        }
        free(s);
        free(g);
    }
    return failed ? -1 : 0;
}

/* The plain product C = alpha*A*B + beta*C (both operands as stored, no bias). */
int oracle_sgemm_f64(int M, int N, int K, float alpha,
                     const float *A, int64_t lda,
                     const float *B, int64_t ldb,
                     float beta, const float *C0, int64_t ldc,
                     double *ref, int64_t ldr,
                     double *bound, int64_t ldbd)
{
    return oracle_gemm_f64(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, NULL, 0, ref, ldr,
                           bound, ldbd);
}

/*
 * Sampled oracle: the same definition for `count` chosen entries (rows[e], cols[e]),
 * each a dot product over ascending k. Used where the full product is too large
 * to evaluate in seconds. Returns 0, -1 if an index is out of range, -2 for a bad op or act.
 */
int oracle_gemm_entries_f64(int opA, int opB, int M, int N, int K, float alpha,
                            const float *A, int64_t lda, const float *B, int64_t ldb,
                            float beta, const float *C0, int64_t ldc,
                            const float *bias, int act,
                            int64_t count, const int64_t *rows, const int64_t *cols,
                            double *ref, double *bound)
{
    if (opA < 0 || opA > 1 || opB < 0 || opB > 1 || act < 0 || act > 1)
        return -2;
    const int use_ab = (alpha != 0.0f) && (K > 0);
    for (int64_t e = 0; e < count; ++e)
        if (rows[e] < 0 || rows[e] >= M || cols[e] < 0 || cols[e] >= N)
            return -1;

#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        const int64_t i = rows[e], j = cols[e];
        double s = 0.0, g = 0.0;
        if (use_ab) {
            for (int k = 0; k < K; ++k) {
                const double p = a_at(A, lda, opA, i, k) * b_at(B, ldb, opB, k, j);
                s += p;
                g += fabs(p);
            }
        }
        const double c0 = (beta == 0.0f) ? 0.0 : (double)C0[i * ldc + j];
        finish(s, g, c0, K, alpha, beta, bias, j, act, &ref[e], bound ? &bound[e] : NULL);
    }
    return 0;
}

int oracle_sgemm_entries_f64(int M, int N, int K, float alpha,
                             const float *A, int64_t lda,
                             const float *B, int64_t ldb,
                             float beta, const float *C0, int64_t ldc,
                             int64_t count, const int64_t *rows, const int64_t *cols,
                             double *ref, double *bound)
{
    return oracle_gemm_entries_f64(0, 0, M, N, K, alpha, A, lda, B, ldb, beta, C0, ldc, NULL, 0, count,
                                   rows, cols, ref, bound);
}
