/*
 * sgemm_oracle.c -- the CPU oracle for C = A x B (FP32 operands, fp64 arithmetic).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link, load or call
 * this file: it is used by tests/, by the smoke check of __graft_entry__.py and by the
 * cpu_baseline leg of bench.py, and by nothing else. It shares no code, header, helper
 * or constant with the HIP library under fp32_gemm_f32_amd/csrc.
 *
 * What it computes is the plain definition of the product that every page builds on:
 *   - "SGEMM: Shared Memory Tiling Visualizer", section "Why Tiling Works (The Math)":
 *     each output element is the dot product of one row of A and one column of B, both
 *     of length K; A is M x K and B is K x N, stored row-major (A[row*K+k], B[k*N+col],
 *     C[row*N+col] in that page's code panel).
 *   - "Shared Memory Tiling", section "The naive kernel": the output element is the
 *     running sum over k of A[row][k] * B[k][col], written (not accumulated) into C.
 * Tiling and register tiling (the other sections and pages) change where the operands
 * are read from and how often, not the sums, so the oracle is the definition written
 * out, with no blocking:
 *
 *     C_ref[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N.
 *
 * Arithmetic: each FP32 operand is widened to double; the product of two FP32 values is
 * exact in double (24 + 24 significand bits <= 53), so the only roundings are the double
 * additions, taken in ascending k. Leading dimensions lda, ldb, ldc (in elements) let
 * the operands be sub-matrices of larger row-major arrays; the pages only show packed
 * arrays (lda = K, ldb = N, ldc = N), which is the special case.
 *
 * Rows are independent, so the OpenMP split over rows leaves every result bit-identical
 * for any thread count. Build: gcc -O2 -ffp-contract=off -fopenmp (no -ffast-math).
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Full product into a double matrix C (M x N, leading dimension ldc). */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda,
                    const float *B, int64_t ldb,
                    double *C, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M; ++i) {
        double *c = C + i * ldc;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = (double)A[i * lda + k];
            const float *b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) c[j] += a * (double)b[j];
        }
    }
    return 0;
}

/*
 * One row i of the product and of the magnitude sum den[j] = sum_k |A[i][k] * B[k][j]|,
 * the denominator of the normalised error used to judge floating-point results.
 */
static void oracle_row(int64_t i, int64_t N, int64_t K,
                       const float *A, int64_t lda, const float *B, int64_t ldb,
                       double *acc, double *den)
{
    for (int64_t j = 0; j < N; ++j) { acc[j] = 0.0; den[j] = 0.0; }
    for (int64_t k = 0; k < K; ++k) {
        const double a = (double)A[i * lda + k];
        const float *b = B + k * ldb;
        for (int64_t j = 0; j < N; ++j) {
            const double p = a * (double)b[j];
            acc[j] += p;
            den[j] += fabs(p);
        }
    }
}

/* Result of comparing an FP32 matrix against the oracle. */
typedef struct {
    double max_err;        /* max over checked elements of |C - C_ref| / den (den > 0)      */
    int64_t arg_i, arg_j;  /* where max_err occurs (first in row-major order on ties)      */
    int64_t n_checked;     /* elements compared                                            */
    int64_t n_inexact;     /* elements with C != (float)C_ref                              */
    int64_t n_nonfinite;   /* elements of C that are NaN or +-Inf                          */
    int64_t n_zero_den_bad;/* elements with den == 0 whose C is not zero                   */
} oracle_report;

static void report_init(oracle_report *r)
{
    r->max_err = 0.0; r->arg_i = -1; r->arg_j = -1;
    r->n_checked = 0; r->n_inexact = 0; r->n_nonfinite = 0; r->n_zero_den_bad = 0;
}

static void report_merge(oracle_report *into, const oracle_report *r)
{
    if (r->arg_i >= 0 &&
        (into->arg_i < 0 || r->max_err > into->max_err ||
         (r->max_err == into->max_err &&
          (r->arg_i < into->arg_i || (r->arg_i == into->arg_i && r->arg_j < into->arg_j))))) {
        into->max_err = r->max_err; into->arg_i = r->arg_i; into->arg_j = r->arg_j;
    }
    into->n_checked += r->n_checked;
    into->n_inexact += r->n_inexact;
    into->n_nonfinite += r->n_nonfinite;
    into->n_zero_den_bad += r->n_zero_den_bad;
}

/*
 * Compare C (FP32, M x N, ldc) against the oracle, row by row, without materialising a
 * double M x N matrix. rows == NULL checks every row; otherwise the nrows listed rows.
 * A non-finite C element counts as an infinite error.
 */
int oracle_check(int64_t M, int64_t N, int64_t K,
                 const float *A, int64_t lda, const float *B, int64_t ldb,
                 const float *Cq, int64_t ldc,
                 const int64_t *rows, int64_t nrows, oracle_report *out)
{
    if (M < 0 || N < 0 || K < 0 || !out) return -1;
    report_init(out);
    const int64_t count = rows ? nrows : M;
    int failed = 0;
#pragma omp parallel
    {
        oracle_report mine;
        report_init(&mine);
        double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *den = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!acc || !den) {
#pragma omp atomic write
            failed = 1;
        } else {
            int64_t t;
#pragma omp for schedule(dynamic, 1)
            for (t = 0; t < count; ++t) {
                const int64_t i = rows ? rows[t] : t;
                if (i < 0 || i >= M) continue;
                oracle_row(i, N, K, A, lda, B, ldb, acc, den);
                for (int64_t j = 0; j < N; ++j) {
                    const float c = Cq[i * ldc + j];
                    double err;
                    mine.n_checked++;
                    if (c != (float)acc[j]) mine.n_inexact++;
                    if (!isfinite(c)) {
                        mine.n_nonfinite++;
                        err = INFINITY;
                    } else if (den[j] == 0.0) {
                        if (c != 0.0f) mine.n_zero_den_bad++;
                        err = (c == 0.0f) ? 0.0 : INFINITY;
                    } else {
                        err = fabs((double)c - acc[j]) / den[j];
                    }
                    if (mine.arg_i < 0 || err > mine.max_err) {
                        mine.max_err = err; mine.arg_i = i; mine.arg_j = j;
                    }
                }
            }
        }
        free(acc);
        free(den);
#pragma omp critical
        report_merge(out, &mine);
    }
    return failed ? -2 : 0;
}

/*
 * Individual elements (ii[t], jj[t]) of the product and their magnitude sums, for
 * sampled checks of shapes too large to compute whole on the CPU.
 */
int oracle_sample(int64_t M, int64_t N, int64_t K,
                  const float *A, int64_t lda, const float *B, int64_t ldb,
                  int64_t n, const int64_t *ii, const int64_t *jj,
                  double *ref, double *den)
{
    if (M < 0 || N < 0 || K < 0) return -1;
    int64_t t;
    for (t = 0; t < n; ++t)
        if (ii[t] < 0 || ii[t] >= M || jj[t] < 0 || jj[t] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n; ++t) {
        double s = 0.0, d = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = (double)A[ii[t] * lda + k] * (double)B[k * ldb + jj[t]];
            s += p;
            d += fabs(p);
        }
        ref[t] = s;
        den[t] = d;
    }
    return 0;
}

/*
 * The transpose that the LDS bank-geometry microbenchmark computes ("Visual walkthrough -
 * Memory hierarchy", Step 6): out[j][i] = in[i][j]. A copy, so exact.
 */
int oracle_transpose(int64_t rows, int64_t cols, const float *in, int64_t ldi,
                     float *out, int64_t ldo)
{
    if (rows < 0 || cols < 0) return -1;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) out[j * ldo + i] = in[i * ldi + j];
    return 0;
}

/* Threads an OpenMP region of the oracle uses (1 when built without OpenMP). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of the oracle's later parallel regions (for timing it on one core);
 * returns the previous count. Results do not depend on it: rows are independent. */
int oracle_set_threads(int n)
{
    const int prev = oracle_threads();
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
    return prev;
}
