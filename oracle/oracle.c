/*
 * oracle.c -- plain CPU reference for fp32 matrix products, accumulated in fp64.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * cpu_baseline / verification leg may load this library. It shares no code,
 * header or constant with the GPU library, and the GPU library never calls it.
 *
 * What it computes (the plain definitions on the pages, nothing else):
 *
 *   GEMM  C[i][j] = sum over k = 0 .. K-1 of A[i][k] * B[k][j]
 *         A is M x K, B is K x N, C is M x N, all row-major.
 *         ("Matrix Operations", docs.vulkan.org ML-inference tutorial, section
 *          "Matrix-Matrix Multiplication (GEMM)", the defining sum; the same sum
 *          in "CUDA Programming (6): Shared Memory and Matrix Multiplication
 *          Optimization" section 3.1 and in "GPU Matrix Multiplication: Tiling
 *          and Shared Memory" section 1, display equation.)
 *
 *   GEMV  y[i] = sum over j = 0 .. N-1 of A[i][j] * x[j]
 *         A is M x N row-major, x has N entries, y has M entries.
 *         ("Matrix Operations", section "Matrix-Vector Multiplication".)
 *
 * Arithmetic. Every input is an fp32 value widened to fp64. The product of two
 * fp32 values has at most 48 significant bits, so it is exact in fp64; only the
 * additions round (round-to-nearest-even). Each output is summed in ascending
 * index order (k for GEMM, j for GEMV), the order in which the defining sum is
 * written. Beside each sum the oracle also returns the sum of the absolute values
 * of the same products, S = sum |A[i][k] * B[k][j]|, which scales the tolerance
 * a floating-point result is held to.
 *
 * Loop order. For GEMM the j loop sits inside the k loop so that B is read along
 * its rows. That swaps two loops over independent outputs; every output still
 * receives exactly the additions of the defining sum, in ascending k, so the
 * result is the same as that of the textbook i-j-k loop nest, bit for bit.
 *
 * Threads. Rows are split into contiguous blocks, one per thread. A row's sums do
 * not depend on the split, so the results are identical for every thread count.
 *
 * Build: gcc -O2, no -ffast-math, -ffp-contract=off (nothing may be reassociated).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_THREAD_FAIL 2

/* ---------------------------------------------------------------- GEMM --- */

struct gemm_job {
    int64_t N, K;
    const float *A;
    int64_t lda;
    const float *B;
    int64_t ldb;
    const int64_t *rows; /* NULL: output row r is matrix row r */
    double *C;           /* nrows x N, row stride ldo */
    double *S;           /* same shape as C, or NULL */
    int64_t ldo;
    int64_t r0, r1;      /* this job's output rows [r0, r1) */
};

static void gemm_rows(const struct gemm_job *jb)
{
    for (int64_t r = jb->r0; r < jb->r1; ++r) {
        const int64_t i = jb->rows ? jb->rows[r] : r;
        double *c = jb->C + r * jb->ldo;
        double *s = jb->S ? jb->S + r * jb->ldo : NULL;
        for (int64_t j = 0; j < jb->N; ++j) {
            c[j] = 0.0;
            if (s) s[j] = 0.0;
        }
        for (int64_t k = 0; k < jb->K; ++k) {
            const double a = (double)jb->A[i * jb->lda + k];
            const float *brow = jb->B + k * jb->ldb;
            for (int64_t j = 0; j < jb->N; ++j) {
                const double p = a * (double)brow[j];
                c[j] += p;
                if (s) s[j] += fabs(p);
            }
        }
    }
}

static void *gemm_thread(void *arg)
{
    gemm_rows((const struct gemm_job *)arg);
    return NULL;
}

/*
 * oracle_gemm_f64: for each requested row i of C, writes the fp64 sums
 * C[i][j] (and S[i][j] if S is not NULL) for all j in [0, N).
 *   rows == NULL: nrows must equal M and output row r is C's row r.
 *   rows != NULL: output row r is C's row rows[r]; each rows[r] lies in [0, M).
 * Output arrays are nrows x N with row stride ldo >= N.
 * K == 0 gives all-zero sums (an empty sum), as the pages' kernels write 0.
 */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const float *A, int64_t lda, const float *B, int64_t ldb,
                    const int64_t *rows, int64_t nrows,
                    double *C, double *S, int64_t ldo, int threads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || lda < (K > 1 ? K : 1) ||
        ldb < (N > 1 ? N : 1) || ldo < (N > 1 ? N : 1))
        return ORACLE_BAD_ARG;
    if (!rows && nrows != M) return ORACLE_BAD_ARG;
    if (nrows == 0 || N == 0) return ORACLE_OK;
    if (!C || (K > 0 && (!A || !B))) return ORACLE_BAD_ARG;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= M) return ORACLE_BAD_ARG;
    if (threads < 1) threads = 1;
    if (threads > nrows) threads = (int)nrows;

    struct gemm_job *jobs = calloc((size_t)threads, sizeof *jobs);
    pthread_t *tid = calloc((size_t)threads, sizeof *tid);
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return ORACLE_THREAD_FAIL;
    }
    for (int t = 0; t < threads; ++t) {
        struct gemm_job jb = {N, K, A, lda, B, ldb, rows, C, S, ldo,
                              nrows * t / threads, nrows * (t + 1) / threads};
        jobs[t] = jb;
    }
    int started = 0, rc = ORACLE_OK;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, gemm_thread, &jobs[t]) != 0) {
            rc = ORACLE_THREAD_FAIL;
            break;
        }
        started = t;
    }
    if (rc == ORACLE_OK) gemm_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
    return rc;
}

/* ---------------------------------------------------------------- GEMV --- */

struct gemv_job {
    int64_t N;
    const float *A;
    int64_t lda;
    const float *x;
    double *y, *s;
    int64_t r0, r1;
};

static void gemv_rows(const struct gemv_job *jb)
{
    for (int64_t i = jb->r0; i < jb->r1; ++i) {
        const float *arow = jb->A + i * jb->lda;
        double acc = 0.0, mag = 0.0;
        for (int64_t j = 0; j < jb->N; ++j) {
            const double p = (double)arow[j] * (double)jb->x[j];
            acc += p;
            mag += fabs(p);
        }
        jb->y[i] = acc;
        if (jb->s) jb->s[i] = mag;
    }
}

static void *gemv_thread(void *arg)
{
    gemv_rows((const struct gemv_job *)arg);
    return NULL;
}

/*
 * oracle_gemv_f64: y[i] = sum_j A[i][j] * x[j] in fp64 for i in [0, M), and
 * s[i] = sum_j |A[i][j] * x[j]| if s is not NULL. A has row stride lda >= N.
 * N == 0 gives y = 0.
 */
int oracle_gemv_f64(int64_t M, int64_t N, const float *A, int64_t lda,
                    const float *x, double *y, double *s, int threads)
{
    if (M < 0 || N < 0 || lda < (N > 1 ? N : 1)) return ORACLE_BAD_ARG;
    if (M == 0) return ORACLE_OK;
    if (!y || (N > 0 && (!A || !x))) return ORACLE_BAD_ARG;
    if (threads < 1) threads = 1;
    if (threads > M) threads = (int)M;

    struct gemv_job *jobs = calloc((size_t)threads, sizeof *jobs);
    pthread_t *tid = calloc((size_t)threads, sizeof *tid);
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return ORACLE_THREAD_FAIL;
    }
    for (int t = 0; t < threads; ++t) {
        struct gemv_job jb = {N, A, lda, x, y, s, M * t / threads, M * (t + 1) / threads};
        jobs[t] = jb;
    }
    int started = 0, rc = ORACLE_OK;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, gemv_thread, &jobs[t]) != 0) {
            rc = ORACLE_THREAD_FAIL;
            break;
        }
        started = t;
    }
    if (rc == ORACLE_OK) gemv_rows(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
    return rc;
}
