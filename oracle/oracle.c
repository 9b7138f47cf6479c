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
 *   CONV  the 2-D convolution of a convolutional layer, from its usual definition
 *         (see oracle_conv2d_f64 below; the pages only say it can be recast as a
 *         matrix product).
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

/* ------------------------------------------------------------- convolution --- */

/*
 * oracle_conv2d_f64: the 2-D convolution (cross-correlation) that a convolutional
 * layer computes, written out from its definition. The pages only say that the core
 * of a convolutional layer can be recast as a matrix product ("Matrix Operations",
 * Introduction; "GPU Matrix Multiplication: Tiling and Shared Memory", closing
 * preview of im2col); the definition used is the usual one:
 *
 *   y[n][k][p][q] = sum over c < C, r < R, s < S of
 *                   x[n][c][p*sh + r*dh - ph][q*sw + s*dw - pw] * w[k][c][r][s]
 *
 * with x taken as 0 outside 0 <= h < H, 0 <= w < W (a padded tap still multiplies that
 * zero by its filter value, as the matrix the layer is recast as holds it), and
 * P = (H + 2 ph - dh (R - 1) - 1)
 * / sh + 1, Q likewise (integer division; P, Q >= 1 here). Layouts, all packed:
 * x is N x C x H x W, w is K x C x R x S, y and s_out are N x K x P x Q. Each output
 * is summed in fp64 in ascending (c, r, s) order; s_out gets the sum of |products|.
 */
struct conv_job {
    int64_t C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, P, Q;
    const float *x, *w;
    double *y, *s;
    int64_t nk0, nk1; /* this job's (image, filter) pairs, n * K + k in [nk0, nk1) */
};

static void conv_pairs(const struct conv_job *jb)
{
    for (int64_t nk = jb->nk0; nk < jb->nk1; ++nk) {
        const int64_t n = nk / jb->K, k = nk % jb->K;
        const float *xn = jb->x + n * jb->C * jb->H * jb->W;
        const float *wk = jb->w + k * jb->C * jb->R * jb->S;
        double *yo = jb->y + nk * jb->P * jb->Q;
        double *so = jb->s ? jb->s + nk * jb->P * jb->Q : NULL;
        for (int64_t p = 0; p < jb->P; ++p)
            for (int64_t q = 0; q < jb->Q; ++q) {
                double acc = 0.0; /* the output, in fp64 */
                double mag = 0.0; /* sum of |products| */
                for (int64_t c = 0; c < jb->C; ++c)
                    for (int64_t r = 0; r < jb->R; ++r)
                        for (int64_t s = 0; s < jb->S; ++s) {
                            const int64_t h = p * jb->sh + r * jb->dh - jb->ph;
                            const int64_t v = q * jb->sw + s * jb->dw - jb->pw;
                            /* a tap in the padding reads a zero of the padded input (an
                             * explicit zero of the matrix the convolution is recast as);
                             * with finite filters it adds nothing, with an infinite or
                             * NaN filter value the product is NaN (IEEE 0 * inf) */
                            const int inside = h >= 0 && h < jb->H && v >= 0 && v < jb->W;
                            const double xv = inside ? (double)xn[(c * jb->H + h) * jb->W + v] : 0.0;
                            const double prod = xv * (double)wk[(c * jb->R + r) * jb->S + s];
                            acc += prod;
                            mag += fabs(prod);
                        }
                yo[p * jb->Q + q] = acc;
                if (so) so[p * jb->Q + q] = mag;
            }
    }
}

static void *conv_thread(void *arg)
{
    conv_pairs((const struct conv_job *)arg);
    return NULL;
}

int oracle_conv2d_f64(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R,
                      int64_t S, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                      int64_t dw, const float *x, const float *w, double *y, double *s,
                      int threads)
{
    if (N < 0 || C < 0 || H < 0 || W < 0 || K < 0 || R < 1 || S < 1 || sh < 1 || sw < 1 ||
        ph < 0 || pw < 0 || dh < 1 || dw < 1)
        return ORACLE_BAD_ARG;
    const int64_t P = (H + 2 * ph - dh * (R - 1) - 1) / sh + 1;
    const int64_t Q = (W + 2 * pw - dw * (S - 1) - 1) / sw + 1;
    if (H + 2 * ph - dh * (R - 1) - 1 < 0 || W + 2 * pw - dw * (S - 1) - 1 < 0) return ORACLE_BAD_ARG;
    const int64_t pairs = N * K;
    if (pairs == 0 || P * Q == 0) return ORACLE_OK;
    /* x may be absent when it has no elements (C, H or W is 0): every tap then reads
     * the zero padding */
    if (!y || (C > 0 && !w) || (C * H * W > 0 && !x)) return ORACLE_BAD_ARG;
    if (threads < 1) threads = 1;
    if (threads > pairs) threads = (int)pairs;

    struct conv_job *jobs = calloc((size_t)threads, sizeof *jobs);
    pthread_t *tid = calloc((size_t)threads, sizeof *tid);
    if (!jobs || !tid) {
        free(jobs);
        free(tid);
        return ORACLE_THREAD_FAIL;
    }
    for (int t = 0; t < threads; ++t) {
        struct conv_job jb = {C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, P, Q, x, w, y, s,
                              pairs * t / threads, pairs * (t + 1) / threads};
        jobs[t] = jb;
    }
    int started = 0, rc = ORACLE_OK;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, conv_thread, &jobs[t]) != 0) {
            rc = ORACLE_THREAD_FAIL;
            break;
        }
        started = t;
    }
    if (rc == ORACLE_OK) conv_pairs(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
    return rc;
}
