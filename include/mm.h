/*
 * mm.h -- C ABI of libmm: fp32 matrix-matrix and matrix-vector products on one
 * AMD Instinct MI355X (gfx950).
 *
 * Operations (plain definitions; the kernels may sum in any order):
 *
 *   GEMM  C = A x B,  C[i][j] = sum over k in [0, K) of A[i][k] * B[k][j]
 *         A is M x K, B is K x N, C is M x N.
 *         ("Matrix Operations", docs.vulkan.org ML-inference tutorial, section
 *          "Matrix-Matrix Multiplication (GEMM)"; the same sum in "CUDA
 *          Programming (6): Shared Memory and Matrix Multiplication
 *          Optimization", section 3.1, and "GPU Matrix Multiplication: Tiling
 *          and Shared Memory", section 1.)
 *
 *   GEMV  y = A x,    y[i] = sum over j in [0, N) of A[i][j] * x[j]
 *         A is M x N, x has N entries, y has M entries.
 *         ("Matrix Operations", section "Matrix-Vector Multiplication".)
 *
 *   CONV  2-D convolution through the GEMM (mm_conv2d_f32 below).
 *
 * Conventions shared by every entry point:
 *   - Layout: row-major. Element (i, k) of A lives at A[i * lda + k], (k, j) of B
 *     at B[k * ldb + j], (i, j) of C at C[i * ldc + j]. The pages lay matrices out
 *     the same way with packed rows; the leading dimensions generalise that.
 *   - Memory: every pointer is device memory owned by the caller (hipMalloc or a
 *     torch tensor on the GPU), 4-byte aligned, and must stay valid until the
 *     work enqueued on `stream` has finished. Inputs are only read; outputs are
 *     only written. Outputs must not overlap inputs (undefined, not checked).
 *     Wider alignment (16 bytes, leading dimensions that are multiples of 4) lets
 *     the kernels use 16-byte loads; it is never required.
 *   - Output: only the logical output elements are written; bytes in
 *     leading-dimension gaps and beyond are left untouched. The output is
 *     overwritten: there is no scaling of, or accumulation into, its old value.
 *     Each element is stored once, except where mm_gemm_f32 splits K in two
 *     halves (below): it then zeroes C and adds the halves into it with device
 *     atomics, so C must be ordinary device memory (not host or managed memory).
 *   - Stream: a hipStream_t passed as void*; NULL means the default stream. Calls
 *     only enqueue work and return; they never synchronise and never allocate.
 *     Errors raised by the device while the work runs surface at the caller's
 *     next synchronisation of that stream.
 *   - Threads: the library keeps no mutable global state (except the per-device
 *     address of mm_gemm_f32_ws_static's scratch, looked up once under a lock); calls
 *     from several host threads, on any streams, are safe (mm_gemm_f32_ws_static:
 *     see there).
 *   - Return value: an mm_status. Arguments are checked on the host before any
 *     HIP call; an invalid call enqueues nothing.
 */
#ifndef MM_H
#define MM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mm_status {
    MM_OK = 0,
    MM_ERR_INVALID_ARG = 1, /* bad size, leading dimension, pointer or config index */
    MM_ERR_NO_DEVICE = 2,   /* no usable HIP device in this process */
    MM_ERR_LAUNCH = 3       /* the HIP runtime refused the launch (see mm_last_error) */
} mm_status;

/*
 * mm_gemm_f32: C = A x B in fp32 (fp32 products, fp32 accumulation on the
 * matrix cores).
 *   M, N, K   sizes, 0 <= M, N, K <= 2^31 - 1.
 *   A, lda    M x K, lda >= max(1, K). May be NULL when M == 0 or K == 0.
 *   B, ldb    K x N, ldb >= max(1, N). May be NULL when K == 0 or N == 0.
 *   C, ldc    M x N, ldc >= max(1, N). May be NULL when M == 0 or N == 0.
 *   stream    hipStream_t or NULL.
 * M == 0 or N == 0: nothing is enqueued and MM_OK is returned.
 * K == 0: C is filled with zeros (the empty sum; the pages' kernels write a
 * zero-initialised sum when the k loop does not run).
 * Products whose C has 128 to 256 tiles of 64 x 64 with N >= 64, N % 4 == 0,
 * K % 32 == 0 and K >= 4096 (K >= 2048 at 128 tiles) run as two K halves, which
 * doubles the workgroups: C is zeroed, then each half adds its tiles into C
 * atomically. With two partial sums the result does not depend on their order, so
 * it is deterministic; it may differ in the last bits from the unsplit kernel's.
 * Errors: MM_ERR_INVALID_ARG (negative or too-large size, leading dimension too
 * small, NULL pointer with a non-empty extent, byte offset overflow),
 * MM_ERR_NO_DEVICE, MM_ERR_LAUNCH.
 */
int mm_gemm_f32(int64_t M, int64_t N, int64_t K,
                const float *A, int64_t lda,
                const float *B, int64_t ldb,
                float *C, int64_t ldc, void *stream);

/*
 * mm_gemv_f32: y = A x in fp32 (fp32 products and accumulation).
 *   M, N      sizes, 0 <= M, N <= 2^31 - 1.
 *   A         M x N with packed rows (leading dimension N). May be NULL when
 *             M == 0 or N == 0.
 *   x         N entries, contiguous. May be NULL when N == 0.
 *   y         M entries, contiguous. May be NULL when M == 0.
 *   stream    hipStream_t or NULL.
 * M == 0: nothing is enqueued. N == 0: y is filled with zeros.
 * Errors: as for mm_gemm_f32.
 */
int mm_gemv_f32(int64_t M, int64_t N, const float *A, const float *x, float *y,
                void *stream);

/*
 * mm_gemv_t_f32: y = A^T x in fp32, y[j] = sum over i in [0, M) of A[i][j] * x[i]:
 * the GEMV of the same row-major matrix applied to its transpose (a column of A
 * dotted with x per output).
 *   M, N      sizes, 0 <= M, N <= 2^31 - 1.
 *   A         M x N with packed rows (leading dimension N).
 *   x         M entries, contiguous. May be NULL when M == 0.
 *   y         N entries, contiguous. May be NULL when N == 0.
 * N == 0: nothing is enqueued. M == 0: y is filled with zeros. The summation order
 * is fixed, so results are deterministic. Errors: as for mm_gemv_f32.
 */
int mm_gemv_t_f32(int64_t M, int64_t N, const float *A, const float *x, float *y,
                  void *stream);

/*
 * mm_gemv_t_f32_ws: y = A^T x as mm_gemv_t_f32, with a caller-owned device workspace
 * that lets it read A along whole rows (1 KB of a row per wave instruction, as the
 * GEMV does): each workgroup sums a 256-column strip over a block of rows into the
 * workspace, and a second launch on the same stream adds the row blocks' partial sums
 * per column in row-block order, so results are deterministic (they may differ from
 * mm_gemv_t_f32's in the last bits: the summation order differs).
 *   workspace        device memory of at least mm_gemv_t_f32_workspace_bytes(M, N)
 *                    bytes, 16-byte aligned; its contents on entry do not matter and
 *                    are overwritten. May be NULL when that size is 0.
 *   workspace_bytes  its size in bytes.
 * Calls that share a workspace must not run at the same time (e.g. keep them on one
 * stream). Shapes for which the row blocks gain nothing (fewer than 512 rows, rows not
 * 16-byte aligned) run the kernel of mm_gemv_t_f32 and leave the workspace untouched.
 * Other arguments and errors: as for mm_gemv_t_f32; MM_ERR_INVALID_ARG also for a
 * workspace that is missing, too small or misaligned.
 *
 * mm_gemv_t_f32_workspace_bytes: bytes of workspace mm_gemv_t_f32_ws needs for (M, N)
 * (0 when it needs none), or -1 for a negative or too large size.
 */
int64_t mm_gemv_t_f32_workspace_bytes(int64_t M, int64_t N);
int mm_gemv_t_f32_ws(int64_t M, int64_t N, const float *A, const float *x, float *y,
                     void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Tile configurations of the GEMM. mm_gemm_f32 picks one per shape; the calls
 * below expose the choice and let a caller (tests, tuning) run a given one.
 *   mm_gemm_f32_num_configs: number of configurations, >= 1.
 *   mm_gemm_f32_config_name: static NUL-terminated description of config `cfg`
 *     (e.g. "256x256x32 w128x64"), or NULL if cfg is out of range.
 *   mm_gemm_f32_select: the config mm_gemm_f32 would use for (M, N, K) (for the
 *     shapes it runs as two K halves, the config of the halves' tile).
 *   mm_gemm_f32_config: mm_gemm_f32 forced to config `cfg`; same arguments and
 *     errors, plus MM_ERR_INVALID_ARG for cfg out of range. Every config gives a
 *     correct product for every shape.
 */
int mm_gemm_f32_num_configs(void);
const char *mm_gemm_f32_config_name(int cfg);
int mm_gemm_f32_select(int64_t M, int64_t N, int64_t K);
int mm_gemm_f32_config(int cfg, int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda,
                       const float *B, int64_t ldb,
                       float *C, int64_t ldc, void *stream);

/*
 * mm_gemm_f32_batched: `batch` independent fp32 GEMMs C_b = A_b x B_b in one launch
 * ("Matrix Operations", "Performance Considerations": processing several matrix
 * products in parallel fills the GPU better). Problem b (0 <= b < batch) uses
 * A + b * stride_a, B + b * stride_b and C + b * stride_c (strides in elements,
 * >= 0; a stride of 0 shares that operand between problems). Each problem has the
 * sizes and leading dimensions of mm_gemm_f32 and the same semantics.
 *   batch     0 <= batch <= 65535; batch == 0 enqueues nothing (pointers may then
 *             be NULL; sizes and leading dimensions are still checked).
 * The C_b must not overlap each other or any input (undefined, not checked).
 * Errors: as for mm_gemm_f32, plus MM_ERR_INVALID_ARG for a negative stride, a
 * batch out of range, or batch offsets that overflow.
 */
int mm_gemm_f32_batched(int64_t batch, int64_t M, int64_t N, int64_t K,
                        const float *A, int64_t lda, int64_t stride_a,
                        const float *B, int64_t ldb, int64_t stride_b,
                        float *C, int64_t ldc, int64_t stride_c, void *stream);

/*
 * mm_gemm_f32_ws: C = A x B as mm_gemm_f32, with a caller-owned device workspace that
 * lets products with few output tiles (the fully-connected layer on a batch of 25 to
 * 256 input vectors, "Matrix Operations", "Performance Considerations": batch
 * processing) split K across workgroups: each of `chunks` (2 to 8) K ranges is
 * multiplied into its own M x N slice of the
 * workspace, and a second launch on the same stream adds the slices in chunk order
 * into C, so results are deterministic (they may differ from mm_gemm_f32's in the last
 * bits: the summation order differs).
 *   workspace        device memory of at least mm_gemm_f32_workspace_bytes(M, N, K)
 *                    bytes, 16-byte aligned; its contents on entry do not matter and
 *                    are overwritten. May be NULL when that size is 0. It must not
 *                    overlap A, B or C.
 *   workspace_bytes  its size in bytes.
 * Calls that share a workspace must not run at the same time (e.g. keep them on one
 * stream). With N % 4 != 0, B is first copied into the workspace with its rows padded
 * to a multiple of 4 floats. Shapes the split does not serve (N <= 24, N % 4 != 0 with
 * N <= 32, N > 256, K < 2048, more than 256 output tiles of 64 x 64, K without a whole
 * number of 16-deep steps per chunk) run mm_gemm_f32's kernels and leave the workspace
 * untouched. Other arguments and errors: as for mm_gemm_f32;
 * MM_ERR_INVALID_ARG also for a workspace that is missing, too small or misaligned.
 *
 * mm_gemm_f32_workspace_bytes: bytes of workspace mm_gemm_f32_ws needs for (M, N, K)
 * (0 when it needs none), or -1 for a negative or too large size.
 */
int64_t mm_gemm_f32_workspace_bytes(int64_t M, int64_t N, int64_t K);
int mm_gemm_f32_ws(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                   const float *B, int64_t ldb, float *C, int64_t ldc,
                   void *workspace, int64_t workspace_bytes, void *stream);

/*
 * mm_gemm_f32_ws_static: mm_gemm_f32_ws without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The K split runs in the library's own static device
 * scratch of MM_STATIC_SCRATCH_BYTES, one per GPU, held until the process ends; the call
 * itself allocates nothing. Results are bit-identical to mm_gemm_f32_ws's for the same
 * arguments (the same kernels in the same order).
 *   Arguments, layout, ownership and zero-size cases as for mm_gemm_f32. `stream` must
 *   belong to the current device (NULL: the current device's default stream).
 * Shapes that mm_gemm_f32_ws serves without its workspace (mm_gemm_f32_workspace_bytes is
 * 0) run mm_gemm_f32's kernels and touch no scratch.
 * Every call on one GPU shares that GPU's scratch, and it keeps the last call's contents
 * (each call overwrites what it reads): calls on one GPU that may overlap in time (on
 * different streams, or from several host threads without ordering) race and give wrong
 * results. Keep them on one stream.
 * Errors: as for mm_gemm_f32, plus MM_ERR_INVALID_ARG when the split needs more than
 * MM_STATIC_SCRATCH_BYTES (mm_gemm_f32_workspace_bytes above it; checked before any HIP
 * call), a stream of another device than the current one, or a device index above 63.
 */
#define MM_STATIC_SCRATCH_BYTES (16 * 1024 * 1024)
int mm_gemm_f32_ws_static(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                          const float *B, int64_t ldb, float *C, int64_t ldc, void *stream);

/*
 * mm_gemm_bf16 / mm_gemm_f16: C = A x B with 16-bit inputs and fp32 accumulation
 * and output ("Matrix Operations", "Performance Considerations": half precision
 * and matrix engines). A and B hold bf16 (mm_gemm_bf16) or IEEE binary16
 * (mm_gemm_f16) bit patterns, 2 bytes per element, row-major with leading
 * dimensions counted in elements; C is fp32. Every product of two 16-bit values is
 * exact in fp32, so C is the fp32 GEMM of the inputs' exact values, summed on the
 * matrix cores in fp32.
 * Arguments, layout, ownership, stream, zero-size cases and errors as for
 * mm_gemm_f32, except: A and B must be 2-byte aligned. Shapes with K >= 32 and with
 * N >= 64 or N % 8 == 0 take the pipeline that loads panels straight into LDS, at any
 * 2-byte alignment and leading dimension; others take register-staged tiles.
 *   mm_gemm_h16_num_configs / mm_gemm_h16_config_name / mm_gemm_h16_select: the
 *     tile configurations of these two calls, as for the fp32 GEMM.
 *   mm_gemm_bf16_config / mm_gemm_f16_config: the calls with config `cfg` forced.
 */
int mm_gemm_bf16(int64_t M, int64_t N, int64_t K,
                 const uint16_t *A, int64_t lda,
                 const uint16_t *B, int64_t ldb,
                 float *C, int64_t ldc, void *stream);
int mm_gemm_f16(int64_t M, int64_t N, int64_t K,
                const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb,
                float *C, int64_t ldc, void *stream);
int mm_gemm_h16_num_configs(void);
const char *mm_gemm_h16_config_name(int cfg);
int mm_gemm_h16_select(int64_t M, int64_t N, int64_t K);
int mm_gemm_bf16_config(int cfg, int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb,
                        float *C, int64_t ldc, void *stream);
int mm_gemm_f16_config(int cfg, int64_t M, int64_t N, int64_t K,
                       const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb,
                       float *C, int64_t ldc, void *stream);

/*
 * mm_conv2d_f32: 2-D convolution (cross-correlation, as in neural networks) in fp32,
 * lowered to the GEMM by im2col ("Matrix Operations", Introduction: a convolutional
 * layer's core recast as a matrix product; "GPU Matrix Multiplication: Tiling and
 * Shared Memory", closing preview of im2col). The pages give no formula; the one
 * computed is the usual definition
 *
 *   y[n][k][p][q] = sum over c < C, r < R, s < S of
 *                   w[k][c][r][s] * x[n][c][p*sh + r*dh - ph][q*sw + s*dw - pw]
 *
 * with x read as 0 at rows outside [0, H) and columns outside [0, W) (zero padding),
 * and the output size P = (H + 2 ph - dh (R - 1) - 1) / sh + 1, Q = (W + 2 pw -
 * dw (S - 1) - 1) / sw + 1 (integer division; see mm_conv2d_out_dim).
 *   N, C, H, W     images, channels, input height, width; >= 0.
 *   K, R, S        filters, filter height, width; K >= 0, R, S >= 1.
 *   sh, sw         strides >= 1; ph, pw: zero padding >= 0; dh, dw: dilation >= 1.
 *   x              N x C x H x W, packed (NCHW). May be NULL if it has no elements.
 *   w              K x C x R x S, packed. May be NULL if it has no elements.
 *   y              N x K x P x Q, packed, written. May be NULL if it has no elements.
 * Products are fp32, accumulated in fp32 on the matrix cores in an order of the
 * kernel's choosing; the im2col matrix is gathered on the fly, never stored, so no
 * workspace is used. C == 0, H == 0 or W == 0 (x has no elements; padding may still give
 * P, Q >= 1, and every tap then reads the padding): y is filled with zeros. No output
 * elements: nothing is enqueued.
 * Errors: MM_ERR_INVALID_ARG for a negative size, a stride, dilation or filter size
 * below 1, negative padding, a filter that does not fit the padded input (P or Q
 * would be below 1), a NULL or unaligned pointer that is used, or sizes beyond the
 * limits: one image (C H W) and the padded plane (H + 2 ph)(W + 2 pw) at most
 * 2^30 - 1 elements; C R S and P Q at most 2^31 - 1; H + 2 ph, W + 2 pw, dh (R - 1),
 * dw (S - 1) below 2^29. Other errors as for mm_gemm_f32.
 */
int mm_conv2d_f32(int64_t N, int64_t C, int64_t H, int64_t W,
                  int64_t K, int64_t R, int64_t S,
                  int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                  const float *x, const float *w, float *y, void *stream);

/*
 * mm_conv2d_out_dim: the output extent along one axis, (in + 2 pad - dil (filter - 1)
 * - 1) / stride + 1, or -1 if an argument is out of range (in < 0, filter < 1,
 * stride < 1, pad < 0, dil < 1, or any above 2^29) or the dilated filter is longer
 * than the padded input.
 */
int64_t mm_conv2d_out_dim(int64_t in, int64_t filter, int64_t stride, int64_t pad,
                          int64_t dil);

/*
 * Tile configurations of the convolution (matrix-core tiles with an im2col gather in
 * place of the B loads: the GEMM's register-staged tiles, and tiles whose gather moves
 * x straight into the LDS), as for the GEMM:
 *   mm_conv2d_f32_num_configs, mm_conv2d_f32_config_name(cfg): count and names;
 *   mm_conv2d_f32_select: the config mm_conv2d_f32 uses for the geometry (same
 *     arguments without the pointers and stream), or -1 if it is invalid;
 *   mm_conv2d_f32_config: mm_conv2d_f32 forced to config `cfg` (MM_ERR_INVALID_ARG
 *     if out of range). Every config is correct for every shape.
 */
int mm_conv2d_f32_num_configs(void);
const char *mm_conv2d_f32_config_name(int cfg);
int mm_conv2d_f32_select(int64_t N, int64_t C, int64_t H, int64_t W,
                         int64_t K, int64_t R, int64_t S,
                         int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw);
int mm_conv2d_f32_config(int cfg, int64_t N, int64_t C, int64_t H, int64_t W,
                         int64_t K, int64_t R, int64_t S,
                         int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                         const float *x, const float *w, float *y, void *stream);

/* mm_status_string: static text for a status code (never NULL). */
const char *mm_status_string(int status);

/* mm_last_error: static or thread-local text describing the last failure seen by
 * this host thread (the HIP error string for MM_ERR_LAUNCH), or "" if none. */
const char *mm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MM_H */
