// mm_api.hip -- the C ABI of libmm (declared in include/mm.h): host-side argument
// checks, shape -> kernel configuration, launch, and status codes.
#include <stdint.h>
#include <stdio.h>

#include "mm.h"
#include "mm_internal.h"

namespace {

thread_local char g_last_error[256] = "";

void set_error(const char *what, hipError_t e)
{
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

void set_error_text(const char *what)
{
    snprintf(g_last_error, sizeof g_last_error, "%s", what);
}

int from_hip(const char *what, hipError_t e)
{
    if (e == hipSuccess) return MM_OK;
    set_error(what, e);
    if (e == hipErrorNoDevice || e == hipErrorInsufficientDriver) return MM_ERR_NO_DEVICE;
    return MM_ERR_LAUNCH;
}

int invalid(const char *why)
{
    set_error_text(why);
    return MM_ERR_INVALID_ARG;
}

constexpr int64_t kMaxDim = 0x7fffffff;

// Byte extent of a rows x cols matrix with row stride ld is
// 4 * ((rows - 1) * ld + cols); true if that fits in int64 (rows, cols >= 1).
bool extent_fits(int64_t rows, int64_t cols, int64_t ld)
{
    const int64_t limit = INT64_MAX / 4;
    if (ld > 0 && rows - 1 > (limit - cols) / ld) return false;
    return true;
}

int check_gemm_dims(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc)
{
    if (M < 0 || N < 0 || K < 0) return invalid("negative size");
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return invalid("size above 2^31 - 1");
    if (lda < (K > 1 ? K : 1)) return invalid("lda < max(1, K)");
    if (ldb < (N > 1 ? N : 1)) return invalid("ldb < max(1, N)");
    if (ldc < (N > 1 ? N : 1)) return invalid("ldc < max(1, N)");
    return MM_OK;
}

// elem: bytes per element of A and B (4 for fp32, 2 for the 16-bit formats).
int check_gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B,
               int64_t ldb, const float *C, int64_t ldc, int elem = 4)
{
    const int d = check_gemm_dims(M, N, K, lda, ldb, ldc);
    if (d != MM_OK) return d;
    if (M > 0 && K > 0 && !A) return invalid("A is NULL");
    if (K > 0 && N > 0 && !B) return invalid("B is NULL");
    if (M > 0 && N > 0 && !C) return invalid("C is NULL");
    if ((uintptr_t)A % elem || (uintptr_t)B % elem || (uintptr_t)C % 4)
        return invalid("pointer not aligned to its element size");
    if (M > 0 && K > 0 && !extent_fits(M, K, lda)) return invalid("A extent overflows");
    if (K > 0 && N > 0 && !extent_fits(K, N, ldb)) return invalid("B extent overflows");
    if (M > 0 && N > 0 && !extent_fits(M, N, ldc)) return invalid("C extent overflows");
    return MM_OK;
}

int run_gemm(int cfg, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
             int64_t ldb, float *C, int64_t ldc, void *stream)
{
    const int st = check_gemm(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != MM_OK) return st;
    if (M == 0 || N == 0) return MM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return from_hip("zero fill launch", mm::zero_fill_launch(C, M, N, ldc, s));
    mm::GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    if (cfg < 0) cfg = mm::gemm_select_config(M, N, K);
    return from_hip("gemm launch", mm::gemm_launch(cfg, a, s));
}

// Batched: every problem's extent and its offset b * stride must fit, strides >= 0.
int run_gemm_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                     int64_t sa, const float *B, int64_t ldb, int64_t sb, float *C, int64_t ldc,
                     int64_t sc, void *stream)
{
    if (batch < 0) return invalid("negative batch");
    if (batch > 65535) return invalid("batch above 65535");
    if (sa < 0 || sb < 0 || sc < 0) return invalid("negative batch stride");
    if (batch == 0) return check_gemm_dims(M, N, K, lda, ldb, ldc);  // pointers may be NULL
    const int st = check_gemm(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != MM_OK) return st;
    if (M == 0 || N == 0) return MM_OK;
    const int64_t limit = INT64_MAX / 8;
    if ((batch - 1) > 0 && (sa > limit / (batch - 1) || sb > limit / (batch - 1) ||
                            sc > limit / (batch - 1)))
        return invalid("batch offset overflows");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) {
        for (int64_t b = 0; b < batch; ++b) {
            const int r = from_hip("zero fill launch", mm::zero_fill_launch(C + b * sc, M, N, ldc, s));
            if (r != MM_OK) return r;
        }
        return MM_OK;
    }
    mm::GemmArgs a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.K = (int)K;
    a.batch = (int)batch;
    a.sa = sa;
    a.sb = sb;
    a.sc = sc;
    return from_hip("batched gemm launch",
                    mm::gemm_launch(mm::gemm_select_config(M, N, K, batch), a, s));
}

int run_gemm16(int cfg, bool bf16, int64_t M, int64_t N, int64_t K, const uint16_t *A,
               int64_t lda, const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    const int st = check_gemm(M, N, K, A, lda, B, ldb, C, ldc, 2);
    if (st != MM_OK) return st;
    if (M == 0 || N == 0) return MM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return from_hip("zero fill launch", mm::zero_fill_launch(C, M, N, ldc, s));
    if (cfg < 0) cfg = mm::gemm16_select_config(M, N, K);
    return from_hip("gemm16 launch", mm::gemm16_launch(cfg, bf16, A, lda, B, ldb, C, ldc, (int)M,
                                                       (int)N, (int)K, s));
}

}  // namespace

extern "C" {

int mm_gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                int64_t ldb, float *C, int64_t ldc, void *stream)
{
    return run_gemm(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int mm_gemm_f32_config(int cfg, int64_t M, int64_t N, int64_t K, const float *A, int64_t lda,
                       const float *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    if (cfg < 0 || cfg >= mm::gemm_num_configs()) return invalid("config index out of range");
    return run_gemm(cfg, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int mm_gemm_f32_num_configs(void) { return mm::gemm_num_configs(); }

const char *mm_gemm_f32_config_name(int cfg) { return mm::gemm_config_name(cfg); }

int mm_gemm_f32_select(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    return mm::gemm_select_config(M, N, K);
}

int mm_gemm_f32_batched(int64_t batch, int64_t M, int64_t N, int64_t K, const float *A,
                        int64_t lda, int64_t stride_a, const float *B, int64_t ldb,
                        int64_t stride_b, float *C, int64_t ldc, int64_t stride_c, void *stream)
{
    return run_gemm_batched(batch, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c,
                            stream);
}

int mm_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                 const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    return run_gemm16(-1, true, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int mm_gemm_f16(int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    return run_gemm16(-1, false, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int mm_gemm_bf16_config(int cfg, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                        const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    if (cfg < 0 || cfg >= mm::gemm16_num_configs()) return invalid("config index out of range");
    return run_gemm16(cfg, true, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int mm_gemm_f16_config(int cfg, int64_t M, int64_t N, int64_t K, const uint16_t *A, int64_t lda,
                       const uint16_t *B, int64_t ldb, float *C, int64_t ldc, void *stream)
{
    if (cfg < 0 || cfg >= mm::gemm16_num_configs()) return invalid("config index out of range");
    return run_gemm16(cfg, false, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int mm_gemm_h16_num_configs(void) { return mm::gemm16_num_configs(); }

const char *mm_gemm_h16_config_name(int cfg) { return mm::gemm16_config_name(cfg); }

int mm_gemm_h16_select(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return 0;
    return mm::gemm16_select_config(M, N, K);
}

int mm_gemv_f32(int64_t M, int64_t N, const float *A, const float *x, float *y, void *stream)
{
    if (M < 0 || N < 0) return invalid("negative size");
    if (M > kMaxDim || N > kMaxDim) return invalid("size above 2^31 - 1");
    if (M > 0 && N > 0 && !A) return invalid("A is NULL");
    if (N > 0 && !x) return invalid("x is NULL");
    if (M > 0 && !y) return invalid("y is NULL");
    if ((uintptr_t)A % 4 || (uintptr_t)x % 4 || (uintptr_t)y % 4)
        return invalid("pointer not aligned to its element size");
    if (M > 0 && N > 0 && !extent_fits(M, N, N)) return invalid("A extent overflows");
    if (M == 0) return MM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (N == 0) return from_hip("zero fill launch", mm::zero_fill_launch(y, 1, M, M, s));
    mm::GemvArgs a;
    a.A = A;
    a.x = x;
    a.y = y;
    a.M = (int)M;
    a.N = (int)N;
    return from_hip("gemv launch", mm::gemv_launch(a, s));
}

int mm_gemv_t_f32(int64_t M, int64_t N, const float *A, const float *x, float *y, void *stream)
{
    if (M < 0 || N < 0) return invalid("negative size");
    if (M > kMaxDim || N > kMaxDim) return invalid("size above 2^31 - 1");
    if (M > 0 && N > 0 && !A) return invalid("A is NULL");
    if (M > 0 && !x) return invalid("x is NULL");
    if (N > 0 && !y) return invalid("y is NULL");
    if ((uintptr_t)A % 4 || (uintptr_t)x % 4 || (uintptr_t)y % 4)
        return invalid("pointer not aligned to its element size");
    if (M > 0 && N > 0 && !extent_fits(M, N, N)) return invalid("A extent overflows");
    if (N == 0) return MM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M == 0) return from_hip("zero fill launch", mm::zero_fill_launch(y, 1, N, N, s));
    mm::GemvArgs a;
    a.A = A;
    a.x = x;
    a.y = y;
    a.M = (int)M;
    a.N = (int)N;
    return from_hip("gemv_t launch", mm::gemv_t_launch(a, s));
}

const char *mm_status_string(int status)
{
    switch (status) {
    case MM_OK: return "ok";
    case MM_ERR_INVALID_ARG: return "invalid argument";
    case MM_ERR_NO_DEVICE: return "no HIP device";
    case MM_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

const char *mm_last_error(void) { return g_last_error; }

}  // extern "C"
