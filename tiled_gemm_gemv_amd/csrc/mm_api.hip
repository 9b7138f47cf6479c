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
    if (cfg < 0 && mm::gemm_split2_ok(M, N, K)) return from_hip("gemm launch", mm::gemm_split2_launch(a, s));
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

constexpr int64_t kConvMaxGeom = int64_t(1) << 29;

// Output extent along one axis, or -1 (arguments as for mm_conv2d_out_dim).
int64_t conv_out_dim(int64_t in, int64_t filter, int64_t stride, int64_t pad, int64_t dil)
{
    if (in < 0 || filter < 1 || stride < 1 || pad < 0 || dil < 1) return -1;
    if (in >= kConvMaxGeom || filter >= kConvMaxGeom || stride >= kConvMaxGeom ||
        pad >= kConvMaxGeom || dil >= kConvMaxGeom)
        return -1;
    const int64_t span = dil * (filter - 1);  // < 2^58
    const int64_t padded = in + 2 * pad;
    if (span >= kConvMaxGeom || padded >= kConvMaxGeom) return -1;
    if (padded - span - 1 < 0) return -1;
    return (padded - span - 1) / stride + 1;
}

// Checks a convolution's arguments and fills `a`. Returns MM_OK, or the error; *work
// is false when there is no output element (nothing to enqueue).
int check_conv(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
               int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
               const float *x, const float *w, const float *y, bool check_pointers,
               mm::ConvArgs &a, bool &work)
{
    work = false;
    if (N < 0 || C < 0 || H < 0 || W < 0 || K < 0) return invalid("negative size");
    if (R < 1 || S < 1) return invalid("filter size below 1");
    if (sh < 1 || sw < 1) return invalid("stride below 1");
    if (ph < 0 || pw < 0) return invalid("negative padding");
    if (dh < 1 || dw < 1) return invalid("dilation below 1");
    const int64_t P = conv_out_dim(H, R, sh, ph, dh), Q = conv_out_dim(W, S, sw, pw, dw);
    if (P < 0 || Q < 0) {
        if (H + 2 * ph >= kConvMaxGeom || W + 2 * pw >= kConvMaxGeom || R >= kConvMaxGeom ||
            S >= kConvMaxGeom || dh >= kConvMaxGeom || dw >= kConvMaxGeom ||
            sh >= kConvMaxGeom || sw >= kConvMaxGeom || dh * (R - 1) >= kConvMaxGeom ||
            dw * (S - 1) >= kConvMaxGeom)
            return invalid("convolution geometry above 2^29");
        return invalid("filter does not fit the padded input");
    }
    if (K > kMaxDim || N > kMaxDim || C > kMaxDim) return invalid("size above 2^31 - 1");
    const int64_t HW = H * W, PQ = P * Q;  // each below 2^58
    const int64_t kMaxImage = (int64_t(1) << 30) - 1;
    if (C > 0 && HW > kMaxImage / C) return invalid("C * H * W above 2^30 - 1");
    // P * Q <= (H + 2 ph)(W + 2 pw), so this also keeps P * Q below 2^30
    if ((H + 2 * ph) * (W + 2 * pw) > kMaxImage) return invalid("padded plane above 2^30 - 1");
    if (C > 0 && R * S > kMaxDim / C) return invalid("C * R * S above 2^31 - 1");
    const int64_t limit = INT64_MAX / 4;
    const int64_t CHW = C * HW, CRS = C * R * S;
    if (N > 0 && CHW > limit / N) return invalid("x extent overflows");
    if (K > 0 && PQ > 0 && N > limit / K / PQ) return invalid("y extent overflows");
    if (check_pointers) {
        const bool has_x = N > 0 && CHW > 0, has_w = K > 0 && CRS > 0, has_y = N > 0 && K > 0;
        if (has_x && !x) return invalid("x is NULL");
        if (has_w && !w) return invalid("w is NULL");
        if (has_y && !y) return invalid("y is NULL");
        if ((uintptr_t)x % 4 || (uintptr_t)w % 4 || (uintptr_t)y % 4)
            return invalid("pointer not aligned to its element size");
    }
    a.N = N;
    a.C = C;
    a.H = H;
    a.W = W;
    a.K = K;
    a.R = R;
    a.S = S;
    a.sh = sh;
    a.sw = sw;
    a.ph = ph;
    a.pw = pw;
    a.dh = dh;
    a.dw = dw;
    a.P = P;
    a.Q = Q;
    a.x = x;
    a.w = w;
    a.y = const_cast<float *>(y);
    work = N > 0 && K > 0;  // P, Q >= 1 here
    return MM_OK;
}

int run_conv(int cfg, int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R,
             int64_t S, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
             const float *x, const float *w, float *y, void *stream)
{
    mm::ConvArgs a;
    bool work;
    const int st = check_conv(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, y, true, a, work);
    if (st != MM_OK || !work) return st;
    return from_hip("conv2d launch", mm::conv_launch(cfg, a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int mm_gemm_f32(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                int64_t ldb, float *C, int64_t ldc, void *stream)
{
    return run_gemm(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int64_t mm_gemm_f32_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return -1;
    if (M == 0 || N == 0 || K == 0) return 0;
    return 4 * mm::gemm_split_ws_floats(M, N, K);
}

int mm_gemm_f32_ws(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                   int64_t ldb, float *C, int64_t ldc, void *workspace, int64_t workspace_bytes, void *stream)
{
    const int64_t need = mm_gemm_f32_workspace_bytes(M, N, K);
    if (need > 0) {
        if (!workspace) return invalid("workspace is NULL");
        if ((uintptr_t)workspace % 16) return invalid("workspace not 16-byte aligned");
        if (workspace_bytes < need) return invalid("workspace smaller than mm_gemm_f32_workspace_bytes");
    }
    if (need <= 0) return run_gemm(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);
    const int st = check_gemm(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != MM_OK) return st;
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
    return from_hip("split gemm launch", mm::gemm_split_launch(a, static_cast<float *>(workspace),
                                                                static_cast<hipStream_t>(stream)));
}

int mm_gemm_f32_ws_static(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                          int64_t ldb, float *C, int64_t ldc, void *stream)
{
    const int64_t need = mm_gemm_f32_workspace_bytes(M, N, K);
    if (need <= 0) return run_gemm(-1, M, N, K, A, lda, B, ldb, C, ldc, stream);  // no scratch used
    const int st = check_gemm(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != MM_OK) return st;
    if (need > MM_STATIC_SCRATCH_BYTES)
        return invalid("the K split of this shape needs more than the MM_STATIC_SCRATCH_BYTES of static scratch");
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
    const int r = mm::gemm_split_static_launch(a, static_cast<hipStream_t>(stream));
    if (r != MM_OK) set_error_text(mm::static_ws_error());
    return r;
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
    if (mm::gemm_split2_ok(M, N, K)) return mm::gemm_split2_config();
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

int64_t mm_gemv_t_f32_workspace_bytes(int64_t M, int64_t N)
{
    if (M < 0 || N < 0 || M > kMaxDim || N > kMaxDim) return -1;
    if (M == 0 || N == 0) return 0;
    return 4 * mm::gemv_t_ws_floats(M, N);
}

int mm_gemv_t_f32_ws(int64_t M, int64_t N, const float *A, const float *x, float *y, void *workspace,
                     int64_t workspace_bytes, void *stream)
{
    const int64_t need = mm_gemv_t_f32_workspace_bytes(M, N);
    if (need > 0) {
        if (!workspace) return invalid("workspace is NULL");
        if ((uintptr_t)workspace % 16) return invalid("workspace not 16-byte aligned");
        if (workspace_bytes < need) return invalid("workspace smaller than mm_gemv_t_f32_workspace_bytes");
    }
    if (need <= 0) return mm_gemv_t_f32(M, N, A, x, y, stream);  // the checks and the strips kernel
    // same checks as mm_gemv_t_f32 (M, N >= 1 here)
    if (!A) return invalid("A is NULL");
    if (!x) return invalid("x is NULL");
    if (!y) return invalid("y is NULL");
    if ((uintptr_t)A % 4 || (uintptr_t)x % 4 || (uintptr_t)y % 4)
        return invalid("pointer not aligned to its element size");
    if (!extent_fits(M, N, N)) return invalid("A extent overflows");
    mm::GemvArgs a;
    a.A = A;
    a.x = x;
    a.y = y;
    a.M = (int)M;
    a.N = (int)N;
    return from_hip("gemv_t launch", mm::gemv_t_ws_launch(a, static_cast<float *>(workspace),
                                                            static_cast<hipStream_t>(stream)));
}

int mm_conv2d_f32(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R, int64_t S,
                  int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                  const float *x, const float *w, float *y, void *stream)
{
    return run_conv(-1, N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, y, stream);
}

int mm_conv2d_f32_config(int cfg, int64_t N, int64_t C, int64_t H, int64_t W, int64_t K,
                         int64_t R, int64_t S, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                         int64_t dh, int64_t dw, const float *x, const float *w, float *y,
                         void *stream)
{
    if (cfg < 0 || cfg >= mm::conv_num_configs()) return invalid("config index out of range");
    return run_conv(cfg, N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, x, w, y, stream);
}

int64_t mm_conv2d_out_dim(int64_t in, int64_t filter, int64_t stride, int64_t pad, int64_t dil)
{
    return conv_out_dim(in, filter, stride, pad, dil);
}

int mm_conv2d_f32_num_configs(void) { return mm::conv_num_configs(); }

const char *mm_conv2d_f32_config_name(int cfg) { return mm::conv_config_name(cfg); }

int mm_conv2d_f32_select(int64_t N, int64_t C, int64_t H, int64_t W, int64_t K, int64_t R,
                         int64_t S, int64_t sh, int64_t sw, int64_t ph, int64_t pw, int64_t dh,
                         int64_t dw)
{
    mm::ConvArgs a;
    bool work;
    if (check_conv(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, nullptr, nullptr, nullptr, false, a,
                   work) != MM_OK)
        return -1;
    return mm::conv_choose_config(a);
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
