// mm_internal.h -- declarations shared by the HIP sources of libmm (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

// Launch grids. HIP's dispatch packet holds each grid dimension in work-items, in
// 32 bits, so a 1-D grid stops at 2^32 / (threads per workgroup) workgroups. A
// launch of more workgroups uses a 2-D grid: kMaxGridX workgroups along x (a
// multiple of 8, so x % 8 is still the XCD a workgroup lands on) times as many rows
// as needed along y. Kernels number workgroups linear_block() = y * gridDim.x + x;
// those at `count` or beyond return at once. Up to kMaxGridX workgroups the grid is
// the plain 1-D one.
constexpr int64_t kMaxGridX = (int64_t(1) << 22) - 8;  // * 1024 threads < 2^32

// Grid of `count` >= 1 workgroups; false if it needs more than 65535 rows.
inline bool grid_for(int64_t count, unsigned &gx, unsigned &gy)
{
    if (count <= kMaxGridX) {
        gx = (unsigned)count;
        gy = 1;
        return true;
    }
    const int64_t rows = (count + kMaxGridX - 1) / kMaxGridX;
    if (rows > 65535) return false;
    gx = (unsigned)kMaxGridX;
    gy = (unsigned)rows;
    return true;
}

__device__ __forceinline__ int64_t linear_block()
{
    return (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
}

// Arguments of one GEMM launch, already validated on the host. Sizes fit in
// int32; offsets are formed in int64.
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    // strided batch: problem b uses A + b * sa, B + b * sb, C + b * sc (elements)
    int batch = 1;
    int64_t sa = 0, sb = 0, sc = 0;
};

// Arguments of one GEMV launch (A has packed rows: leading dimension N).
struct GemvArgs {
    const float *A;
    const float *x;
    float *y;
    int M, N;
};

// Time model for choosing a tile shape (arbitrary units): a CU computes a BM x BN tile
// at `tflops` when fill_waves or more waves share it, and proportionally slower with
// fewer (latency is then exposed; 8 for register-staged tiles, fewer for the tiles whose
// panels the LDS DMA loads: one 4-wave workgroup per CU of the 128 x 128 direct tile
// measured about 80% of its full rate, of the 64 x 64 ones about 70%). The busiest CU gets ceil(tiles / 256) tiles; it runs them in
// sets of at most wg_per_cu concurrent workgroups, and a last, smaller set runs at its
// own occupancy.
inline double tile_time(int64_t tiles, int bm, int bn, int waves, int wg_per_cu, double tflops,
                        double fill_waves = 8)
{
    constexpr int64_t kCus = 256;
    const int64_t t = (tiles + kCus - 1) / kCus;
    auto set_time = [&](int64_t wgs) {
        double fill = (double)(wgs * waves) / fill_waves;
        if (fill > 1.0) fill = 1.0;
        return (double)wgs * bm * bn / (tflops * fill);
    };
    const int64_t full = t / wg_per_cu, rem = t % wg_per_cu;
    return (double)full * set_time(wg_per_cu) + (rem ? set_time(rem) : 0.0);
}

// K-steps of depth bk cover ceil(K / bk) bk rows: a partial last step costs a full one.
inline double k_steps_factor(int64_t K, int bk)
{
    return K > 0 ? (double)((K + bk - 1) / bk * bk) / (double)K : 1.0;
}

// GEMM tile configurations, in the order of the public config index.
int gemm_num_configs();
const char *gemm_config_name(int cfg);
// batch: number of independent problems launched together (tiles are counted over all).
int gemm_select_config(int64_t M, int64_t N, int64_t K, int64_t batch = 1);
// The modelled time of tile config `cfg` (a macro-tile config; others: a large value).
double gemm_config_time(int cfg, int64_t M, int64_t N, int64_t K, int64_t batch);
// Enqueue config `cfg` of the GEMM (K >= 1, M >= 1, N >= 1).
hipError_t gemm_launch(int cfg, const GemmArgs &a, hipStream_t stream);
// K split across workgroups through a caller workspace (mm_gemm.hip): the number of K
// chunks for (M, N, K) (0: no split), the workspace it needs (floats) and the launch
// (the product per chunk into the workspace, then the sum in chunk order into C).
int gemm_split_chunks(int64_t M, int64_t N, int64_t K);
int64_t gemm_split_ws_floats(int64_t M, int64_t N, int64_t K);
hipError_t gemm_split_launch(const GemmArgs &a, float *ws, hipStream_t stream);
// The K split with the library's static device scratch as its workspace
// (mm_static_ws.hip): an mm_status (text of a failure from static_ws_error()).
int gemm_split_static_launch(const GemmArgs &a, hipStream_t stream);
const char *static_ws_error();
// K split in two halves without a workspace (mm_gemm.hip): true where mm_gemm_f32 takes
// it, and the launch (C zeroed, then both halves added into it).
bool gemm_split2_ok(int64_t M, int64_t N, int64_t K);
int gemm_split2_config();  // the config index of the halves' tile
hipError_t gemm_split2_launch(const GemmArgs &a, hipStream_t stream);

// Narrow-C GEMM (mm_gemm_skinny.hip): 16 x 64 tiles of C, K split over W waves
// per workgroup, L / (column blocks) 16-deep chunks per wave per round. Correct for
// any shape.
template <int W, int L>
hipError_t gemm_skinny_launch(const GemmArgs &a, hipStream_t stream);
// Narrow C with A moved into LDS in whole row segments (mm_gemm_narrow.hip): true where it
// takes the shape (N <= 64, N % 4 == 0, K a multiple of its round), and the launch (other
// shapes run config 8's 16-row kernel).
bool gemm_narrow_ok(const GemmArgs &a);
hipError_t gemm_narrow_launch(const GemmArgs &a, hipStream_t stream);

// fp32 GEMM with panels loaded straight into LDS (mm_gemm_direct.hip); any shape and
// alignment, except T256, which takes only shapes direct_f32_wide_ok(a, 256) accepts
// (hipErrorInvalidValue otherwise). T64S8 / T64S4: 64 x 64 tiles with 8 / 4 LDS stages.
// direct_f32_wide_ok(a, bn): every B load of a tile bn wide can take 16-byte lanes
// (K % 16 == 0, and N % 4 == 0 or N >= bn) and the lane offsets fit 32 bits.
enum class DirectTile { T256, T128, T64S8, T64S4, T64K2, T128M16 };
bool direct_f32_wide_ok(const GemmArgs &a, int bn);
hipError_t gemm_direct_launch(DirectTile t, const GemmArgs &a, hipStream_t stream);
// The 64 x 64 direct tile (4 stages; K-steps over two wave groups where K % 32 == 0, as
// config 14) with an epilogue that adds each tile into C atomically; a.batch problems may
// share C (sc = 0).
hipError_t gemm_direct64_add_launch(const GemmArgs &a, hipStream_t stream);

// GEMM for C with few columns (mm_gemm_cols.hip): one wave per row, B staged in LDS;
// correct for any shape, meant for N <= 4.
hipError_t gemm_cols_launch(const GemmArgs &a, hipStream_t stream);

// GEMM with 16-bit inputs (mm_gemm_h16.hip); A and B hold bf16 (bf16 = true) or
// binary16 bit patterns, C is fp32. M, N, K >= 1.
int gemm16_num_configs();
const char *gemm16_config_name(int cfg);
int gemm16_select_config(int64_t M, int64_t N, int64_t K);
hipError_t gemm16_launch(int cfg, bool bf16, const void *A, int64_t lda, const void *B, int64_t ldb,
                         float *C, int64_t ldc, int M, int N, int K, hipStream_t stream);

// A 2-D convolution (mm_conv.hip): x is N x C x H x W, w is K x C x R x S, y is
// N x K x P x Q, all packed; strides sh, sw, padding ph, pw, dilation dh, dw.
struct ConvArgs {
    int64_t N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, P, Q;
    const float *x;
    const float *w;
    float *y;
};

// Convolution configurations: tile shapes of the GEMM (BMxBNxBK and wave tile as there).
int conv_num_configs();
const char *conv_config_name(int cfg);
// Choice for the implicit GEMM of M filters by N output positions by K = C R S.
int conv_select_config(int64_t M, int64_t N, int64_t K);
// The configuration conv_launch uses for a shape when none is given.
int conv_choose_config(const ConvArgs &a);
// Enqueue the convolution (cfg < 0: choose). The caller has checked the shape:
// N, K, P, Q >= 1, C >= 0, one image of x and the padded plane (H + 2 ph)(W + 2 pw)
// below 2^30 elements, C R S and P Q below 2^31, H + 2 ph, W + 2 pw, dh (R - 1),
// dw (S - 1) below 2^29.
hipError_t conv_launch(int cfg, const ConvArgs &a, hipStream_t stream);

// Enqueue the GEMV (M >= 1, N >= 1).
hipError_t gemv_launch(const GemvArgs &a, hipStream_t stream);

// Enqueue the transposed GEMV y = A^T x (mm_gemv_t.hip); x has M entries, y has N.
// M >= 1, N >= 1.
hipError_t gemv_t_launch(const GemvArgs &a, hipStream_t stream);
// y = A^T x in row blocks with partial sums in a workspace of gemv_t_ws_floats(M, N)
// floats (16-byte aligned), then a second launch that adds them; shapes that gain
// nothing from it (or whose rows are not 16-byte aligned) run gemv_t_launch and leave
// the workspace alone. M, N >= 1.
int64_t gemv_t_ws_floats(int64_t M, int64_t N);
hipError_t gemv_t_ws_launch(const GemvArgs &a, float *ws, hipStream_t stream);

// Enqueue a fill of the rows x cols matrix at p (row stride ld) with zeros.
hipError_t zero_fill_launch(float *p, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

}  // namespace mm
