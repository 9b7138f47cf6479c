// mm_gemv_t.hip -- transposed fp32 GEMV y = A^T x, y[j] = sum over i of A[i][j] * x[i],
// for a row-major M x N matrix A (x has M entries, y has N).
//
// The plain definition is the GEMV of "Matrix Operations" (docs.vulkan.org
// ML-inference tutorial, "Matrix-Vector Multiplication") applied to the transpose:
// each output is a column of A dotted with x. Reading A column-wise would stride
// by a whole row per element, so the kernel still streams A along its rows and
// gives each workgroup a strip of STRIP columns (16, 32 or 64, chosen so that the N /
// STRIP strips give about one workgroup per CU) over all M rows:
//   * a wave reads 64 / (STRIP / 4) rows x 4 STRIP bytes per instruction (lane l: row
//     l / (STRIP / 4) of the group, 4 columns at 4 (l % (STRIP / 4))), 16-byte loads, up
//     to 16 instructions in flight; the waves take interleaved groups of rows;
//   * each lane keeps 4 column sums; at the end the lanes that share columns are
//     combined with a butterfly, then the waves in LDS in wave order, so the
//     summation order is fixed and results are deterministic;
//   * consecutive strips go to the same XCD (the launch order is renumbered as in the
//     GEMM), so neighbouring pieces of a 128-byte line are read through one L2.
// Rows that are not 16-byte aligned (N % 4 != 0 or an unaligned A) use 4-byte loads.
//
// With a workspace (gemv_t_ws_launch) the rows are read as the GEMV reads them: a
// workgroup takes a 256-column strip of a block of rows, so a wave instruction reads
// 1 KB of one row; the 16 waves of the workgroup take interleaved rows, 16 in flight
// each, and their sums meet in LDS in wave order. Each workgroup writes its strip of
// the row block's partial y to the workspace, and a second launch adds the row blocks'
// partials per column in row-block order (deterministic). A single launch that let the
// last workgroup of a strip add the partials needs device-scope release/acquire fences,
// which on this GPU write back and invalidate a whole XCD's L2 per workgroup: measured
// far slower than the second launch.
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kStrip = 16;        // columns per workgroup
constexpr int kWaves = 4;         // waves per workgroup
constexpr int kDepth = 16;        // row groups in flight per wave

__device__ __forceinline__ int strip_of_block(int bid, int nblocks)
{
    const int q = nblocks / 8, r = nblocks % 8;
    const int xcd = bid % 8, slot = bid / 8;
    return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

template <bool VEC, int STRIP = kStrip, int WAVES = kWaves>
__global__ __launch_bounds__(WAVES * 64) void gemv_t_kernel(GemvArgs p)
{
    constexpr int LPR = STRIP / 4;          // lanes per row (4 columns each)
    constexpr int RPL = 64 / LPR;           // rows per wave instruction
    __shared__ f32x4 partial[(WAVES - 1) * 64];
    const int64_t strips = ((int64_t)p.N + STRIP - 1) / STRIP;
    const int64_t bid = linear_block();
    if (bid >= strips) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int strip = strip_of_block((int)bid, (int)strips);
    const int j0 = strip * STRIP + 4 * (lane % LPR);   // this lane's first column
    const int rsub = lane / LPR;                         // row within a group of RPL rows
    const int ncols = p.N - j0;                          // columns left from j0 (may be <= 0)

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // row groups g = w, w + WAVES, ...; a round takes kDepth of them
    const int groups = (p.M + RPL - 1) / RPL;
    for (int g0 = w; g0 < groups; g0 += WAVES * kDepth) {
        f32x4 va[kDepth];
        float vx[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int i = (g0 + d * WAVES) * RPL + rsub;
            const bool row_ok = i < p.M;
            const float *src = p.A + (int64_t)(row_ok ? i : 0) * p.N + j0;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (row_ok) {
                if (VEC && ncols >= 4) {
                    v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src));
                } else {
                    if (ncols > 0) v[0] = src[0];
                    if (ncols > 1) v[1] = src[1];
                    if (ncols > 2) v[2] = src[2];
                    if (ncols > 3) v[3] = src[3];
                }
            }
            va[d] = v;
            vx[d] = row_ok ? p.x[i] : 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            acc[0] += va[d][0] * vx[d];
            acc[1] += va[d][1] * vx[d];
            acc[2] += va[d][2] * vx[d];
            acc[3] += va[d][3] * vx[d];
        }
    }
    // lanes l, l ^ LPR, l ^ 2 LPR, ... (same l % LPR) hold the same 4 columns
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    if (w > 0 && lane < LPR) partial[(w - 1) * 64 + lane] = acc;
    __syncthreads();
    if (w > 0 || lane >= LPR) return;  // no barrier follows
#pragma unroll 1
    for (int v = 1; v < WAVES; ++v) acc += partial[(v - 1) * 64 + lane];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        if (c < ncols) p.y[j0 + c] = acc[c];
}

constexpr int kWide = 256;     // columns per row-block workgroup (1 KB of a row per wave)
constexpr int kRbWaves = 16;   // waves per row-block workgroup
constexpr int kRbDepth = 16;   // rows in flight per wave
constexpr int kMinBlockRows = kRbWaves * kRbDepth;

// Pass 1: partial y of row block rb over columns [256 cs, 256 cs + 256) into
// part[rb * N + j]. N % 4 == 0, A 16-byte aligned.
__global__ __launch_bounds__(kRbWaves * 64) void gemv_t_rows_kernel(GemvArgs p, float *part, int blocks,
                                                                     int block_rows)
{
    __shared__ f32x4 red[kRbWaves][64];
    const int64_t strips = ((int64_t)p.N + kWide - 1) / kWide;
    const int64_t bid = linear_block();
    if (bid >= strips * blocks) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int rb = (int)(bid / strips), cs = (int)(bid % strips);
    const int j = cs * kWide + 4 * lane;
    const bool col_ok = j < p.N;  // then j + 3 < N too (N % 4 == 0)
    const int r0 = rb * block_rows;
    const int r1 = min(p.M, r0 + block_rows);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = r0 + w; t0 < r1; t0 += kRbWaves * kRbDepth) {
        f32x4 va[kRbDepth];
        float vx[kRbDepth];
#pragma unroll
        for (int d = 0; d < kRbDepth; ++d) {
            const int i = t0 + d * kRbWaves;
            const bool ok = i < r1;
            va[d] = (ok && col_ok) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.A + (int64_t)i * p.N + j))
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
            vx[d] = ok ? p.x[i] : 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < kRbDepth; ++d) {
            acc[0] += va[d][0] * vx[d];
            acc[1] += va[d][1] * vx[d];
            acc[2] += va[d][2] * vx[d];
            acc[3] += va[d][3] * vx[d];
        }
    }
    red[w][lane] = acc;
    __syncthreads();
    if (w != 0 || !col_ok) return;  // no barrier follows
    f32x4 s = red[0][lane];
#pragma unroll
    for (int v = 1; v < kRbWaves; ++v) s += red[v][lane];
    *reinterpret_cast<f32x4 *>(part + (int64_t)rb * p.N + j) = s;
}

// Pass 2: y[j .. j + 3] = sum over row blocks, in order, of the partials (one lane per 4
// columns, 64 lanes per workgroup, so that N = 4096 spreads over 16 CUs). The loads go out
// 16 at a time (a loop of dependent load-add steps would pay one memory round trip per row
// block; with at most 16 blocks, as at N >= 4096, one round trip in all); past the last
// block they read as zeros, which leave the sum as it is. Against 8 loads a round on
// 256-lane workgroups: 4096 x 4096 16.0 -> 15.3 us per call.
__global__ __launch_bounds__(64) void gemv_t_sum_kernel(const float *part, float *y, int N, int blocks)
{
    const int64_t j = 4 * (linear_block() * 64 + threadIdx.x);
    if (j >= N) return;
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < blocks; r0 += 16) {
        f32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            v[u] = (r0 + u < blocks) ? *reinterpret_cast<const f32x4 *>(part + (int64_t)(r0 + u) * N + j)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 16; ++u) t += v[u];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) y[j + c] = t[c];
}

// Row blocks for (M, N): about 256 workgroups in all, at least kMinBlockRows rows each
// (0: the strips kernel serves the shape better, or its rows are not 16-byte aligned).
int row_blocks(int64_t M, int64_t N)
{
    if (N % 4 != 0) return 0;
    const int64_t strips = (N + kWide - 1) / kWide;
    int64_t blocks = (256 + strips - 1) / strips;
    const int64_t most = M / kMinBlockRows;
    if (blocks > most) blocks = most;
    return blocks >= 2 ? (int)blocks : 0;
}

}  // namespace

int64_t gemv_t_ws_floats(int64_t M, int64_t N)
{
    return (int64_t)row_blocks(M, N) * N;
}

hipError_t gemv_t_ws_launch(const GemvArgs &a, float *ws, hipStream_t stream)
{
    const int blocks = row_blocks(a.M, a.N);
    if (blocks == 0 || (uintptr_t)a.A % 16 != 0) return gemv_t_launch(a, stream);
    const int block_rows = (int)(((int64_t)a.M + blocks - 1) / blocks);
    const int64_t strips = ((int64_t)a.N + kWide - 1) / kWide;
    unsigned gx, gy;
    if (!grid_for(strips * blocks, gx, gy)) return hipErrorInvalidConfiguration;
    GemvArgs arg = a;
    int nb = blocks, br = block_rows;
    void *args1[] = {&arg, &ws, &nb, &br};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&gemv_t_rows_kernel), dim3(gx, gy),
                                   dim3(kRbWaves * 64), args1, 0, stream);
    if (e != hipSuccess) return e;
    const int64_t lanes = ((int64_t)a.N + 3) / 4;
    if (!grid_for((lanes + 63) / 64, gx, gy)) return hipErrorInvalidConfiguration;
    const float *part = ws;
    float *y = a.y;
    int n = a.N;
    void *args2[] = {&part, &y, &n, &nb};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_t_sum_kernel), dim3(gx, gy), dim3(64), args2, 0,
                           stream);
}

// Strip width by N: about one workgroup per CU. With N / 16 strips far above 256 the
// 64-byte row pieces of 16-column strips cost (8192 x 8192: 75.4 us against 53.8 with
// 32 columns; 4096 x 16384: 76.9 against 46.6 with 64 columns on 8 waves); with fewer
// strips than CUs the wide ones leave CUs idle (4096 x 4096: 19.1 us with 16 columns,
// 22.4 with 32, 28.1 with 64). Rows that are not 16-byte aligned keep 16-column strips.
hipError_t gemv_t_launch(const GemvArgs &a, hipStream_t stream)
{
    const bool vec = (a.N % 4 == 0) && ((uintptr_t)a.A % 16 == 0);
    const int strip = !vec || a.N <= 16 * 384 ? 16 : a.N <= 32 * 384 ? 32 : 64;
    const int waves = strip == 64 ? 8 : kWaves;
    const int64_t strips = ((int64_t)a.N + strip - 1) / strip;
    unsigned gx, gy;
    if (!grid_for(strips, gx, gy)) return hipErrorInvalidConfiguration;
    GemvArgs arg = a;
    void *args[] = {&arg};
    const void *fn = !vec         ? reinterpret_cast<const void *>(&gemv_t_kernel<false>)
                     : strip == 16 ? reinterpret_cast<const void *>(&gemv_t_kernel<true>)
                     : strip == 32 ? reinterpret_cast<const void *>(&gemv_t_kernel<true, 32, 4>)
                                   : reinterpret_cast<const void *>(&gemv_t_kernel<true, 64, 8>);
    return hipLaunchKernel(fn, dim3(gx, gy), dim3(waves * 64), args, 0, stream);
}

}  // namespace mm
