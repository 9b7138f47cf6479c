// mm_gemm_cols.hip -- fp32 GEMM C = A x B for C with 1 to 4 columns: the
// fully-connected layer of "Matrix Operations" (docs.vulkan.org ML-inference
// tutorial, "Matrix-Vector Multiplication") on a batch of up to four input vectors
// ("Performance Considerations", batch processing), i.e. a GEMV with several x.
//
// The work is 2 N FLOP per element of A, far below what even the vector ALUs do per
// byte of HBM, so the kernel is the GEMV's row stream with N dot products per row:
//   * a wave owns two rows of A and reads them in 16-byte pieces (1 KB per wave
//     instruction), every piece of a 1024-k round requested before any arithmetic;
//   * a workgroup of four waves stages each round of B (1024 k x up to 4 columns,
//     16 KB) in LDS once for its eight rows (two buffers alternate between rounds,
//     one barrier per round); each lane multiplies its four k of A by the matching
//     four rows of B from LDS;
//   * per-lane sums are combined across the wave by a butterfly; the summation order
//     is fixed, so results are deterministic.
// Column blocks: a workgroup handles 4 columns; C with more columns takes more
// workgroups (A is then read once per block; mm_gemm_f32 uses this kernel only for
// N <= 4). A strided batch runs on the grid's z dimension.
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kRowsPerWave = 2;
constexpr int kRows = kWaves * kRowsPerWave;   // rows of C per workgroup
constexpr int kRound = 1024;     // k per round
constexpr int kPiecesPerRound = kRound / 256;  // 16-byte pieces per lane per row

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Four consecutive floats of a row at p, the first `valid` of them (zeros beyond).
template <bool VEC>
__device__ __forceinline__ f32x4 row_piece(const float *p, int valid)
{
    if (valid >= 4) {
        if constexpr (VEC) return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        return f32x4{p[0], p[1], p[2], p[3]};
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid > 0) v[0] = p[0];
    if (valid > 1) v[1] = p[1];
    if (valid > 2) v[2] = p[2];
    return v;
}

// NC: columns per workgroup (1, 2 or 4); VEC: A rows 16-byte aligned.
template <int NC, bool VEC>
__global__ __launch_bounds__(kWaves * 64) void gemm_cols_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) float xs[2][kRound * NC];
    const int64_t tiles_m = ((int64_t)p.M + kRows - 1) / kRows;
    const int64_t tiles = tiles_m * (((int64_t)p.N + NC - 1) / NC);
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    p.A += blockIdx.z * p.sa;
    p.B += blockIdx.z * p.sb;
    p.C += blockIdx.z * p.sc;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m0 = (int)(bid % tiles_m) * kRows + w * kRowsPerWave;
    const int n0 = (int)(bid / tiles_m) * NC;

    const float *arow[kRowsPerWave];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
        const int row = m0 + r;
        arow[r] = p.A + (int64_t)(row < p.M ? row : 0) * p.lda;  // spare rows read row 0
    }
    float acc[kRowsPerWave][NC];
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int n = 0; n < NC; ++n) acc[r][n] = 0.f;

    constexpr int XPT = kRound * NC / (kWaves * 64);  // B elements each thread stages
    int buf = 0;
    for (int k0 = 0; k0 < p.K; k0 += kRound, buf ^= 1) {
        // B rows k0 .. k0 + kRound - 1, columns n0 .. n0 + NC - 1, zeros outside
        float xv[XPT];
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int e = threadIdx.x + i * kWaves * 64;
            const int k = k0 + e / NC, n = n0 + e % NC;
            xv[i] = (k < p.K && n < p.N) ? p.B[(int64_t)k * p.ldb + n] : 0.f;
        }
        f32x4 va[kRowsPerWave][kPiecesPerRound];
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
            for (int u = 0; u < kPiecesPerRound; ++u) {
                const int k = k0 + 4 * (u * 64 + lane);
                va[r][u] = row_piece<VEC>(arow[r] + k, p.K - k);
            }
        // B was requested first, so writing it waits for B alone. Buffer buf was
        // last read two rounds ago, before the barrier of the previous round.
        float *xb = xs[buf];
#pragma unroll
        for (int i = 0; i < XPT; ++i) xb[threadIdx.x + i * kWaves * 64] = xv[i];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kPiecesPerRound; ++u) {
            const float *xk = xb + 4 * (u * 64 + lane) * NC;  // rows 4 (u * 64 + lane) ..
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x[NC];
                if constexpr (NC == 4) {
                    const f32x4 v = *reinterpret_cast<const f32x4 *>(xk + 4 * j);
                    x[0] = v[0];
                    x[1] = v[1];
                    x[2] = v[2];
                    x[3] = v[3];
                } else {
#pragma unroll
                    for (int n = 0; n < NC; ++n) x[n] = xk[NC * j + n];
                }
#pragma unroll
                for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
                    for (int n = 0; n < NC; ++n) acc[r][n] += va[r][u][j] * x[n];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int n = 0; n < NC; ++n) acc[r][n] = wave_sum(acc[r][n]);
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r) {
            const int row = m0 + r;
            if (row < p.M)
#pragma unroll
                for (int n = 0; n < NC; ++n)
                    if (n0 + n < p.N) p.C[(int64_t)row * p.ldc + n0 + n] = acc[r][n];
        }
    }
}

template <int NC>
hipError_t launch_nc(const GemmArgs &a, hipStream_t stream)
{
    const bool vec = (a.lda % 4 == 0) && ((uintptr_t)a.A % 16 == 0) && (a.batch == 1 || a.sa % 4 == 0);
    const int64_t tiles = (((int64_t)a.M + kRows - 1) / kRows) * (((int64_t)a.N + NC - 1) / NC);
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    const void *fn = vec ? reinterpret_cast<const void *>(&gemm_cols_kernel<NC, true>)
                         : reinterpret_cast<const void *>(&gemm_cols_kernel<NC, false>);
    GemmArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(fn, dim3(gx, gy, (unsigned)a.batch), dim3(kWaves * 64), args, 0, stream);
}

}  // namespace

hipError_t gemm_cols_launch(const GemmArgs &a, hipStream_t stream)
{
    if (a.N == 1) return launch_nc<1>(a, stream);
    if (a.N == 2) return launch_nc<2>(a, stream);
    return launch_nc<4>(a, stream);
}

}  // namespace mm
