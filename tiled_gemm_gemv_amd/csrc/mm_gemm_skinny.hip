// mm_gemm_skinny.hip -- fp32 GEMM C = A x B for narrow C: the fully-connected layer
// y = A x of "Matrix Operations" (docs.vulkan.org ML-inference tutorial,
// "Matrix-Vector Multiplication") applied to a small batch, i.e. B holds a few
// input vectors as columns (N up to 64). The pages' batching remark ("Performance
// Considerations", batch processing) is this case.
//
// With N this small the work per byte of A is N/2 FLOP, so A has to stream from
// HBM about once while the matrix cores do at most a few percent of a square
// GEMM's work per byte. A macro-tile GEMM would give each workgroup 64 or more
// rows and leave most CUs idle (4096 rows / 64 = 64 workgroups); here:
//   * a workgroup owns 16 rows of C and 64 columns (v_mfma_f32_16x16x4_f32, four
//     16 x 16 accumulator blocks), so 4096 rows fill 256 CUs;
//   * its W waves split K: wave w takes 16-deep chunks w*U .. w*U+U-1, then every
//     W*U-th run of chunks; their sums meet in LDS and wave 0 adds them in wave order;
//   * A is read once, in 16-byte pieces along its rows; B (K x 64 at most, shared
//     by every workgroup) is read from L2 with 4-byte loads, 16 consecutive columns
//     per quarter-wave.
// k order inside a 16-deep chunk: v_mfma_f32_16x16x4_f32 multiplies a 16 x 4 slice
// of A by a 4 x 16 slice of B; lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16].
// At MFMA step s, lanes with l / 16 = g feed k = 4g + s, so each lane's four A values
// of a chunk are one 16-byte load, and every k of the chunk is added exactly once.
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSkinnyRows = 16;   // rows of C per workgroup
constexpr int kSkinnyCols = 64;   // columns of C per workgroup
constexpr int kChunk = 16;        // k per chunk

template <bool VEC>
__device__ __forceinline__ f32x4 load4s(const float *p, int valid)
{
    if (valid >= 4) {
        if constexpr (VEC) return *reinterpret_cast<const f32x4 *>(p);
        return f32x4{p[0], p[1], p[2], p[3]};
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid > 0) v[0] = p[0];
    if (valid > 1) v[1] = p[1];
    if (valid > 2) v[2] = p[2];
    return v;
}

// NB: 16-column blocks of C handled (1..4); W: waves splitting K; U: chunks per wave
// per round (all of a round's loads are issued before its MFMAs).
// VEC_B (NB = 4, B's rows 16-byte aligned), on tiles whose 64 columns all lie in C:
// the blocks' columns are interleaved, column c of block nb being column n0 + NB c + nb of
// C, so the NB values a lane feeds the NB blocks at one MFMA step are NB consecutive floats
// of one row of B: one 16-byte load instead of four 4-byte loads, which cost the same
// address cycles each (4096 x 64 x 4096: 51 -> 58-60 TFLOP/s; with NB = 2 and 8-byte loads
// 4096 x 32 x 4096 lost 8-28%). Other tiles keep the blocks side by side (column
// n0 + 16 nb + c) and load B by the float.
template <int NB, int W, int U, bool VEC_A, bool VEC_B>
__global__ __launch_bounds__(W * 64) void gemm_skinny_kernel(GemmArgs p)
{
    static_assert(!VEC_B || NB == 4, "vector B loads of 4 floats");
    __shared__ f32x4 partial[(W > 1 ? W - 1 : 1) * NB * 64];
    // workgroup -> (row block, column block): row blocks vary fastest
    const int64_t tiles_m = (p.M + kSkinnyRows - 1) / kSkinnyRows;
    const int64_t tiles = tiles_m * ((p.N + kSkinnyCols - 1) / kSkinnyCols);
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    // problem of a strided batch: grid layer blockIdx.z
    p.A += blockIdx.z * p.sa;
    p.B += blockIdx.z * p.sb;
    p.C += blockIdx.z * p.sc;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int m0 = (int)(bid % tiles_m) * kSkinnyRows;
    const int n0 = (int)(bid / tiles_m) * kSkinnyCols;
    const int row = m0 + c16;
    const bool row_ok = row < p.M;
    const float *arow = p.A + (int64_t)(row_ok ? row : m0) * p.lda;

    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = (p.K + kChunk - 1) / kChunk;
    // every lane's NB columns inside C (wave-uniform): interleaved blocks, vector loads of B
    const bool full_cols = VEC_B && n0 + NB * 16 <= p.N;
    // this lane's column in block nb: col0 + nb * cstep
    const int col0 = full_cols ? n0 + NB * c16 : n0 + c16, cstep = full_cols ? 1 : 16;
    for (int c0 = w * U; c0 < nchunks; c0 += W * U) {
        f32x4 a[U];
        float b[U][4][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (c0 + u) * kChunk + 4 * g;   // this lane's first k of the chunk
            const int valid_a = row_ok ? p.K - k : 0;  // <= 0 past the end of K
            a[u] = load4s<VEC_A>(arow + k, valid_a);
            if (full_cols) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kk = k + s;
                    // rows past K read row K - 1 and are replaced by zeros
                    const float *src = p.B + (int64_t)min(kk, p.K - 1) * p.ldb + col0;
                    typedef float fv __attribute__((ext_vector_type(NB)));
                    const fv v = *reinterpret_cast<const fv *>(src);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) b[u][s][nb] = kk < p.K ? v[nb] : 0.f;
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int kk = k + s;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const int col = col0 + nb * cstep;
                        b[u][s][nb] = (kk < p.K && col < p.N) ? p.B[(int64_t)kk * p.ldb + col] : 0.f;
                    }
                }
            }
        }
        // every load of the round goes out before the first MFMA
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u][s], b[u][s][nb], acc[nb],
                                                                   0, 0, 0);
    }

    if constexpr (W > 1) {
        if (w > 0) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) partial[((w - 1) * NB + nb) * 64 + lane] = acc[nb];
        }
        __syncthreads();
        if (w > 0) return;  // no barrier follows
#pragma unroll 1
        for (int v = 1; v < W; ++v)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] += partial[((v - 1) * NB + nb) * 64 + lane];
    }

    // Accumulator layout of v_mfma_f32_16x16x4_f32: lane l, register r holds row
    // 4 * (l / 16) + r, column l % 16 of the 16 x 16 block (column col0 + nb cstep of C).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = m0 + 4 * g + r;
            const int j = col0 + nb * cstep;
            if (i < p.M && j < p.N) p.C[(int64_t)i * p.ldc + j] = acc[nb][r];
        }
}

template <int NB, int W, int U>
hipError_t launch_nb(const GemmArgs &a, bool vec, hipStream_t stream)
{
    const int64_t tiles = ((a.M + kSkinnyRows - 1) / kSkinnyRows) * ((a.N + kSkinnyCols - 1) / kSkinnyCols);
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    // B's rows (and the batch's B matrices) aligned for loads of 4 floats
    constexpr bool kVecNb = NB == 4;
    const bool vec_b = kVecNb && a.ldb % NB == 0 && a.sb % NB == 0 && (uintptr_t)a.B % (4 * NB) == 0;
    const void *fn;
    if (vec_b) fn = vec ? reinterpret_cast<const void *>(&gemm_skinny_kernel<NB, W, U, true, kVecNb>)
                        : reinterpret_cast<const void *>(&gemm_skinny_kernel<NB, W, U, false, kVecNb>);
    else fn = vec ? reinterpret_cast<const void *>(&gemm_skinny_kernel<NB, W, U, true, false>)
                  : reinterpret_cast<const void *>(&gemm_skinny_kernel<NB, W, U, false, false>);
    GemmArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(fn, dim3(gx, gy, (unsigned)a.batch), dim3(W * 64), args, 0, stream);
}

}  // namespace

// Narrow-C GEMM: 16 x 64 tiles of C, K split over W waves per workgroup. A wave
// keeps L / NB chunks of loads in flight per round, so that fewer column blocks
// (fewer B registers per chunk) mean more of A in flight.
template <int W, int L>
hipError_t gemm_skinny_launch(const GemmArgs &a, hipStream_t stream)
{
    const bool vec = (a.lda % 4 == 0) && ((uintptr_t)a.A % 16 == 0);
    // columns actually present in a tile: all 64 unless N is smaller
    const int cols = a.N < kSkinnyCols ? a.N : kSkinnyCols;
    if (cols <= 16) return launch_nb<1, W, L>(a, vec, stream);
    if (cols <= 32) return launch_nb<2, W, (L / 2 > 1 ? L / 2 : 1)>(a, vec, stream);
    if (cols <= 48) return launch_nb<3, W, (L / 3 > 1 ? L / 3 : 1)>(a, vec, stream);
    return launch_nb<4, W, (L / 4 > 1 ? L / 4 : 1)>(a, vec, stream);
}

template hipError_t gemm_skinny_launch<8, 16>(const GemmArgs &, hipStream_t);
template hipError_t gemm_skinny_launch<4, 16>(const GemmArgs &, hipStream_t);
template hipError_t gemm_skinny_launch<16, 4>(const GemmArgs &, hipStream_t);

}  // namespace mm
