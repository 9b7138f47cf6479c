// mm_gemm_narrow.hip -- fp32 GEMM C = A x B for narrow C (N <= 64) with A streamed in
// whole row segments: the fully-connected layer on a small batch ("Matrix Operations",
// docs.vulkan.org ML-inference tutorial, "Matrix-Vector Multiplication"; the batching
// remark of "Performance Considerations").
//
// The 16-row MFMA tile (v_mfma_f32_16x16x4_f32) wants, in each lane, 4 consecutive k of
// one of 16 rows; loaded that way, a wave instruction reads 64 bytes from each of 16 rows,
// and A streams at about 4 TB/s where whole-row reads (1 KB of one row per instruction, as
// the GEMV reads) reach 5.7 TB/s (measured on MI355X, 64 MiB, cold). So here the LDS DMA
// moves A into LDS in whole row segments, and the MFMA operands are read from there:
//   * a workgroup owns 16 rows of C and NB 16-column blocks (N <= 16 NB); K runs in rounds
//     of KR k. A round's A tile (16 x KR) and B tile (KR x 16 NB) go HBM -> LDS by
//     global_load_lds_dwordx4 into a ring of NS stages, the loads of round r + NS - 1
//     issued once every wave is past round r's barrier;
//   * the W waves split each round's 16-k chunks (wave w: chunks w, w + W, ...); a chunk
//     is 4 MFMA steps per column block; the waves' sums meet in LDS at the end and wave 0
//     adds them in wave order (deterministic);
//   * A tile: row i, 16-byte chunk c at slot c ^ (i % 16), so the 16 lanes that read one
//     chunk of 16 rows at once hit 16 distinct bank groups;
//   * B tile: the blocks' columns are interleaved (column c of block nb is column
//     n0 + NB c + nb of C), so the NB values a lane feeds the NB blocks at one step are NB
//     consecutive floats of a row (one LDS read); B's rows are permuted within groups of 4
//     (row 4q + s at 4q + (s + q) % 4) so that the 4 rows one read instruction touches
//     (k = 4g + s, g = 0..3) start in different bank groups.
// Shapes: K a multiple of KR (every round whole), N a multiple of 4 (no 16-byte chunk of B
// crosses a row end; chunks past N are clamped to the last one and feed only unstored
// columns), rows past M clamped to M - 1. Others run the 16-row kernel of mm_gemm_skinny.hip.
#include "mm_direct.h"

namespace mm {
namespace {

template <int NB_, int W_, int KR_, int NS_>
struct NarrowTile {
    static constexpr int NB = NB_, W = W_, KR = KR_, NS = NS_;
    static constexpr int NT = W * 64;
    static constexpr int A_ROW = KR * 4;                 // bytes of a row of the A tile
    static constexpr int A_CPR = A_ROW / 16;             // its 16-byte chunks
    static constexpr int A_BYTES = 16 * A_ROW;
    static constexpr int B_ROW = NB * 64;                // bytes of a row of the B tile
    static constexpr int B_CPR = B_ROW / 16;
    static constexpr int B_BYTES = KR * B_ROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LOADS = STAGE / 1024 / W;       // 1 KB DMA loads per wave per round
    static constexpr int CHUNKS = KR / 16 / W;           // 16-k chunks per wave per round
    static_assert(NB == 1 || NB == 2 || NB == 4, "1, 2 or 4 column blocks");
    static_assert(A_ROW <= 1024 && 1024 % A_ROW == 0 && 1024 % B_ROW == 0, "whole rows per DMA load");
    static_assert(STAGE % (1024 * W) == 0 && KR % (16 * W) == 0, "whole loads and chunks per wave");
    static_assert(A_CPR <= 64 && A_CPR % 16 == 0, "A rows of 16 to 64 chunks");
    static_assert(NS * STAGE <= 160 * 1024, "stages must fit the 160 KB LDS");
    static_assert((NS - 2) * LOADS <= 63, "vmcnt range");
    static_assert((W - 1) * NB * 64 * 16 <= NS * STAGE, "the waves' sums fit the ring");
};

// B tile row slot of row r (a permutation within each group of 4 rows) and its inverse
__device__ __forceinline__ int b_slot(int r) { return (r & ~3) | (((r & 3) + (r >> 2)) & 3); }
__device__ __forceinline__ int b_row(int slot) { return (slot & ~3) | (((slot & 3) - (slot >> 2)) & 3); }

template <class T>
__global__ __launch_bounds__(T::NT) void gemm_narrow_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) char lds[T::NS * T::STAGE];
    const int64_t tiles_m = (p.M + 15) / 16;
    const int64_t tiles = tiles_m * ((p.N + 16 * T::NB - 1) / (16 * T::NB));
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    p.A += blockIdx.z * p.sa;
    p.B += blockIdx.z * p.sb;
    p.C += blockIdx.z * p.sc;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int m0 = (int)(bid % tiles_m) * 16;
    const int n0 = (int)(bid / tiles_m) * (16 * T::NB);

    // the sources of this wave's DMA loads at k0 = 0: load t of a round (t = w, w + W, ...)
    // fills bytes [1024 t, 1024 t + 1024) of the stage, lane l its 16 bytes at 16 l
    const float *src[T::LOADS];
    int64_t kstep[T::LOADS];  // elements the source advances per round
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) {
        const int byte = (w + i * T::W) * 1024 + 16 * lane;
        if (byte < T::A_BYTES) {
            const int row = byte / T::A_ROW, slot = (byte % T::A_ROW) / 16;
            const int chunk = slot ^ (row & 15);
            src[i] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + 4 * chunk;
            kstep[i] = T::KR;
        } else {
            const int b = byte - T::A_BYTES;
            const int slot_row = b / T::B_ROW, chunk = (b % T::B_ROW) / 16;
            const int krow = b_row(slot_row);
            const int col = min(n0 + 4 * chunk, p.N - 4);
            src[i] = p.B + (int64_t)krow * p.ldb + col;
            kstep[i] = (int64_t)T::KR * p.ldb;
        }
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_char *)lds;
    const int rounds = p.K / T::KR;
    auto issue = [&](int r) {
        const unsigned st = lds0 + (r % T::NS) * T::STAGE;
#pragma unroll
        for (int i = 0; i < T::LOADS; ++i)
            load_to_lds<16>(st + (w + i * T::W) * 1024, src[i] + r * kstep[i]);
    };

    // operand byte offsets in a stage for this wave's chunk j of a round (k = 16 (w + j W)
    // + 4 g + s): A one 16-byte read, B one read of NB floats per step s
    int a_off[T::CHUNKS], b_off[T::CHUNKS][4];
#pragma unroll
    for (int j = 0; j < T::CHUNKS; ++j) {
        const int ch = w + j * T::W;  // the chunk in the round
        a_off[j] = c16 * T::A_ROW + 16 * ((4 * ch + g) ^ c16);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b_off[j][s] = T::A_BYTES + b_slot(16 * ch + 4 * g + s) * T::B_ROW + 4 * T::NB * c16;
    }

    f32x4 acc[T::NB];
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    typedef float bvec __attribute__((ext_vector_type(T::NB)));
    for (int r = 0; r < T::NS - 1 && r < rounds; ++r) issue(r);
    for (int r = 0; r < rounds; ++r) {
        wait_steps<T::LOADS, T::NS - 2>(rounds - 1 - r);
        __syncthreads();  // round r in LDS; every wave done with the stage issue overwrites
        if (r + T::NS - 1 < rounds) issue(r + T::NS - 1);
        const lds_char *st = (const lds_char *)lds + (r % T::NS) * T::STAGE;
#pragma unroll
        for (int j = 0; j < T::CHUNKS; ++j) {
            const f32x4 a = *(const __attribute__((address_space(3))) f32x4 *)(st + a_off[j]);
            bvec b[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) b[s] = *(const __attribute__((address_space(3))) bvec *)(st + b_off[j][s]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int nb = 0; nb < T::NB; ++nb) {
                    acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s][nb], acc[nb], 0, 0, 0);
                }
        }
    }

    // the waves' sums: waves 1 .. W - 1 to LDS, wave 0 adds them in wave order
    __syncthreads();  // every wave is done with the ring
    f32x4 *part = (f32x4 *)lds;
    if (w > 0) {
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) part[((w - 1) * T::NB + nb) * 64 + lane] = acc[nb];
    }
    __syncthreads();
    if (w > 0) return;  // no barrier follows
#pragma unroll  // all reads first, then the adds in wave order
    for (int v = 1; v < T::W; ++v)
#pragma unroll
        for (int nb = 0; nb < T::NB; ++nb) acc[nb] += part[((v - 1) * T::NB + nb) * 64 + lane];
    // accumulator layout of v_mfma_f32_16x16x4_f32: lane l, register q holds row
    // 4 (l / 16) + q, column l % 16 of the block, i.e. column n0 + NB (l % 16) + nb of C
#pragma unroll
    for (int nb = 0; nb < T::NB; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = m0 + 4 * g + q, jc = n0 + T::NB * c16 + nb;
            if (i < p.M && jc < p.N) p.C[(int64_t)i * p.ldc + jc] = acc[nb][q];
        }
}

template <class T>
hipError_t launch_narrow(const GemmArgs &a, hipStream_t stream)
{
    const int64_t tiles = ((a.M + 15) / 16) * ((a.N + 16 * T::NB - 1) / (16 * T::NB));
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    GemmArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_narrow_kernel<T>), dim3(gx, gy, (unsigned)a.batch),
                           dim3(T::NT), args, 0, stream);
}

}  // namespace

bool gemm_narrow_ok(const GemmArgs &a)
{
    const int kr = a.N > 32 ? 128 : 256;
    return a.N >= 1 && a.N <= 64 && a.N % 4 == 0 && a.K >= kr && a.K % kr == 0;
}

// Shapes it does not take run the 16-row kernel (config 8's).
hipError_t gemm_narrow_launch(const GemmArgs &a, hipStream_t stream)
{
    if (!gemm_narrow_ok(a)) return gemm_skinny_launch<16, 4>(a, stream);
    if (a.N <= 16) return launch_narrow<NarrowTile<1, 16, 256, 4>>(a, stream);
    if (a.N <= 32) return launch_narrow<NarrowTile<2, 16, 256, 3>>(a, stream);
    return launch_narrow<NarrowTile<4, 8, 128, 4>>(a, stream);
}

}  // namespace mm
