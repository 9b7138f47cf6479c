// mm_gemm.hip -- fp32 GEMM C = A x B on the gfx950 matrix cores.
//
// The method is the shared-memory tiled product ("Matrix Operations",
// docs.vulkan.org ML-inference tutorial, "Tiled Implementation with Shared
// Memory"; "CUDA Programming (6)", sections 3.2-3.3; "GPU Matrix
// Multiplication: Tiling and Shared Memory", section 3): each workgroup owns one
// tile of C, walks the K dimension in steps, stages the matching panels of A and
// B in on-chip memory (here the LDS), and accumulates partial dot products in
// registers. Out-of-range elements are staged as zeros and only in-range C is
// written (the pages' boundary handling). Beyond the pages' version, sized for
// CDNA4:
//   * macro-tiles up to 256 x 256 per workgroup, each wave owning a 128 x 64 (or
//     smaller) register-blocked sub-tile (the pages' register blocking);
//   * the inner product runs on v_mfma_f32_32x32x2_f32 (fp32 in, fp32 out);
//   * two LDS stages (the pages' prefetching, with the second buffer that makes
//     it race-free): the next K-step is read from HBM into registers while the
//     current one is multiplied, then written to the other stage; one barrier
//     per K-step;
//   * 16-byte global loads and 16-byte LDS reads/writes when rows are 16-byte
//     aligned (the pages' vectorisation), 4-byte loads otherwise;
//   * the workgroup -> tile map undoes the round-robin dealing of workgroups to
//     the 8 XCDs, so neighbouring tiles share an L2.
//
// LDS layout per stage: A panel as BM rows of BK k-values, B panel transposed as
// BN rows of BK k-values, both with a row pitch of BK + 4 floats. With k
// contiguous, every MFMA operand is a 16-byte LDS read; the 4-float pad spreads
// the 32 rows a wave reads at once over distinct banks.
//
// k order inside a K-step. v_mfma_f32_32x32x2_f32 multiplies a 32 x 2 slice of A
// by a 2 x 32 slice of B: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32].
// Lanes 0-31 feed k = s and lanes 32-63 feed k = BK/2 + s at MFMA step s, so over
// the BK/2 steps each k in the K-step is added exactly once and each lane's
// operands for four steps sit in one 16-byte LDS word. The sum is the same sum in
// a different order.
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;  // MI355X deals consecutive workgroups to 8 XCDs in turn

template <int BM_, int BN_, int BK_, int WM_, int WN_, int GROUP_M_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int GROUP_M = GROUP_M_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;  // 32 x 32 accumulator blocks per wave
    static constexpr int PITCH = BK + 4;               // LDS row pitch, floats
    static constexpr int A_TILE = BM * PITCH;
    static constexpr int B_TILE = BN * PITCH;
    static constexpr int STAGE = A_TILE + B_TILE;      // floats per LDS stage
    static constexpr int KQ = BK / 4;                  // 4-float groups along k
    static constexpr int A_CHUNKS = BM * KQ;           // 16-byte pieces of an A panel
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_BLOCKS = KQ * (BN / 4);     // 4 x 4 pieces of a B panel
    static constexpr int B_PER_T = (B_BLOCKS + NT - 1) / NT;
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(BK % 8 == 0, "BK must be a multiple of 8");
    static_assert(2 * STAGE * 4 <= 160 * 1024, "two stages must fit the 160 KB LDS");
};

// 4 consecutive floats at p (in range).
template <bool VEC>
__device__ __forceinline__ f32x4 load4(const float *p)
{
    if constexpr (VEC) {
        return *reinterpret_cast<const f32x4 *>(p);
    } else {
        return f32x4{p[0], p[1], p[2], p[3]};
    }
}

// The first `valid` of 4 consecutive floats at p, zeros for the rest (valid may
// be <= 0 or >= 4). Nothing outside the valid range is read.
template <bool VEC>
__device__ __forceinline__ f32x4 load4_masked(const float *p, int valid)
{
    if (valid >= 4) return load4<VEC>(p);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid > 0) v[0] = p[0];
    if (valid > 1) v[1] = p[1];
    if (valid > 2) v[2] = p[2];
    return v;
}

// Launch index -> (tile row, tile column) of C.
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n,
                                              int group_m, int &tm, int &tn)
{
    // Workgroup bid runs on XCD bid % 8. Renumber so that each XCD receives one
    // contiguous run of logical tiles (a bijection for any nblocks).
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    const int logical = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
    // Within a run, walk group_m tile rows at a time, column by column, so that
    // workgroups running together share rows of A and columns of B.
    const int per_group = group_m * tiles_n;
    const int g = logical / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * per_group;
    tm = first_m + in_g % gm;
    tn = in_g / gm;
}

template <class T, bool VEC_A, bool VEC_B>
__global__ __launch_bounds__(T::NT) void gemm_f32_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];

    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, T::GROUP_M, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / T::WAVES_N) * T::WM;
    const int wn0 = (wave % T::WAVES_N) * T::WN;
    const bool inner_mn = (m0 + T::BM <= p.M) && (n0 + T::BN <= p.N);
    const int nk = (p.K + T::BK - 1) / T::BK;

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    f32x4 ra[T::A_PER_T];     // staged A: one 16-byte piece of a row each
    f32x4 rb[T::B_PER_T][4];  // staged B: 4 k-rows x 4 columns each

    // HBM -> registers for K-step kt. Piece c of thread tid is index tid + c * NT.
    // A piece: row idx / KQ, k-group idx % KQ (a row's pieces are adjacent lanes).
    // B piece: k-group idx % KQ, column group idx / KQ.
    auto global_load = [&](int kt) {
        const int k0 = kt * T::BK;
        const bool full = inner_mn && (k0 + T::BK <= p.K);
#pragma unroll
        for (int c = 0; c < T::A_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::A_CHUNKS % T::NT == 0 || idx < T::A_CHUNKS) {
                const int row = idx / T::KQ, kg = idx % T::KQ;
                const int gm = m0 + row, gk = k0 + 4 * kg;
                if (full) {
                    ra[c] = load4<VEC_A>(p.A + (int64_t)gm * p.lda + gk);
                } else {
                    const int valid = (gm < p.M) ? p.K - gk : 0;
                    ra[c] = load4_masked<VEC_A>(p.A + (int64_t)gm * p.lda + gk, valid);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < T::B_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::B_BLOCKS % T::NT == 0 || idx < T::B_BLOCKS) {
                const int kg = idx % T::KQ, ng = idx / T::KQ;
                const int gn = n0 + 4 * ng;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int gk = k0 + 4 * kg + r;
                    if (full) {
                        rb[c][r] = load4<VEC_B>(p.B + (int64_t)gk * p.ldb + gn);
                    } else {
                        const int valid = (gk < p.K) ? p.N - gn : 0;
                        rb[c][r] = load4_masked<VEC_B>(p.B + (int64_t)gk * p.ldb + gn, valid);
                    }
                }
            }
        }
    };

    // registers -> LDS stage `buf` (B transposed on the way in).
    auto lds_store = [&](int buf) {
        float *As = lds + buf * T::STAGE;
        float *Bs = As + T::A_TILE;
#pragma unroll
        for (int c = 0; c < T::A_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::A_CHUNKS % T::NT == 0 || idx < T::A_CHUNKS) {
                const int row = idx / T::KQ, kg = idx % T::KQ;
                *reinterpret_cast<f32x4 *>(As + row * T::PITCH + 4 * kg) = ra[c];
            }
        }
#pragma unroll
        for (int c = 0; c < T::B_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::B_BLOCKS % T::NT == 0 || idx < T::B_BLOCKS) {
                const int kg = idx % T::KQ, ng = idx / T::KQ;
#pragma unroll
                for (int col = 0; col < 4; ++col) {
                    const f32x4 v = {rb[c][0][col], rb[c][1][col], rb[c][2][col], rb[c][3][col]};
                    *reinterpret_cast<f32x4 *>(Bs + (4 * ng + col) * T::PITCH + 4 * kg) = v;
                }
            }
        }
    };

    // One K-step on LDS stage `buf`.
    auto multiply = [&](int buf) {
        const int half = (lane >> 5) * (T::BK / 2);
        const float *As = lds + buf * T::STAGE + (wm0 + (lane & 31)) * T::PITCH + half;
        const float *Bs = lds + buf * T::STAGE + T::A_TILE + (wn0 + (lane & 31)) * T::PITCH + half;
#pragma unroll
        for (int q = 0; q < T::BK / 8; ++q) {
            f32x4 a[T::FM], b[T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                a[i] = *reinterpret_cast<const f32x4 *>(As + i * 32 * T::PITCH + 4 * q);
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                b[j] = *reinterpret_cast<const f32x4 *>(Bs + j * 32 * T::PITCH + 4 * q);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
#pragma unroll
                    for (int j = 0; j < T::FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s],
                                                                         acc[i][j], 0, 0, 0);
        }
    };

    if (nk > 0) {
        global_load(0);
        lds_store(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) global_load(kt + 1);
        multiply(cur);
        // The other stage was last read in step kt - 1, which every wave finished
        // before the barrier that ended that step.
        if (kt + 1 < nk) lds_store(cur ^ 1);
        __syncthreads();
    }

    // Accumulator block layout of v_mfma_f32_32x32x2_f32: lane l, register r holds
    // row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32 of the 32 x 32 block.
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                const int gn = n0 + wn0 + j * 32 + col_l;
                if (inner_mn || (gm < p.M && gn < p.N))
                    p.C[(int64_t)gm * p.ldc + gn] = acc[i][j][r];
            }
}

template <class T>
hipError_t launch_tile(const GemmArgs &a, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool va = (a.lda % 4 == 0) && ((uintptr_t)a.A % 16 == 0);
    const bool vb = (a.ldb % 4 == 0) && ((uintptr_t)a.B % 16 == 0);
    const void *fn;
    if (va && vb)
        fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, true, true>);
    else if (va)
        fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, true, false>);
    else if (vb)
        fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, false, true>);
    else
        fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, false, false>);
    GemmArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(fn, dim3((unsigned)tiles), dim3(T::NT), args, 0, stream);
}

using TileL = Tile<256, 256, 32, 128, 64, 8>;
using TileM = Tile<128, 128, 32, 64, 64, 8>;
using TileS = Tile<64, 64, 32, 32, 32, 8>;

struct ConfigEntry {
    const char *name;
    hipError_t (*launch)(const GemmArgs &, hipStream_t);
    int bm, bn;
};

const ConfigEntry kConfigs[] = {
    {"256x256x32 w128x64 (8 waves)", &launch_tile<TileL>, 256, 256},
    {"128x128x32 w64x64 (4 waves)", &launch_tile<TileM>, 128, 128},
    {"64x64x32 w32x32 (4 waves)", &launch_tile<TileS>, 64, 64},
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

int64_t tiles_for(int cfg, int64_t M, int64_t N)
{
    const ConfigEntry &c = kConfigs[cfg];
    return ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
}

}  // namespace

int gemm_num_configs() { return kNumConfigs; }

const char *gemm_config_name(int cfg)
{
    return (cfg >= 0 && cfg < kNumConfigs) ? kConfigs[cfg].name : nullptr;
}

// Largest tile that still gives every one of the 256 CUs work: a big tile reuses
// each staged element more often, a small one fills the chip on small shapes.
int gemm_select_config(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    if (tiles_for(0, M, N) >= 512) return 0;
    if (tiles_for(1, M, N) >= 256) return 1;
    return 2;
}

hipError_t gemm_launch(int cfg, const GemmArgs &a, hipStream_t stream)
{
    return kConfigs[cfg].launch(a, stream);
}

}  // namespace mm
