// mm_gemm_tile.h -- the tiled fp32 matrix-core kernel behind the GEMM (mm_gemm.hip)
// and the implicit-GEMM convolution (mm_conv.hip). Internal to libmm.
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
//
// An operand policy Ops says where the B panel comes from and where C goes:
// DenseOperands (below) reads B as a matrix; the convolution gathers B from the
// input image on the fly (mm_conv.hip).
#pragma once

#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kXcds = 8;  // MI355X deals consecutive workgroups to 8 XCDs in turn

// PF_: how many K-steps ahead the HBM loads run (1 or 2). With 2, a second set of
// staging registers lets a request overlap two K-steps of MFMAs instead of one.
// KS_: waves that share each WM x WN output block. Each takes 1/KS of every K-step's
// k range; at the end the partial sums meet in LDS and are added in a fixed order.
// It puts more waves on each SIMD when C has few tiles, with no memory beyond C.
// MID_ (PF = 1): write the next K-step's staged data to LDS halfway through the
// current step's MFMAs rather than after them, so the wait for those loads and the
// LDS writes overlap matrix work. Off where the registers are already full (the
// fragments of both halves and the staged data are then live together).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int GROUP_M_, int PF_ = 1, int KS_ = 1,
          bool MID_ = true>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int GROUP_M = GROUP_M_, PF = PF_, KS = KS_;
    static constexpr bool MID = MID_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int WAVES_MN = WAVES_M * WAVES_N;
    static constexpr int NT = WAVES_MN * KS * 64;
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
    static_assert(PF == 1 || PF == 2, "prefetch depth 1 or 2");
    static_assert((BK / 8) % KS == 0, "each k share must be whole 4-step groups");
    static_assert(KS == 1 || (KS - 1) * BM * BN <= 2 * STAGE, "partial sums must fit the LDS");
    static_assert(NT <= 1024, "at most 1024 threads per workgroup");
    // One K-step's worth of a thread's staged HBM data.
    struct Staged {
        f32x4 a[A_PER_T];     // one 16-byte piece of an A row each
        f32x4 b[B_PER_T][4];  // 4 k-rows x 4 columns of B each
    };
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

// Operand policies. A policy says where the B panel comes from and where C goes:
//   Cols columns<T>(p, n0, idx)       state of B piece idx's columns, fixed over K;
//   load_b<T, VEC>(p, cols, k0, n0, idx, full, b)
//                                     HBM -> registers: piece idx of the K-step at k0
//                                     (16 elements, zeros outside the operand);
//   store_b<T>(Bs, idx, b)            registers -> the LDS panel (BN rows of BK
//                                     k-values, row pitch PITCH);
//   int64_t c_column(p, gn)           offset of C's column gn (C[m][n] at
//                                     C + c_column(n) + m * ldc).
// Pieces idx cover the BK x BN panel exactly once between them.

// The plain product: B is a K x N matrix with row stride ldb, and C element (m, n)
// is at C + m * ldc + n. Piece idx is the 4 x 4 block at k-group idx % KQ, column
// group idx / KQ, so the lanes of a wave read 8 rows x 128 contiguous bytes each.
struct DenseOperands {
    static constexpr bool kMatrixB = true;
    struct Cols {};
    template <class T>
    __device__ Cols columns(const GemmArgs &, int, int) const { return {}; }
    template <class T, bool VEC>
    __device__ __forceinline__ void load_b(const GemmArgs &p, const Cols &, int k0, int n0, int idx,
                                           bool full, f32x4 (&b)[4]) const
    {
        const int gk = k0 + 4 * (idx % T::KQ), gn = n0 + 4 * (idx / T::KQ);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float *src = p.B + (int64_t)(gk + r) * p.ldb + gn;
            if (full) {
                b[r] = load4<VEC>(src);
            } else {
                const int valid = (gk + r < p.K) ? p.N - gn : 0;
                b[r] = load4_masked<VEC>(src, valid);
            }
        }
    }
    // b[r] is k-row r of 4 columns: transposed on the way into LDS
    template <class T>
    __device__ __forceinline__ void store_b(float *Bs, int idx, const f32x4 (&b)[4]) const
    {
        const int kg = idx % T::KQ, ng = idx / T::KQ;
#pragma unroll
        for (int col = 0; col < 4; ++col) {
            const f32x4 v = {b[0][col], b[1][col], b[2][col], b[3][col]};
            *reinterpret_cast<f32x4 *>(Bs + (4 * ng + col) * T::PITCH + 4 * kg) = v;
        }
    }
    __device__ int64_t c_column(const GemmArgs &, int gn) const { return gn; }
};

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

template <class T, bool VEC_A, bool VEC_B, class Ops>
__global__ __launch_bounds__(T::NT) void gemm_f32_kernel(GemmArgs p, Ops ops)
{
    __shared__ __attribute__((aligned(16))) float lds[2 * T::STAGE];

    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block((int)bid, (int)tiles, tiles_m, tiles_n, T::GROUP_M, tm, tn);

    // problem of a strided batch: grid layer blockIdx.z
    p.A += blockIdx.z * p.sa;
    p.B += blockIdx.z * p.sb;
    p.C += blockIdx.z * p.sc;
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ks = wave / T::WAVES_MN;              // which share of each K-step
    const int wmn = wave % T::WAVES_MN;             // which output block
    const int wm0 = (wmn / T::WAVES_N) * T::WM;
    const int wn0 = (wmn % T::WAVES_N) * T::WN;
    const bool inner_mn = (m0 + T::BM <= p.M) && (n0 + T::BN <= p.N);
    const int nk = (p.K + T::BK - 1) / T::BK;

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // What the B source needs to know about the columns of each B piece this thread
    // stages (the same columns in every K-step).
    typename Ops::Cols cols[T::B_PER_T];
#pragma unroll
    for (int c = 0; c < T::B_PER_T; ++c) cols[c] = ops.template columns<T>(p, n0, tid + c * T::NT);

    typename T::Staged r0, r1;

    // HBM -> registers for K-step kt. Piece c of thread tid is index tid + c * NT.
    // A piece: row idx / KQ, k-group idx % KQ (a row's pieces are adjacent lanes).
    // B piece: 16 elements of the BK x BN panel, placed by Ops.
    auto global_load = [&](int kt, typename T::Staged &st) {
        const int k0 = kt * T::BK;
        const bool full = inner_mn && (k0 + T::BK <= p.K);
#pragma unroll
        for (int c = 0; c < T::A_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::A_CHUNKS % T::NT == 0 || idx < T::A_CHUNKS) {
                const int row = idx / T::KQ, kg = idx % T::KQ;
                const int gm = m0 + row, gk = k0 + 4 * kg;
                if (full) {
                    st.a[c] = load4<VEC_A>(p.A + (int64_t)gm * p.lda + gk);
                } else {
                    const int valid = (gm < p.M) ? p.K - gk : 0;
                    st.a[c] = load4_masked<VEC_A>(p.A + (int64_t)gm * p.lda + gk, valid);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < T::B_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::B_BLOCKS % T::NT == 0 || idx < T::B_BLOCKS)
                ops.template load_b<T, VEC_B>(p, cols[c], k0, n0, idx, full, st.b[c]);
        }
    };

    // registers -> LDS stage `buf` (B stored column by column, k contiguous).
    auto lds_store = [&](int buf, const typename T::Staged &st) {
        float *As = lds + buf * T::STAGE;
        float *Bs = As + T::A_TILE;
#pragma unroll
        for (int c = 0; c < T::A_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::A_CHUNKS % T::NT == 0 || idx < T::A_CHUNKS) {
                const int row = idx / T::KQ, kg = idx % T::KQ;
                *reinterpret_cast<f32x4 *>(As + row * T::PITCH + 4 * kg) = st.a[c];
            }
        }
#pragma unroll
        for (int c = 0; c < T::B_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::B_BLOCKS % T::NT == 0 || idx < T::B_BLOCKS) ops.template store_b<T>(Bs, idx, st.b[c]);
        }
    };

    // One K-step on LDS stage `buf`: this wave's share of its 4-step groups.
    // `mid` runs halfway through the MFMA stream (used to write the next stage).
    auto multiply = [&](int buf, auto &&mid) {
        constexpr int QS = T::BK / 8 / T::KS;
        const int half = (lane >> 5) * (T::BK / 2) + ks * QS * 4;
        const float *As = lds + buf * T::STAGE + (wm0 + (lane & 31)) * T::PITCH + half;
        const float *Bs = lds + buf * T::STAGE + T::A_TILE + (wn0 + (lane & 31)) * T::PITCH + half;
        // Fragments are double-buffered: the LDS reads of 4-step group q + 1 are
        // issued before the MFMAs of group q, so their latency hides behind MFMAs.
        f32x4 a[2][T::FM], b[2][T::FN];
        auto read_frags = [&](int q, f32x4 (&fa)[T::FM], f32x4 (&fb)[T::FN]) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                fa[i] = *reinterpret_cast<const f32x4 *>(As + i * 32 * T::PITCH + 4 * q);
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                fb[j] = *reinterpret_cast<const f32x4 *>(Bs + j * 32 * T::PITCH + 4 * q);
        };
        read_frags(0, a[0], b[0]);
#pragma unroll
        for (int q = 0; q < QS; ++q) {
            if (q + 1 < QS) read_frags(q + 1, a[(q + 1) & 1], b[(q + 1) & 1]);
            if (q == QS / 2) mid();
            // keep those reads ahead of this group's MFMAs (the scheduler would
            // otherwise sink them next to their use)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
#pragma unroll
                    for (int j = 0; j < T::FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            a[q & 1][i][s], b[q & 1][j][s], acc[i][j], 0, 0, 0);
        }
    };

    auto nothing = [] {};
    if constexpr (T::PF == 1) {
        if (nk > 0) {
            global_load(0, r0);
            lds_store(0, r0);
            __syncthreads();
        }
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) global_load(kt + 1, r0);
            // The other stage was last read in step kt - 1, which every wave
            // finished before the barrier that ended that step.
            if constexpr (T::MID) {
                multiply(cur, [&] {
                    if (kt + 1 < nk) lds_store(cur ^ 1, r0);
                });
            } else {
                multiply(cur, nothing);
                if (kt + 1 < nk) lds_store(cur ^ 1, r0);
            }
            __syncthreads();
        }
    } else {
        // Two staging buffers. At the top of an even step kt, r0 is free and r1
        // holds step kt + 1; the loads for step kt + 2 go to r0. Step kt + 1's
        // data, requested a whole K-step earlier, is written to the other LDS
        // stage halfway through step kt's MFMAs (that stage was last read in step
        // kt - 1, before the barrier that ended it), so a K-step ends with just
        // the barrier. The loop is unrolled by two so that each buffer is a fixed
        // set of registers.
        if (nk > 0) {
            global_load(0, r0);
            lds_store(0, r0);
        }
        if (nk > 1) global_load(1, r1);
        __syncthreads();
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            if (kt + 2 < nk) global_load(kt + 2, r0);
            multiply(0, [&] { lds_store(1, r1); });
            __syncthreads();
            if (kt + 3 < nk) global_load(kt + 3, r1);
            multiply(1, [&] {
                if (kt + 2 < nk) lds_store(0, r0);
            });
            __syncthreads();
        }
        if (kt < nk) multiply(0, nothing);  // odd number of K-steps: the last one is in stage 0
    }

    if constexpr (T::KS > 1) {
        // Waves of shares 1..KS-1 park their sums in LDS (reused: every wave is past
        // its last LDS read after this barrier); share 0 adds them in share order.
        constexpr int BLOCK = T::FM * T::FN * 16 * 64;  // floats per wave's sums
        __syncthreads();
        if (ks > 0) {
            float *dst = lds + ((ks - 1) * T::WAVES_MN + wmn) * BLOCK + lane;
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) dst[((i * T::FN + j) * 16 + r) * 64] = acc[i][j][r];
        }
        __syncthreads();
        if (ks > 0) return;  // no barrier follows
#pragma unroll 1
        for (int g = 1; g < T::KS; ++g) {
            const float *src = lds + ((g - 1) * T::WAVES_MN + wmn) * BLOCK + lane;
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] += src[((i * T::FN + j) * 16 + r) * 64];
        }
    }

    // Accumulator block layout of v_mfma_f32_32x32x2_f32: lane l, register r holds
    // row 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32 of the 32 x 32 block.
    // Element (m, n) of C is at C + ops.c_column(n) + m * ldc.
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
            const int gn = n0 + wn0 + j * 32 + col_l;
            const int64_t cbase = ops.c_column(p, gn);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                if (inner_mn || (gm < p.M && gn < p.N))
                    p.C[cbase + (int64_t)gm * p.ldc] = acc[i][j][r];
            }
        }
}

// Enqueue tile shape T over the whole of C with B source / C layout `ops`. 16-byte
// loads are used for A when its rows are 16-byte aligned, and for B when Ops
// reads B as a matrix (Ops::kMatrixB) whose rows are.
template <class T, class Ops>
hipError_t launch_tile_ops(const GemmArgs &a, const Ops &ops, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool va = (a.lda % 4 == 0) && ((uintptr_t)a.A % 16 == 0);
    const bool vb = Ops::kMatrixB && (a.ldb % 4 == 0) && ((uintptr_t)a.B % 16 == 0);
    const void *fn;
    if constexpr (Ops::kMatrixB) {
        if (va && vb)
            fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, true, true, Ops>);
        else if (va)
            fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, true, false, Ops>);
        else if (vb)
            fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, false, true, Ops>);
        else
            fn = reinterpret_cast<const void *>(&gemm_f32_kernel<T, false, false, Ops>);
    } else {
        fn = va ? reinterpret_cast<const void *>(&gemm_f32_kernel<T, true, false, Ops>)
                : reinterpret_cast<const void *>(&gemm_f32_kernel<T, false, false, Ops>);
    }
    (void)vb;
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    GemmArgs arg = a;
    Ops o = ops;
    void *args[] = {&arg, &o};
    return hipLaunchKernel(fn, dim3(gx, gy, (unsigned)a.batch), dim3(T::NT), args, 0, stream);
}

// The tile shapes of the fp32 GEMM (public config indices 0-5).
using T256x256k32 = Tile<256, 256, 32, 128, 64, 8, 1, 1, false>;
using T128x128k32p2 = Tile<128, 128, 32, 64, 64, 8, 2>;
using T128x128k32s2 = Tile<128, 128, 32, 64, 64, 8, 1, 2>;
using T64x64k64p2 = Tile<64, 64, 64, 32, 32, 8, 2>;
using T64x64k64p2s2 = Tile<64, 64, 64, 32, 32, 8, 2, 2>;
using T128x64k64s2 = Tile<128, 64, 64, 64, 32, 8, 1, 2>;

}  // namespace
}  // namespace mm
