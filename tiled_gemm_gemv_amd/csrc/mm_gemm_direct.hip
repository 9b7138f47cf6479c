// mm_gemm_direct.hip -- fp32 GEMM C = A x B with panels moved from HBM straight into
// LDS: the tiled product of mm_gemm_tile.h ("Matrix Operations", docs.vulkan.org
// ML-inference tutorial, "Tiled Implementation with Shared Memory"; "CUDA Programming
// (6)", sections 3.2-3.3) with the staging step done by gfx950's LDS DMA.
//
// global_load_lds_dword{,x4} writes each lane's 4 or 16 bytes to LDS at M0 + 4 * lane or
// M0 + 16 * lane without passing through registers. The waves then never write LDS
// themselves (except to clear a partial last K-step), so the end of a K-step is only a
// wait and a barrier, and no registers hold staged data: the ring runs NS = 2, 4 or 8
// stages deep, step kt + NS - 1 loading while step kt is multiplied (the 256 x 256 tile
// takes K-steps of 32 in two 64 KB stages when K % 32 == 0, else of 16 in four; the
// others take K-steps of 32 in half their stages when the lean build applies and
// K % 32 == 0, else of 16). The stage layout, the k order and the MFMA step are in
// mm_direct.h.
//   * Load width. A lane's bytes land at a fixed place, so each lane fetches the
//     element(s) the permutations put there, and 4- and 16-byte lanes build the same
//     LDS image. Full K-steps load A with 16-byte lanes whatever its alignment (gfx950
//     serves 16-byte loads from any 4-byte-aligned address, also into LDS; a full step's
//     chunks never cross a row end). B takes 16-byte lanes too: with N >= BN the last
//     tile column's B panel starts at N - BN, so that no chunk crosses the row end (its
//     columns left of its own origin belong to the tile before and are not stored again:
//     each C element is written once). Only with N < BN and N % 4 != 0 does B take 4-byte
//     lanes.
//   * Edges: rows past M and columns past N are clamped to in-range data that only feeds
//     C elements that are not stored. A partial last K-step (K % 16 != 0) loads both
//     panels with 4-byte lanes at k clamped to K - 1, then the workgroup writes zeros
//     over the k >= K entries of both panels between two barriers.
//   * Addressing. Lean builds (K % 16 == 0, N % 4 == 0 or N >= BN, leading dimensions
//     that keep the offsets below 2^32) take the load's scalar-base form: the tile's corner at the
//     K-step in scalar registers plus a byte offset per lane fixed for the whole K loop,
//     so a load needs no vector instruction. General builds keep a 64-bit pointer per
//     lane.
//   * One barrier per K-step, after an explicit s_waitcnt vmcnt that counts the loads of
//     the steps issued after it (a partial last step issues more loads than a full one,
//     which only makes that count conservative). The loads are issued from inline asm
//     (M0 set there): the compiler cannot tell the stages apart and would otherwise wait
//     for every load in flight before each LDS read, which removes the pipeline. No
//     other code in these kernels uses M0.
#include "mm_direct.h"

namespace mm {
namespace {

// SB: address the 16-byte lanes of full K-steps from a scalar base (the host checked that
// the per-lane offsets fit 32 bits; lean builds always do).
// ADD: add the tile into C atomically instead of storing it (gemm_direct64_add_launch).
template <class T, bool SB, bool ADD>
__global__ __launch_bounds__(T::NT) void gemm_f32_direct_kernel(GemmArgs p)
{
    constexpr bool SADDR = !T::GEN || SB;
    __shared__ __attribute__((aligned(1024))) char lds[T::NS * T::STAGE];
    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block((int)bid, (int)tiles, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    // origin of the B panel: n0, or N - BN for a last tile column that would cross N (its
    // columns left of n0 belong to the tile before and are not stored)
    const int nb0 = p.N >= T::BN ? min(n0, p.N - T::BN) : n0;
    // problem of a strided batch: grid layer blockIdx.z
    p.A += blockIdx.z * p.sa;
    p.B += blockIdx.z * p.sb;
    p.C += blockIdx.z * p.sc;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, in a scalar register
    // the wave's place in the tile's wave grid, and its group of each K-step's k (KS = 2)
    const int wg = T::KS == 1 ? w : w % T::GRID, kg = T::KS == 1 ? 0 : w / T::GRID;
    const int wm0 = (wg / (T::BN / T::WN)) * T::WM, wn0 = (wg % (T::BN / T::WN)) * T::WN;
    const int nk = (p.K + T::BK - 1) / T::BK;

    // The 16-byte lanes of full K-steps are addressed from the tile's corner at the K-step
    // (a scalar base) plus a fixed byte offset per lane; direct_f32_offsets_fit keeps those
    // offsets below 2^32. (B's are used only by tiles whose chunks all take 16-byte lanes:
    // with N >= BN every chunk lies inside B's rows, else N % 4 == 0 and chunks past N are
    // clamped to the last one, min(col, N - 4) >= nb0.)
    unsigned aoff[T::A16], boff[T::B16];
    if constexpr (SADDR) {
#pragma unroll
        for (int i = 0; i < T::A16; ++i) {
            const int o = (T::A16 * w + i) * 1024 + 16 * lane;
            const int row = o / T::A_ROW, chunk = (o % T::A_ROW) / 16;
            aoff[i] = (unsigned)(((int64_t)(min(m0 + row, p.M - 1) - m0) * p.lda + 4 * (chunk ^ swz_a<T>(row))) * 4);
        }
#pragma unroll
        for (int i = 0; i < T::B16; ++i) {
            const int o = (T::B16 * w + i) * 1024 + 16 * lane;
            const int krow = o / T::B_ROW, chunk = (o % T::B_ROW) / 16;
            const int col = nb0 + 4 * (chunk ^ swz_b<T>(krow));
            boff[i] = (unsigned)(((int64_t)krow * p.ldb + (min(col, p.N - 4) - nb0)) * 4);
        }
    }

    // Without the scalar base: each load's lane lands at a fixed panel byte; the
    // element(s) stored there are this lane's source. 16-byte lanes of full K-steps:
    // asrc/bsrc address them at k0 = 0 (unused, and dropped by the compiler, with it).
    const float *asrc[T::A16];
    const float *bsrc[T::B16];
#pragma unroll
    for (int i = 0; i < T::A16; ++i) {
        const int o = (T::A16 * w + i) * 1024 + 16 * lane;  // panel byte
        const int row = o / T::A_ROW, chunk = (o % T::A_ROW) / 16;
        asrc[i] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + 4 * (chunk ^ swz_a<T>(row));
    }
    // B chunks stay inside their row when N % 4 == 0 (clamped to the last chunk) or when
    // the panel starts at least BN columns before N
    const bool wide_b = !T::GEN || (p.N % 4 == 0) || (p.N >= T::BN);
#pragma unroll
    for (int i = 0; i < T::B16; ++i) {
        const int o = (T::B16 * w + i) * 1024 + 16 * lane;
        const int krow = o / T::B_ROW, chunk = (o % T::B_ROW) / 16;
        const int col = nb0 + 4 * (chunk ^ swz_b<T>(krow));
        bsrc[i] = p.B + (int64_t)krow * p.ldb + max(min(col, p.N - 4), 0);
    }
    // 4-byte lanes: source of load i at K-step k0, k clamped to K - 1 (partial step)
    auto a4_src = [&](int i, int k0) {
        const int o = (T::A4 * w + i) * 256 + 4 * lane;
        const int row = o / T::A_ROW, slot = (o % T::A_ROW) / 4;
        const int k = min(k0 + 4 * ((slot >> 2) ^ swz_a<T>(row)) + (slot & 3), p.K - 1);
        return p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + k;
    };
    auto b4_src = [&](int i, int k0) {
        const int o = (T::B4 * w + i) * 256 + 4 * lane;
        const int krow = o / T::B_ROW, slot = (o % T::B_ROW) / 4;
        const int col = nb0 + 4 * ((slot >> 2) ^ swz_b<T>(krow)) + (slot & 3);
        return p.B + (int64_t)min(k0 + krow, p.K - 1) * p.ldb + min(col, p.N - 1);
    };
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_char *)lds;  // LDS byte offset of the array
    const int nk_full = p.K / T::BK;  // full K-steps; a partial one follows if K % 16 != 0

    DirectOffsets<T> off;
    direct_offsets<T>(lane, wm0, wn0, off, kg * T::QW);

    typename T::Acc acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < T::ACC; ++r) acc[i][jj][r] = 0.f;

    auto multiply = [&](int kt) { direct_mma<T>((const lds_char *)lds + (kt % T::NS) * T::STAGE, off, acc); };

    // The K loop, compiled once per kind of tile (16- or 4-byte B lanes), so that a K-step
    // tests nothing but whether it has a step to issue.
    auto k_loop = [&](auto wide_tag) {
        constexpr bool WIDE = decltype(wide_tag)::value;
        constexpr int L = WIDE ? T::LOADS_WIDE : T::LOADS_NARROW_B;
        auto issue_full = [&](int kt) {
            const unsigned st = lds0 + (kt % T::NS) * T::STAGE;
            const int k0 = kt * T::BK;
            if constexpr (SADDR) {
                const float *abase = p.A + (int64_t)m0 * p.lda + k0;
#pragma unroll
                for (int i = 0; i < T::A16; ++i) load_to_lds_s16(st + (T::A16 * w + i) * 1024, abase, aoff[i]);
            } else {
#pragma unroll
                for (int i = 0; i < T::A16; ++i) load_to_lds<16>(st + (T::A16 * w + i) * 1024, asrc[i] + k0);
            }
            if constexpr (WIDE && SADDR) {
                const float *bbase = p.B + (int64_t)k0 * p.ldb + nb0;
#pragma unroll
                for (int i = 0; i < T::B16; ++i)
                    load_to_lds_s16(st + T::A_BYTES + (T::B16 * w + i) * 1024, bbase, boff[i]);
            } else if constexpr (WIDE) {
#pragma unroll
                for (int i = 0; i < T::B16; ++i)
                    load_to_lds<16>(st + T::A_BYTES + (T::B16 * w + i) * 1024, bsrc[i] + (int64_t)k0 * p.ldb);
            } else {
#pragma unroll
                for (int i = 0; i < T::B4; ++i)
                    load_to_lds<4>(st + T::A_BYTES + (T::B4 * w + i) * 256, b4_src(i, k0));
            }
        };
        // the partial last step: 4-byte lanes, k clamped (cleared after it lands)
        auto issue_partial = [&](int kt) {
            if constexpr (T::GEN) {
                const unsigned st = lds0 + (kt % T::NS) * T::STAGE;
                const int k0 = kt * T::BK;
#pragma unroll
                for (int i = 0; i < T::A4; ++i) load_to_lds<4>(st + (T::A4 * w + i) * 256, a4_src(i, k0));
#pragma unroll
                for (int i = 0; i < T::B4; ++i)
                    load_to_lds<4>(st + T::A_BYTES + (T::B4 * w + i) * 256, b4_src(i, k0));
            }
        };
        auto issue = [&](int kt) {
            if (kt < nk_full) issue_full(kt);
            else if (T::GEN && kt < nk) issue_partial(kt);
        };
        for (int s = 0; s < T::NS - 1; ++s) issue(s);
        for (int kt = 0; kt < nk_full; ++kt) {
            // step kt's loads are done when at most the later steps' loads are outstanding
            // (a partial step among them issues more than L: the count is then conservative)
            wait_steps<L, T::NS - 2>(nk - 1 - kt);
            // every wave's loads for stage kt are in LDS, and every wave is done with the
            // stage the next issue overwrites (read in step kt - 1)
            __syncthreads();
            const int next = kt + T::NS - 1;
            if (next < nk_full) issue_full(next);
            else if (T::GEN && next < nk) issue_partial(next);
            multiply(kt);
        }
        if (T::GEN && nk_full < nk) {
            wait_vmcnt<0>();
            __syncthreads();
            // zeros over k >= K in both panels (no load is in flight into this stage and
            // no wave reads it before the barrier below)
            lds_char *st = (lds_char *)lds + (nk_full % T::NS) * T::STAGE;
            const int kr = p.K - nk_full * T::BK, nz = T::BK - kr;
            for (int e = threadIdx.x; e < T::BM * nz; e += T::NT) {
                const int r = e / nz, k = kr + e % nz;
                *(lds_float *)(st + r * T::A_ROW + 16 * ((k >> 2) ^ swz_a<T>(r)) + 4 * (k & 3)) = 0.f;
            }
            for (int e = threadIdx.x; e < nz * T::BN; e += T::NT)
                *(lds_float *)(st + T::A_BYTES + (kr + e / T::BN) * T::B_ROW + 4 * (e % T::BN)) = 0.f;
            __syncthreads();
            multiply(nk_full);
        }
    };
    if (!T::GEN || wide_b) k_loop(std::true_type{});
    else k_loop(std::false_type{});

    if constexpr (T::KS == 2) {
        // group 1's sums to LDS (lane-minor: conflict-free), group 0 adds them to its own
        __syncthreads();  // every wave is done with the stages
        lds_float *x = (lds_float *)lds + wg * (T::FM * T::FN * 16 * 64) + lane;
        static_assert(T::GRID * T::FM * T::FN * 16 * 64 * 4 <= T::NS * T::STAGE, "the sums fit the ring");
        if (kg == 1) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[((i * T::FN + jj) * 16 + r) * 64] = acc[i][jj][r];
        }
        __syncthreads();
        if (kg == 1) return;  // no barrier follows
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jj][r] += x[((i * T::FN + jj) * 16 + r) * 64];
    }

    if constexpr (ADD) direct_store_add<T>(p, m0, nb0, n0, wm0, wn0, lane, acc);
    else direct_store<T>(p, m0, nb0, n0, wm0, wn0, lane, acc, [](int gn) { return gn; });
}

template <class T, bool SB = true, bool ADD = false>
hipError_t launch_direct(const GemmArgs &a, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    GemmArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_f32_direct_kernel<T, SB, ADD>),
                           dim3(gx, gy, (unsigned)a.batch), dim3(T::NT), args, 0, stream);
}

}  // namespace

// The per-lane byte offsets from a tile's corner (below 256 rows of A, 32 rows of B and
// 256 columns) fit 32 bits.
static bool direct_f32_offsets_fit(const GemmArgs &a)
{
    constexpr int64_t kOffMax = int64_t(1) << 32;
    return 4 * (255 * a.lda + 32) < kOffMax && 4 * (31 * a.ldb + 256) < kOffMax;
}

bool direct_f32_wide_ok(const GemmArgs &a, int bn)
{
    return a.K % 16 == 0 && a.N >= 4 && (a.N % 4 == 0 || a.N >= bn) && direct_f32_offsets_fit(a);
}

namespace {

// The kernel without the partial-step and narrow-lane code where the shape allows it: its
// K loop is leaner (measured up to 20% faster on the 64 x 64 tile, whose waves issue only
// 8 MFMAs per K-step). Where K % 32 == 0 too, K-steps of 32 in half as many stages (the
// same LDS): whole 128-byte A lines and twice the MFMAs per barrier, 1-8% faster on the
// 128 x 128 and 64 x 64 tiles.
template <int BM, int BN, int WM, int WN, int NS, bool ADD = false, bool M16 = false>
hipError_t launch_lean_or_general(const GemmArgs &a, hipStream_t stream)
{
    if (direct_f32_wide_ok(a, BN) && a.K % 32 == 0)
        return launch_direct<DirectF32<BM, BN, WM, WN, NS / 2, false, 32, 1, M16>, true, ADD>(a, stream);
    if (direct_f32_wide_ok(a, BN))
        return launch_direct<DirectF32<BM, BN, WM, WN, NS, false, 16, 1, M16>, true, ADD>(a, stream);
    return direct_f32_offsets_fit(a) ? launch_direct<DirectF32<BM, BN, WM, WN, NS, true, 16, 1, M16>, true, ADD>(a, stream)
                                     : launch_direct<DirectF32<BM, BN, WM, WN, NS, true, 16, 1, M16>, false, ADD>(a, stream);
}

}  // namespace

hipError_t gemm_direct_launch(DirectTile t, const GemmArgs &a, hipStream_t stream)
{
    switch (t) {
    case DirectTile::T256:
        // K-steps of 32 (two 64 KB stages) where K allows, else of 16 (four 32 KB stages)
        if (!direct_f32_wide_ok(a, 256)) return hipErrorInvalidValue;
        if (a.K % 32 == 0) return launch_direct<DirectF32<256, 256, 128, 64, 2, false, 32>>(a, stream);
        return launch_direct<DirectF32<256, 256, 128, 64, 4, false>>(a, stream);
    case DirectTile::T128:
        return launch_lean_or_general<128, 128, 64, 64, 4>(a, stream);
    case DirectTile::T128M16:
        return launch_lean_or_general<128, 128, 64, 64, 4, false, true>(a, stream);
    case DirectTile::T64S8:
        return launch_lean_or_general<64, 64, 32, 32, 8>(a, stream);
    case DirectTile::T64S4:
        return launch_lean_or_general<64, 64, 32, 32, 4>(a, stream);
    case DirectTile::T64K2:
        // each K-step's k split over two groups of 4 waves (two waves per SIMD where a CU
        // holds one tile); other shapes run the T64S4 kernel
        if (direct_f32_wide_ok(a, 64) && a.K % 32 == 0)
            return launch_direct<DirectF32<64, 64, 32, 32, 4, false, 32, 2>>(a, stream);
        return launch_lean_or_general<64, 64, 32, 32, 4>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_direct64_add_launch(const GemmArgs &a, hipStream_t stream)
{
    if (direct_f32_wide_ok(a, 64) && a.K % 32 == 0)
        return launch_direct<DirectF32<64, 64, 32, 32, 4, false, 32, 2>, true, true>(a, stream);
    return launch_lean_or_general<64, 64, 32, 32, 4, true>(a, stream);
}

}  // namespace mm
