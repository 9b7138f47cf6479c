// mm_gemm_direct.hip -- fp32 GEMM C = A x B with panels moved from HBM straight into
// LDS: the tiled product of mm_gemm_tile.h ("Matrix Operations", docs.vulkan.org
// ML-inference tutorial, "Tiled Implementation with Shared Memory"; "CUDA Programming
// (6)", sections 3.2-3.3) with the staging step done by gfx950's LDS DMA.
//
// global_load_lds_dword{,x4} writes each lane's 4 or 16 bytes to LDS at M0 + VEC * lane
// without passing through registers. The waves then never write LDS themselves (except
// to clear a partial last K-step), so the end of a K-step is only a wait and a barrier,
// and no registers hold staged data: the ring runs NS = 4 or 8 stages deep, step
// kt + NS - 1 loading while step kt is multiplied.
//   * BK = 16. A panel: BM rows of 64 bytes. The 16-byte chunk c of row r sits in slot
//     c ^ swz_a(r), so that a wave's reads of 32 rows at one k hit distinct banks. Each
//     lane reads 4 consecutive k of its row with one 16-byte read.
//   * B panel: 16 rows of BN floats, row-major. v_mfma_f32_32x32x2_f32 takes one B value
//     per lane per step, so a lane reads its column's value of the step's k row with a
//     4-byte read; rows r and r + 8 (read by the two wave halves at once) are put on
//     opposite halves of the banks by swz_b.
//   * The LDS image is the same whatever the DMA width: a lane's bytes land at a fixed
//     place, so each lane fetches the element the permutations put there. 16-byte lanes
//     need K % 16 == 0, N % 4 == 0, lda and ldb multiples of 4 and 16-byte aligned A and
//     B (direct_f32_wide_ok); 4-byte lanes take any shape and alignment (four times the
//     load instructions).
//   * k order: as in the register-staged kernel, lanes 0-31 take k = 4 q + j and lanes
//     32-63 k = 8 + 4 q + j at step j of group q, so each k of the K-step is added once,
//     in the same order, and both kernels give the same bits.
//   * One barrier per K-step, after an explicit s_waitcnt vmcnt that counts the loads of
//     the steps issued after it. The loads are issued from inline asm (M0 set there): the
//     compiler cannot tell the stages apart and would otherwise wait for every load in
//     flight before each LDS read, which removes the pipeline. No other code in these
//     kernels uses M0.
//   * Edges: rows past M and columns past N are clamped to in-range data that only feeds
//     C elements that are not stored. A partial last K-step (K % 16 != 0, 4-byte lanes
//     only) loads clamped k, then the workgroup writes zeros over the k >= K entries of
//     both panels between two barriers.
#include "mm_gemm_tile.h"

namespace mm {
namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;

template <int BM_, int BN_, int WM_, int WN_, int NS_, int VEC_>
struct DirectF32 {
    static constexpr int BM = BM_, BN = BN_, BK = 16, NS = NS_, WM = WM_, WN = WN_, VEC = VEC_;
    static constexpr int WAVES = (BM / WM) * (BN / WN), NT = WAVES * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int A_BYTES = BM * BK * 4, B_BYTES = BK * BN * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int B_ROW = BN * 4;                          // bytes per B row
    static constexpr int LOAD_BYTES = 64 * VEC;                   // one wave instruction
    static constexpr int A_LOADS = A_BYTES / LOAD_BYTES / WAVES;  // per wave per K-step
    static constexpr int B_LOADS = B_BYTES / LOAD_BYTES / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static_assert(VEC == 4 || VEC == 16, "4- or 16-byte lanes");
    static_assert(A_BYTES % (LOAD_BYTES * WAVES) == 0 && B_BYTES % (LOAD_BYTES * WAVES) == 0,
                  "whole loads");
    static_assert(B_ROW >= 256 && B_ROW <= 1024, "B rows of 64 to 256 floats");
    static_assert(NS * STAGE <= 160 * 1024, "stages must fit the 160 KB LDS");
    static_assert((NS - 2) * LOADS <= 63, "vmcnt range");
};

__device__ __forceinline__ int swz_a(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int swz_b(int krow) { return ((krow >> 3) & 1) * 8; }

// VEC bytes per lane from src into LDS at lds_addr + VEC * lane (lds_addr wave-uniform).
template <int VEC>
__device__ __forceinline__ void load_to_lds(unsigned lds_addr, const float *src)
{
    if constexpr (VEC == 16)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src) : "memory");
    else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                     :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait until at most min(steps, S) K-steps of L loads each are outstanding.
template <int L, int S>
__device__ __forceinline__ void wait_steps(int steps)
{
    if constexpr (S > 0) {
        if (steps >= S) {
            wait_vmcnt<S * L>();
            return;
        }
        wait_steps<L, S - 1>(steps);
    } else {
        wait_vmcnt<0>();
    }
}

template <class T>
__global__ __launch_bounds__(T::NT) void gemm_f32_direct_kernel(GemmArgs p)
{
    __shared__ __attribute__((aligned(1024))) char lds[T::NS * T::STAGE];
    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block((int)bid, (int)tiles, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    // problem of a strided batch: grid layer blockIdx.z
    p.A += blockIdx.z * p.sa;
    p.B += blockIdx.z * p.sb;
    p.C += blockIdx.z * p.sc;

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int wm0 = (w / (T::BN / T::WN)) * T::WM, wn0 = (w % (T::BN / T::WN)) * T::WN;
    const int nk = (p.K + T::BK - 1) / T::BK;

    // Each load's lane lands at a fixed panel byte; the element stored there is this
    // lane's source. asrc/bsrc address it at k0 = 0; ak/bk are its k within a K-step.
    const float *asrc[T::A_LOADS];
    const float *bsrc[T::B_LOADS];
    int ak[T::A_LOADS], bk[T::B_LOADS];
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
        const int o = (T::A_LOADS * w + i) * T::LOAD_BYTES + T::VEC * lane;  // panel byte
        const int row = o / 64, slot = (o % 64) / 4;                         // 4-byte slot
        ak[i] = 4 * ((slot >> 2) ^ swz_a(row)) + (slot & 3);
        asrc[i] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + ak[i];
    }
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) {
        const int o = (T::B_LOADS * w + i) * T::LOAD_BYTES + T::VEC * lane;
        const int krow = o / T::B_ROW, slot = (o % T::B_ROW) / 4;
        const int col = n0 + 4 * ((slot >> 2) ^ swz_b(krow)) + (slot & 3);
        bk[i] = krow;
        bsrc[i] = p.B + (int64_t)krow * p.ldb + min(col, T::VEC == 16 ? p.N - 4 : p.N - 1);
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_char *)lds;  // LDS byte offset of the array
    auto issue = [&](int kt) {
        const unsigned st = lds0 + (kt % T::NS) * T::STAGE;
        const int k0 = kt * T::BK;
        // 16-byte lanes come with K % 16 == 0: no partial step
        if (T::VEC == 16 || k0 + T::BK <= p.K) {
#pragma unroll
            for (int i = 0; i < T::A_LOADS; ++i)
                load_to_lds<T::VEC>(st + (T::A_LOADS * w + i) * T::LOAD_BYTES, asrc[i] + k0);
#pragma unroll
            for (int i = 0; i < T::B_LOADS; ++i)
                load_to_lds<T::VEC>(st + T::A_BYTES + (T::B_LOADS * w + i) * T::LOAD_BYTES,
                                    bsrc[i] + (int64_t)k0 * p.ldb);
        } else if constexpr (T::VEC == 4) {
            // partial last step: k clamped to K - 1 (cleared after it lands)
#pragma unroll
            for (int i = 0; i < T::A_LOADS; ++i)
                load_to_lds<T::VEC>(st + (T::A_LOADS * w + i) * T::LOAD_BYTES,
                                    asrc[i] + (min(k0 + ak[i], p.K - 1) - ak[i]));
#pragma unroll
            for (int i = 0; i < T::B_LOADS; ++i)
                load_to_lds<T::VEC>(st + T::A_BYTES + (T::B_LOADS * w + i) * T::LOAD_BYTES,
                                    bsrc[i] + (int64_t)(min(k0 + bk[i], p.K - 1) - bk[i]) * p.ldb);
        }
    };

    // operand addresses inside a stage (bytes): A per group q and block i; B per group q,
    // step j and block jj (k = 8 (lane / 32) + 4 q + j, column wn0 + 32 jj + lane % 32)
    int a_off[2][T::FM], b_off[2][4][T::FN];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int row = wm0 + 32 * i + (lane & 31);
            a_off[q][i] = row * 64 + 16 * ((q + 2 * (lane >> 5)) ^ swz_a(row));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int jj = 0; jj < T::FN; ++jj) {
                const int krow = 8 * (lane >> 5) + 4 * q + j;
                const int col = wn0 + 32 * jj + (lane & 31);
                b_off[q][j][jj] = T::A_BYTES + krow * T::B_ROW + 16 * ((col >> 2) ^ swz_b(krow)) +
                                  4 * (col & 3);
            }
    }

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.f;

    for (int s = 0; s < T::NS - 1 && s < nk; ++s) issue(s);
    for (int kt = 0; kt < nk; ++kt) {
        // step kt's loads are done when at most the later steps' loads are outstanding
        wait_steps<T::LOADS, T::NS - 2>(nk - 1 - kt);
        // every wave's loads for stage kt are in LDS, and every wave is done with the
        // stage the next issue overwrites (read in step kt - 1)
        __syncthreads();
        if (kt + T::NS - 1 < nk) issue(kt + T::NS - 1);
        lds_char *st = (lds_char *)lds + (kt % T::NS) * T::STAGE;
        if (T::VEC == 4 && kt * T::BK + T::BK > p.K) {
            // partial last step: zeros over k >= K in both panels (no load is in flight
            // into this stage and no wave reads it before the barrier below)
            const int kr = p.K - kt * T::BK, nz = T::BK - kr;
            for (int e = threadIdx.x; e < T::BM * nz; e += T::NT) {
                const int r = e / nz, k = kr + e % nz;
                *(lds_float *)(st + r * 64 + 16 * ((k >> 2) ^ swz_a(r)) + 4 * (k & 3)) = 0.f;
            }
            for (int e = threadIdx.x; e < nz * T::BN; e += T::NT)
                *(lds_float *)(st + T::A_BYTES + (kr + e / T::BN) * T::B_ROW + 4 * (e % T::BN)) = 0.f;
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f32x4 a[T::FM];
            float b[4][T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                a[i] = *(const __attribute__((address_space(3))) f32x4 *)(st + a_off[q][i]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int jj = 0; jj < T::FN; ++jj) b[j][jj] = *(const lds_float *)(st + b_off[q][j][jj]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
#pragma unroll
                    for (int jj = 0; jj < T::FN; ++jj)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][j], b[j][jj], acc[i][jj],
                                                                         0, 0, 0);
        }
    }

    // accumulator layout of v_mfma_f32_32x32x2_f32: lane l, register r holds row
    // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of the 32 x 32 block
    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                const int gn = n0 + wn0 + jj * 32 + col_l;
                if (gm < p.M && gn < p.N) p.C[(int64_t)gm * p.ldc + gn] = acc[i][jj][r];
            }
}

template <class T>
hipError_t launch_direct(const GemmArgs &a, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    GemmArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_f32_direct_kernel<T>),
                           dim3(gx, gy, (unsigned)a.batch), dim3(T::NT), args, 0, stream);
}

template <int BM, int BN, int WM, int WN, int NS>
hipError_t launch_either(const GemmArgs &a, hipStream_t stream)
{
    return direct_f32_wide_ok(a) ? launch_direct<DirectF32<BM, BN, WM, WN, NS, 16>>(a, stream)
                                 : launch_direct<DirectF32<BM, BN, WM, WN, NS, 4>>(a, stream);
}

}  // namespace

bool direct_f32_wide_ok(const GemmArgs &a)
{
    const bool aligned = (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 &&
                         (a.batch == 1 || (a.sa % 4 == 0 && a.sb % 4 == 0));
    return a.K % 16 == 0 && a.N >= 4 && a.N % 4 == 0 && a.lda % 4 == 0 && a.ldb % 4 == 0 && aligned;
}

hipError_t gemm_direct_launch(DirectTile t, const GemmArgs &a, hipStream_t stream)
{
    switch (t) {
    case DirectTile::T256:  // 16-byte lanes only
        if (!direct_f32_wide_ok(a)) return hipErrorInvalidValue;
        return launch_direct<DirectF32<256, 256, 128, 64, 4, 16>>(a, stream);
    case DirectTile::T128:
        return launch_either<128, 128, 64, 64, 4>(a, stream);
    case DirectTile::T64S8:
        return launch_either<64, 64, 32, 32, 8>(a, stream);
    case DirectTile::T64S4:
        return launch_either<64, 64, 32, 32, 4>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mm
