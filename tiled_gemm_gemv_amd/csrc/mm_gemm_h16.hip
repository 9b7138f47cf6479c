// mm_gemm_h16.hip -- GEMM with 16-bit inputs (bf16 or fp16) and fp32 accumulation:
// C = A x B with A and B in a 16-bit format and C in fp32.
//
// "Matrix Operations" (docs.vulkan.org ML-inference tutorial, "Performance
// Considerations / Data Types") notes that half precision can run twice as fast as
// fp32 where the hardware supports it, and ("Specialized Hardware") that matrix
// engines go further. On gfx950 the dense 16-bit matrix rate is 16 times the fp32
// one. The products of two 16-bit values are exact in fp32 (at most 22 significant
// bits), so C is the same sum as the fp32 GEMM of the inputs' exact values, summed
// in fp32 in a different order.
//
// Same scheme as the fp32 kernel (mm_gemm.hip): one workgroup per BM x BN tile of
// C, two LDS stages, HBM loads for the next K-step in flight during the current
// step's MFMAs, one barrier per K-step, masked loads at the edges, XCD-aware tile
// order. Differences:
//   * v_mfma_f32_32x32x16_{bf16,f16}: lane l supplies A[l % 32][8 (l / 32) + e] and
//     B[8 (l / 32) + e][l % 32] for e = 0..7, i.e. one 16-byte LDS read per operand;
//     MFMA step s of a K-step covers k = 16 s .. 16 s + 15;
//   * BK = 64 elements (128 bytes) per K-step; LDS rows are padded by 8 elements;
//   * B is transposed into k-contiguous LDS rows as 8 x 4 blocks of 16-bit values
//     (each thread loads 8 rows of 4 columns, 8 bytes each, and regroups them into 4
//     LDS rows of 8 k-values).
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kXcds = 8;

// PF_: K-steps of HBM loads in flight (1 or 2, as in the fp32 kernel). At 16-bit
// rates a K-step of MFMAs is shorter than a load's latency, so the second set of
// staging registers matters more here.
template <int BM_, int BN_, int WM_, int WN_, int PF_ = 1>
struct Tile16 {
    static constexpr int BM = BM_, BN = BN_, BK = 64, WM = WM_, WN = WN_, PF = PF_;
    static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int FM = WM / 32, FN = WN / 32;
    static constexpr int PITCH = BK + 8;            // elements (144 bytes)
    static constexpr int A_TILE = BM * PITCH;       // elements
    static constexpr int STAGE = (BM + BN) * PITCH;
    static constexpr int KG = BK / 8;               // 16-byte groups along k
    static constexpr int A_CHUNKS = BM * KG;
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int B_BLOCKS = KG * (BN / 4);  // 8 x 4 blocks of a B panel
    static constexpr int B_PER_T = (B_BLOCKS + NT - 1) / NT;
    static_assert(2 * STAGE * 2 <= 160 * 1024, "two stages must fit the 160 KB LDS");
    struct Staged {
        u32x4 a[A_PER_T];
        u32x2 b[B_PER_T][8];  // 8 k-rows x 4 columns each
    };
};

// 8 consecutive 16-bit values at p (in range) as 16 bytes.
template <bool VEC>
__device__ __forceinline__ u32x4 load8(const unsigned short *p)
{
    if constexpr (VEC) {
        return *reinterpret_cast<const u32x4 *>(p);
    } else {
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (unsigned)p[2 * q] | ((unsigned)p[2 * q + 1] << 16);
        return v;
    }
}

// 4 consecutive 16-bit values at p (in range) as 8 bytes.
template <bool VEC>
__device__ __forceinline__ u32x2 load4h(const unsigned short *p)
{
    if constexpr (VEC) {
        return *reinterpret_cast<const u32x2 *>(p);
    } else {
        return u32x2{(unsigned)p[0] | ((unsigned)p[1] << 16), (unsigned)p[2] | ((unsigned)p[3] << 16)};
    }
}

template <bool VEC>
__device__ __forceinline__ u32x2 load4h_masked(const unsigned short *p, int valid)
{
    if (valid >= 4) return load4h<VEC>(p);
    u32x2 v = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e < valid) v[e >> 1] |= (unsigned)p[e] << (16 * (e & 1));
    return v;
}

// The first `valid` of 8 consecutive values at p, zeros after; nothing past them is read.
template <bool VEC>
__device__ __forceinline__ u32x4 load8_masked(const unsigned short *p, int valid)
{
    if (valid >= 8) return load8<VEC>(p);
    u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (e < valid) v[e >> 1] |= (unsigned)p[e] << (16 * (e & 1));
    return v;
}

__device__ __forceinline__ void tile_of_block16(int bid, int nblocks, int tiles_m, int tiles_n,
                                                int &tm, int &tn)
{
    const int q = nblocks / kXcds, r = nblocks % kXcds;
    const int xcd = bid % kXcds, slot = bid / kXcds;
    const int logical = (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
    constexpr int group_m = 8;
    const int per_group = group_m * tiles_n;
    const int g = logical / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in_g = logical - g * per_group;
    tm = first_m + in_g % gm;
    tn = in_g / gm;
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

struct Gemm16Args {
    const unsigned short *A;
    const unsigned short *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
};

template <class T, bool BF16, bool VEC_A, bool VEC_B>
__global__ __launch_bounds__(T::NT) void gemm_h16_kernel(Gemm16Args p)
{
    __shared__ __attribute__((aligned(16))) unsigned short lds[2 * T::STAGE];

    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block16((int)bid, (int)tiles, tiles_m, tiles_n, tm, tn);
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

    typename T::Staged r0, r1;

    auto global_load = [&](int kt, typename T::Staged &st) {
        const int k0 = kt * T::BK;
        const bool full = inner_mn && (k0 + T::BK <= p.K);
#pragma unroll
        for (int c = 0; c < T::A_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::A_CHUNKS % T::NT == 0 || idx < T::A_CHUNKS) {
                const int row = idx / T::KG, kg = idx % T::KG;
                const int gm = m0 + row, gk = k0 + 8 * kg;
                const unsigned short *src = p.A + (int64_t)gm * p.lda + gk;
                st.a[c] = full ? load8<VEC_A>(src)
                               : load8_masked<VEC_A>(src, gm < p.M ? p.K - gk : 0);
            }
        }
#pragma unroll
        for (int c = 0; c < T::B_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::B_BLOCKS % T::NT == 0 || idx < T::B_BLOCKS) {
                const int kg = idx % T::KG, ng = idx / T::KG;
                const int gn = n0 + 4 * ng;
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int gk = k0 + 8 * kg + r;
                    const unsigned short *src = p.B + (int64_t)gk * p.ldb + gn;
                    st.b[c][r] = full ? load4h<VEC_B>(src)
                                      : load4h_masked<VEC_B>(src, gk < p.K ? p.N - gn : 0);
                }
            }
        }
    };

    auto lds_store = [&](int buf, const typename T::Staged &st) {
        unsigned short *As = lds + buf * T::STAGE;
        unsigned short *Bs = As + T::A_TILE;
#pragma unroll
        for (int c = 0; c < T::A_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::A_CHUNKS % T::NT == 0 || idx < T::A_CHUNKS) {
                const int row = idx / T::KG, kg = idx % T::KG;
                *reinterpret_cast<u32x4 *>(As + row * T::PITCH + 8 * kg) = st.a[c];
            }
        }
#pragma unroll
        for (int c = 0; c < T::B_PER_T; ++c) {
            const int idx = tid + c * T::NT;
            if (T::B_BLOCKS % T::NT == 0 || idx < T::B_BLOCKS) {
                const int kg = idx % T::KG, ng = idx / T::KG;
                // st.b[c][r] holds 4 columns of B's k-row r of the block (two values per
                // word); column col of the block becomes one k-contiguous LDS row.
#pragma unroll
                for (int col = 0; col < 4; ++col) {
                    const int w = col >> 1;
                    const int sh = 16 * (col & 1);
                    u32x4 v;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const unsigned lo = (st.b[c][2 * q][w] >> sh) & 0xffffu;
                        const unsigned hi = (st.b[c][2 * q + 1][w] >> sh) & 0xffffu;
                        v[q] = lo | (hi << 16);
                    }
                    *reinterpret_cast<u32x4 *>(Bs + (4 * ng + col) * T::PITCH + 8 * kg) = v;
                }
            }
        }
    };

    auto multiply = [&](int buf, auto &&mid) {
        const int koff = (lane >> 5) * 8;
        const unsigned short *As = lds + buf * T::STAGE + (wm0 + (lane & 31)) * T::PITCH + koff;
        const unsigned short *Bs =
            lds + buf * T::STAGE + T::A_TILE + (wn0 + (lane & 31)) * T::PITCH + koff;
        u32x4 a[2][T::FM], b[2][T::FN];
        auto read_frags = [&](int s, u32x4 (&fa)[T::FM], u32x4 (&fb)[T::FN]) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                fa[i] = *reinterpret_cast<const u32x4 *>(As + i * 32 * T::PITCH + 16 * s);
#pragma unroll
            for (int j = 0; j < T::FN; ++j)
                fb[j] = *reinterpret_cast<const u32x4 *>(Bs + j * 32 * T::PITCH + 16 * s);
        };
        read_frags(0, a[0], b[0]);
#pragma unroll
        for (int s = 0; s < T::BK / 16; ++s) {
            if (s + 1 < T::BK / 16) read_frags(s + 1, a[(s + 1) & 1], b[(s + 1) & 1]);
            if (s == T::BK / 32) mid();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j)
                    acc[i][j] = mfma16<BF16>(a[s & 1][i], b[s & 1][j], acc[i][j]);
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
            multiply(cur, nothing);
            // the other stage was last read in step kt - 1, before the barrier ending it
            if (kt + 1 < nk) lds_store(cur ^ 1, r0);
            __syncthreads();
        }
    } else {
        // Two staging buffers, loop unrolled by two (see the fp32 kernel): the loads
        // for step kt + 2 are issued at the top of step kt; step kt + 1's data is
        // written to the other stage halfway through step kt's MFMAs.
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
        if (kt < nk) multiply(0, nothing);
    }

    // accumulator layout as for the fp32 32x32 blocks
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

template <class T, bool BF16>
hipError_t launch16(const Gemm16Args &a, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool va = (a.lda % 8 == 0) && ((uintptr_t)a.A % 16 == 0);
    const bool vb = (a.ldb % 4 == 0) && ((uintptr_t)a.B % 8 == 0);
    const void *fn;
    if (va && vb)
        fn = reinterpret_cast<const void *>(&gemm_h16_kernel<T, BF16, true, true>);
    else if (va)
        fn = reinterpret_cast<const void *>(&gemm_h16_kernel<T, BF16, true, false>);
    else if (vb)
        fn = reinterpret_cast<const void *>(&gemm_h16_kernel<T, BF16, false, true>);
    else
        fn = reinterpret_cast<const void *>(&gemm_h16_kernel<T, BF16, false, false>);
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    Gemm16Args arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(fn, dim3(gx, gy), dim3(T::NT), args, 0, stream);
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS pipeline (the fast path for aligned shapes).
//
// gfx950's global_load_lds_dwordx4 moves 16 bytes per lane from memory straight into
// LDS (lane l's bytes land at M0 + 16 l), with no staging registers. That frees the
// registers the loop above spends on staged data, so the pipeline can run NS = 4 LDS
// stages deep: the loads for K-step kt + 3 are issued while step kt's MFMAs run, which
// covers three K-steps of MFMA time instead of one. BK = 32 (64-byte A rows); where
// K % 64 == 0, BK = 64 in two stages of twice the size (the same LDS): each A row of a
// step is then one whole 128-byte line (a 64-byte row is half a line, and the DMA's LDS
// writes of such rows count bank-conflict cycles), with twice the MFMAs per barrier
// (measured +2-5% on the 256 x 256 tile, +5-17% on the 128 x 128 one, +17-30% on the
// 64 x 64 one).
//   * A panel (BM rows x BK k): stored as loaded, 2 BK bytes per row; the 16-byte
//     chunks of row r sit in slots c ^ swz_a(r), so that the MFMA operand reads of 32
//     rows at one k fall in distinct banks (no padding; the load pattern applies the
//     permutation by choosing which chunk each lane fetches).
//   * B panel (BK k rows x BN): stored row-major as loaded, chunks of row k in slots
//     c ^ swz_b(k). The MFMA wants 8 consecutive k of one column per lane; gfx950's
//     ds_read_b64_tr_b16 provides them: in each group of 16 lanes, result lane i,
//     element c is element i % 4 of the 4 values lane 4 c + i / 4 addressed. Lane j of a
//     group therefore addresses row k0 + j / 4, columns n + 4 (j % 4), and result lane i
//     receives column n + i at rows k0 .. k0 + 3; two such reads give the 8 k.
//   * One barrier per K-step, after an explicit wait for the step's loads (vmcnt
//     counts the loads of the steps issued after it). The loads are issued from inline
//     asm so that the compiler does not add a wait for all of them before every LDS read.
//   * Requirements (checked on the host): K % 32 == 0 (K % 64 == 0 for BK = 64), N % 8 == 0, lda and ldb
//     multiples of 8 elements, A and B 16-byte aligned. Rows past M and column chunks
//     past N are clamped to in-range ones; they only feed C elements that are not
//     stored. K needs no mask (whole K-steps).
template <int BM_, int BN_, int WM_, int WN_, int BK_ = 32, int NS_ = 4>
struct Direct16 {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_, WM = WM_, WN = WN_;
    static constexpr int WAVES = (BM / WM) * (BN / WN), NT = WAVES * 64;
    static constexpr int FM = WM / 32, FN = WN / 32, KS = BK / 16;  // KS: 16-k MFMA steps
    static constexpr int A_ROW = BK * 2, A_CPR = A_ROW / 16;        // A row bytes, 16-byte chunks
    static constexpr int A_ROWS_PER_LOAD = 1024 / A_ROW;
    static constexpr int A_BYTES = BM * A_ROW, B_BYTES = BK * BN * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int B_ROW = BN * 2;                      // bytes per B row
    static constexpr int A_LOADS = A_BYTES / 1024 / WAVES;    // 1 KB loads per wave per step
    static constexpr int B_LOADS = B_BYTES / 1024 / WAVES;
    static constexpr int B_ROWS_PER_LOAD = 1024 / B_ROW;
    static_assert(BK == 32 || BK == 64, "K-steps of 32 or 64");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0,
                  "whole 1 KB loads per wave");
    static_assert((NS - 2) * (A_LOADS + B_LOADS) <= 63, "vmcnt range");
    static_assert(BN >= 64 && BN % 32 == 0 && WN % 32 == 0 && WM % 32 == 0, "tile shape");
    static_assert(NS * STAGE <= 160 * 1024, "stages must fit the 160 KB LDS");
};

// A rows of 64 bytes (BK = 32): two rows per 128 bytes of banks. Rows of 128 bytes
// (BK = 64): the 8 chunk slots of any 8 (or, on 64 banks, 16) consecutive rows read at
// one k are distinct.
template <class T>
__device__ __forceinline__ int swz_a16(int row)
{
    if constexpr (T::A_CPR == 4) return ((row >> 1) ^ (row >> 3)) & 3;
    else return ((row >> 1) & 7) ^ ((row & 1) << 2);
}

template <class T>
__device__ __forceinline__ int swz_b16(int krow)
{
    return (krow % (T::BN / 32)) * 4;  // spreads 4 consecutive rows over the banks
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// 16 bytes per lane from base + voff into LDS at lds_addr + 16 * lane (lds_addr and base
// wave-uniform, in scalar registers; voff the lane's byte offset), so that a load takes no
// vector instruction. The LDS address is the asm statement's M0 operand ("{m0}"), which
// the compiler writes right before the load; the s_nop is the one wait state a global load
// with LDS = 1 needs after an SALU write of M0 (the hazard recognizer does not look inside
// an asm string).
__device__ __forceinline__ void load_to_lds_s(unsigned lds_addr, const unsigned short *base, unsigned voff)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait until at most min(later, S) K-steps of L loads each are outstanding.
template <int L, int S>
__device__ __forceinline__ void wait_later(int later)
{
    if constexpr (S == 0) {
        wait_vmcnt<0>();
    } else {
        if (later >= S) wait_vmcnt<S * L>();
        else wait_later<L, S - 1>(later);
    }
}

template <class T, bool BF16>
__global__ __launch_bounds__(T::NT) void gemm_h16_direct_kernel(Gemm16Args p)
{
    __shared__ __attribute__((aligned(1024))) char lds[T::NS * T::STAGE];
    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block16((int)bid, (int)tiles, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, in a scalar register
    const int wm0 = (w / (T::BN / T::WN)) * T::WM, wn0 = (w % (T::BN / T::WN)) * T::WN;
    const int nk = p.K / T::BK;

    // this lane's byte offsets from the tile's corner at the K-step (the loads' scalar
    // base, advanced by BK per step); direct_ok keeps them below 2^32
    unsigned aoff[T::A_LOADS], boff[T::B_LOADS];
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i) {
        const int row = T::A_ROWS_PER_LOAD * (T::A_LOADS * w + i) + lane / T::A_CPR;
        const int chunk = (lane % T::A_CPR) ^ swz_a16<T>(row);
        aoff[i] = (unsigned)(((int64_t)(min(m0 + row, p.M - 1) - m0) * p.lda + 8 * chunk) * 2);
    }
#pragma unroll
    for (int i = 0; i < T::B_LOADS; ++i) {
        constexpr int CPR = T::B_ROW / 16;  // 16-byte chunks per B row
        const int krow = T::B_ROWS_PER_LOAD * (T::B_LOADS * w + i) + lane / CPR;
        const int chunk = (lane % CPR) ^ swz_b16<T>(krow);
        // N % 8 == 0: min(n0 + 8 chunk, N - 8) >= n0
        boff[i] = (unsigned)(((int64_t)krow * p.ldb + (min(n0 + 8 * chunk, p.N - 8) - n0)) * 2);
    }
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_char *)lds;  // LDS byte offset of the array
    auto issue = [&](int kt) {
        const unsigned st = lds0 + (kt % T::NS) * T::STAGE;
        const unsigned short *abase = p.A + (int64_t)m0 * p.lda + (int64_t)kt * T::BK;
        const unsigned short *bbase = p.B + (int64_t)kt * T::BK * p.ldb + n0;
#pragma unroll
        for (int i = 0; i < T::A_LOADS; ++i) load_to_lds_s(st + (T::A_LOADS * w + i) * 1024, abase, aoff[i]);
#pragma unroll
        for (int i = 0; i < T::B_LOADS; ++i)
            load_to_lds_s(st + T::A_BYTES + (T::B_LOADS * w + i) * 1024, bbase, boff[i]);
    };

    // operand addresses inside a stage (bytes), for the 16-k MFMA steps of a K-step
    int a_off[T::KS][T::FM], b_off[T::KS][2][T::FN];
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int row = wm0 + 32 * i + (lane & 31);
            a_off[ks][i] = row * T::A_ROW + 16 * ((2 * ks + (lane >> 5)) ^ swz_a16<T>(row));
        }
        const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const int krow = 16 * ks + 8 * (g >> 1) + 4 * h + (j16 >> 2);
                const int col = wn0 + 32 * j + 16 * (g & 1) + 4 * (j16 & 3);
                b_off[ks][h][j] = T::A_BYTES + krow * T::B_ROW +
                                  16 * ((col >> 3) ^ swz_b16<T>(krow)) + 8 * ((col >> 2) & 1);
            }
    }

    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    constexpr int LOADS = T::A_LOADS + T::B_LOADS;  // per wave per K-step
    for (int s = 0; s < T::NS - 1 && s < nk; ++s) issue(s);
    for (int kt = 0; kt < nk; ++kt) {
        // step kt's loads are done when at most the later steps' loads are outstanding
        wait_later<LOADS, T::NS - 2>(nk - 1 - kt);
        // every wave's loads for stage kt are in LDS, and every wave is done with the
        // stage the next issue overwrites (read in step kt - 1)
        __syncthreads();
        if (kt + T::NS - 1 < nk) issue(kt + T::NS - 1);
        const lds_char *st = (const lds_char *)lds + (kt % T::NS) * T::STAGE;
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            u32x4 a[T::FM], b[T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                a[i] = *(const __attribute__((address_space(3))) u32x4 *)(st + a_off[ks][i]);
#pragma unroll
            for (int j = 0; j < T::FN; ++j) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(st + b_off[ks][0][j]));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(st + b_off[ks][1][j]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                b[j] = u32x4{l2[0], l2[1], h2[0], h2[1]};
            }
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int j = 0; j < T::FN; ++j) acc[i][j] = mfma16<BF16>(a[i], b[j], acc[i][j]);
        }
    }

    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                const int gn = n0 + wn0 + j * 32 + col_l;
                if (gm < p.M && gn < p.N) p.C[(int64_t)gm * p.ldc + gn] = acc[i][j][r];
            }
}

// The direct pipeline's requirements (see above).
bool direct_ok(const Gemm16Args &a)
{
    // the per-lane byte offsets from a tile's corner (below 256 rows of A, 64 rows of B
    // and 256 columns) must fit 32 bits
    constexpr int64_t kOffMax = int64_t(1) << 32;
    return a.K % 32 == 0 && a.N >= 8 && a.N % 8 == 0 && a.lda % 8 == 0 && a.ldb % 8 == 0 &&
           (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.B % 16 == 0 && 2 * (255 * a.lda + 64) < kOffMax &&
           2 * (63 * a.ldb + 256) < kOffMax;
}

template <class T, bool BF16>
hipError_t launch16_direct(const Gemm16Args &a, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (a.K % T::BK) return hipErrorInvalidValue;
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    Gemm16Args arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_h16_direct_kernel<T, BF16>),
                           dim3(gx, gy), dim3(T::NT), args, 0, stream);
}

using D16L = Direct16<256, 256, 128, 64>;
using D16M = Direct16<128, 128, 64, 64>;
using D16S = Direct16<64, 64, 32, 32>;
// K-steps of 64 in half the stages (the same LDS), for K % 64 == 0
using D16L64 = Direct16<256, 256, 128, 64, 64, 2>;
using D16M64 = Direct16<128, 128, 64, 64, 64, 2>;
using D16S64 = Direct16<64, 64, 32, 32, 64, 2>;

template <class T, class T64, bool BF16>
hipError_t launch16_direct_k(const Gemm16Args &a, hipStream_t stream)
{
    return a.K % 64 == 0 ? launch16_direct<T64, BF16>(a, stream) : launch16_direct<T, BF16>(a, stream);
}

using T16L = Tile16<256, 256, 128, 64>;
using T16M = Tile16<128, 128, 64, 64>;
using T16S = Tile16<64, 64, 32, 32>;
using T16Mp2 = Tile16<128, 128, 64, 64, 2>;
using T16Sp2 = Tile16<64, 64, 32, 32, 2>;

}  // namespace

int gemm16_num_configs() { return 8; }

const char *gemm16_config_name(int cfg)
{
    static const char *names[] = {"256x256x64 w128x64 pf1 (8 waves)", "128x128x64 w64x64 pf1 (4 waves)",
                                  "64x64x64 w32x32 pf1 (4 waves)", "128x128x64 w64x64 pf2 (4 waves)",
                                  "64x64x64 w32x32 pf2 (4 waves)",
                                  "256x256x32 w128x64 direct-to-LDS 4 stages (8 waves; K % 64 == 0: K-steps of 64, 2 stages)",
                                  "128x128x32 w64x64 direct-to-LDS 4 stages (4 waves; K % 64 == 0: K-steps of 64, 2 stages)",
                                  "64x64x32 w32x32 direct-to-LDS 4 stages (4 waves; K % 64 == 0: K-steps of 64, 2 stages)"};
    return (cfg >= 0 && cfg < 8) ? names[cfg] : nullptr;
}

int gemm16_select_config(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    // 5, 6 and 7 are the direct pipelines; on shapes they cannot take they run the
    // register-staged kernels of their size (configs 0, 3 and 4). Smaller tiles where the
    // big ones would leave CUs idle (1024^3 bf16: 243 TFLOP/s on the 64 x 64 direct tile
    // against 144 staged).
    if (((M + 255) / 256) * ((N + 255) / 256) >= 200) return 5;
    if (((M + 127) / 128) * ((N + 127) / 128) >= 200) return 6;
    return 7;
}

hipError_t gemm16_launch(int cfg, bool bf16, const void *A, int64_t lda, const void *B, int64_t ldb,
                         float *C, int64_t ldc, int M, int N, int K, hipStream_t stream)
{
    Gemm16Args a;
    a.A = static_cast<const unsigned short *>(A);
    a.B = static_cast<const unsigned short *>(B);
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = M;
    a.N = N;
    a.K = K;
    switch (cfg) {
    case 0: return bf16 ? launch16<T16L, true>(a, stream) : launch16<T16L, false>(a, stream);
    case 1: return bf16 ? launch16<T16M, true>(a, stream) : launch16<T16M, false>(a, stream);
    case 2: return bf16 ? launch16<T16S, true>(a, stream) : launch16<T16S, false>(a, stream);
    case 3: return bf16 ? launch16<T16Mp2, true>(a, stream) : launch16<T16Mp2, false>(a, stream);
    case 4: return bf16 ? launch16<T16Sp2, true>(a, stream) : launch16<T16Sp2, false>(a, stream);
    // the direct pipelines; shapes they do not take run the same tile size staged
    // through registers
    case 5:
        if (!direct_ok(a)) return gemm16_launch(0, bf16, A, lda, B, ldb, C, ldc, M, N, K, stream);
        return bf16 ? launch16_direct_k<D16L, D16L64, true>(a, stream) : launch16_direct_k<D16L, D16L64, false>(a, stream);
    case 6:
        if (!direct_ok(a)) return gemm16_launch(3, bf16, A, lda, B, ldb, C, ldc, M, N, K, stream);
        return bf16 ? launch16_direct_k<D16M, D16M64, true>(a, stream) : launch16_direct_k<D16M, D16M64, false>(a, stream);
    default:
        if (!direct_ok(a)) return gemm16_launch(4, bf16, A, lda, B, ldb, C, ldc, M, N, K, stream);
        return bf16 ? launch16_direct_k<D16S, D16S64, true>(a, stream) : launch16_direct_k<D16S, D16S64, false>(a, stream);
    }
}

}  // namespace mm
