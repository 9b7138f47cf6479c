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
// Two kernels. The direct HBM -> LDS pipeline (further below; configs 5-10, the ones
// mm_gemm_bf16 / mm_gemm_f16 choose) serves every shape with K >= 32 and N >= 64 or
// N % 8 == 0, at any 2-byte alignment. The register-staged kernel here serves the rest
// (and configs 0-4). It follows the fp32 kernel (mm_gemm.hip): one workgroup per
// BM x BN tile of C, two LDS stages, HBM loads for the next K-step in flight during the
// current step's MFMAs, one barrier per K-step, masked loads at the edges, XCD-aware
// tile order. Differences:
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
// Direct HBM -> LDS pipeline.
//
// gfx950's global_load_lds_dwordx4 moves 16 bytes per lane from memory straight into
// LDS (lane l's bytes land at M0 + 16 l), with no staging registers. That frees the
// registers the loop above spends on staged data, so the pipeline runs NS LDS stages
// deep: the loads for K-step kt + NS - 1 are issued while step kt's MFMAs run. K-steps
// of BK = 64 make each A row of a step one whole 128-byte line (a 64-byte row is half a
// line, and the DMA's LDS writes of such rows count bank-conflict cycles), with twice the
// MFMAs per barrier of BK = 32 (measured +2-5% on the 256 x 256 tile, +5-17% on the
// 128 x 128 one, +17-30% on the 64 x 64 one).
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
//     With one wave group, the step's first operand reads go out right after the barrier
//     and the next step's loads after them.
//   * Any alignment: a lane's 16 bytes are read from wherever its 8 elements start (rows
//     of odd length put half the rows at 2-byte alignment; the device's unaligned access
//     mode serves such loads, into LDS as into registers), so neither the leading
//     dimensions nor the base pointers need more than the elements' 2-byte alignment.
//   * Edges, with every 16-byte chunk inside the matrix:
//       - rows past M are clamped to row M - 1; they only feed C rows that are not stored;
//       - columns: with N >= BN the last tile column's B panel starts at N - BN instead of
//         its own origin (every chunk inside B's rows); the columns left of the origin
//         belong to the tile before and are not stored again, so each C element is
//         written once. With N < BN (one tile column) N must be a multiple of 8 and
//         chunks past N are clamped to the last one (they feed only unstored columns);
//       - K % BK != 0: one more step, run first, loads k in [K - BK, K). Its first
//         BK - K % BK k overlap the whole steps that follow: once its loads have landed,
//         the workgroup writes zeros over those k in both panels (between two barriers), so
//         they add 0 * 0 (also where A or B holds an infinity or a NaN).
//     These need K >= BK and offsets from a tile's corner that fit 32 bits (direct_ok).
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_>
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
    static_assert(NS >= 2 && (NS - 2) * (A_LOADS + B_LOADS) <= 63, "vmcnt range");
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

// A transposed B read (ds_read_b64_tr_b16) touches 64 bytes of each of the rows 4q .. 4q + 3
// and 4q + 8 .. 4q + 11, 512 bytes in all, i.e. two passes over the 64 banks at best: each
// 64-byte quarter of the banks should serve two of those rows. Rows of 256 bytes or more
// span every quarter: XOR-ing the chunk index by 4 (krow % 4) puts rows 4q .. 4q + 3 on four
// different quarters. A 128-byte row (BN = 64) spans two quarters, chosen by the row's
// parity: XOR-ing by 4 ((krow >> 1) & 1) sends rows 4q and 4q + 2 (and 4q + 1, 4q + 3) to
// different halves of their pair of quarters (krow % 2 instead stacks four rows on one
// quarter: 1.33 conflict cycles per LDS instruction measured on the 64 x 64 tile).
template <class T>
__device__ __forceinline__ int swz_b16(int krow)
{
    if constexpr (T::BN == 64) return ((krow >> 1) & 1) * 4;
    else return (krow % (T::BN / 32)) * 4;
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

// KG wave groups of T::WAVES waves each share a workgroup and its tile: group g takes the
// K-steps s with s % KG == g into a ring of its own, and at the end group 1 hands its
// accumulators to group 0 through LDS, which adds them (in that fixed order) and stores
// the tile. Two groups put twice the waves and twice the loads in flight on the CU that
// holds the tile, for shapes with about one tile per CU.
template <class T, bool BF16, int KG>
__global__ __launch_bounds__(T::NT * KG) void gemm_h16_direct_kernel(Gemm16Args p)
{
    static_assert(KG == 1 || (KG == 2 && T::WAVES * T::FM * T::FN * 16 * 64 * 4 <= KG * T::NS * T::STAGE),
                  "group 1's accumulators must fit the stages");
    __shared__ __attribute__((aligned(1024))) char lds[KG * T::NS * T::STAGE];
    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block16((int)bid, (int)tiles, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    // origin of the B panel: n0, or N - BN for a last tile column that would cross N
    const int nb0 = p.N >= T::BN ? min(n0, p.N - T::BN) : 0;

    const int lane = threadIdx.x & 63;
    const int wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index, in a scalar register
    const int grp = KG == 1 ? 0 : wg / T::WAVES, w = KG == 1 ? wg : wg % T::WAVES;  // K group, wave in it
    const int wm0 = (w / (T::BN / T::WN)) * T::WM, wn0 = (w % (T::BN / T::WN)) * T::WN;
    // K-steps: with K % BK != 0 step 0 is the tail, k in [K - BK, K); it shares its first
    // ov k with the whole steps, which follow as steps 1 .. nk - 1 (k0 = (s - 1) BK)
    const int nk_full = p.K / T::BK;              // whole K-steps (>= 1)
    const int ov = (T::BK - p.K % T::BK) % T::BK;
    const int tail = ov ? 1 : 0;
    const int nk = nk_full + tail;
    const int nj = (nk + KG - 1) / KG;            // ring steps of every group (the last may idle)
    const int my_steps = KG == 1 ? nk : (nk - grp + KG - 1) / KG;  // steps of this group

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
        int col = nb0 + 8 * chunk;               // N >= BN: inside the row
        if (p.N < T::BN) col = min(col, p.N - 8);  // N % 8 == 0 here
        boff[i] = (unsigned)(((int64_t)krow * p.ldb + (col - nb0)) * 2);
    }
    // this group's ring
    const unsigned ring0 = (unsigned)(uintptr_t)(lds_char *)lds + grp * T::NS * T::STAGE;
    auto issue = [&](int j) {  // the group's ring step j: K-step s = j KG + grp
        const int s = j * KG + grp;
        const unsigned st = ring0 + (j % T::NS) * T::STAGE;
        const int k0 = (tail && s == 0) ? p.K - T::BK : (s - tail) * T::BK;
        const unsigned short *abase = p.A + (int64_t)m0 * p.lda + k0;
        const unsigned short *bbase = p.B + (int64_t)k0 * p.ldb + nb0;
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

    const lds_char *ring = (const lds_char *)lds + grp * T::NS * T::STAGE;
    auto multiply = [&](int j, auto &&between) {
        const lds_char *st = ring + (j % T::NS) * T::STAGE;
        u32x4 a[2][T::FM], b[2][T::FN];
        auto operands = [&](int ks, int buf) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                a[buf][i] = *(const __attribute__((address_space(3))) u32x4 *)(st + a_off[ks][i]);
#pragma unroll
            for (int jj = 0; jj < T::FN; ++jj) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(st + b_off[ks][0][jj]));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(st + b_off[ks][1][jj]));
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                b[buf][jj] = u32x4{l2[0], l2[1], h2[0], h2[1]};
            }
        };
        // software-pipelined: the LDS reads of MFMA step ks + 1 go out before the MFMAs of
        // step ks (a second register set), so their latency hides behind those MFMAs
        // (+1-3.5% on the large shapes; the sums are those of the plain loop, in its order)
        operands(0, 0);
        between();
#pragma unroll
        for (int ks = 0; ks < T::KS; ++ks) {
            if (ks + 1 < T::KS) operands(ks + 1, (ks + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < T::FN; ++jj)
                    acc[i][jj] = mfma16<BF16>(a[ks & 1][i], b[ks & 1][jj], acc[i][jj]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    constexpr int LOADS = T::A_LOADS + T::B_LOADS;  // per wave per K-step
    for (int j = 0; j < T::NS - 1 && j < my_steps; ++j) issue(j);
    // ring step 0, peeled: step j's loads are done when at most the later steps' loads are
    // outstanding; after the barrier every wave's loads for stage j are in LDS, and every
    // wave is done with the stage the next issue overwrites (read in step j - 1)
    wait_later<LOADS, T::NS - 2>(my_steps - 1);
    __syncthreads();
    if (T::NS - 1 < my_steps) issue(T::NS - 1);
    if (tail) {
        // K-step 0 (group 0's first) is the tail: zeros over the ov k it shares with the
        // whole steps, in both panels; its loads have landed (the wait and barrier above),
        // and nothing reads the stage before the barrier below
        if (grp == 0) {
            lds_char *st = (lds_char *)lds;
            for (int e = threadIdx.x; e < T::BM * ov; e += T::NT) {
                const int r = e / ov, k = e - r * ov;
                *(__attribute__((address_space(3))) unsigned short *)(
                    st + r * T::A_ROW + 16 * ((k >> 3) ^ swz_a16<T>(r)) + 2 * (k & 7)) = 0;
            }
            for (int e = threadIdx.x; e < ov * (T::B_ROW / 16); e += T::NT)
                *(__attribute__((address_space(3))) u32x4 *)(st + T::A_BYTES + 16 * e) = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();
    }
    if (my_steps > 0) multiply(0, [] {});
    for (int j = 1; j < nj; ++j) {
        wait_later<LOADS, T::NS - 2>(my_steps - 1 - j);
        __syncthreads();
        auto next = [&] {
            if (j + T::NS - 1 < my_steps) issue(j + T::NS - 1);
        };
        if constexpr (KG == 1) {
            // the first MFMA step's operand reads go out before the next step's DMA loads, so
            // that their latency passes while those loads issue: after the barrier every wave
            // of a SIMD would otherwise issue its loads and then wait on its first reads with
            // the matrix core idle (same bits; measured +2-8% on the 256 x 256 tile at the
            // large shapes, +5% on the 64 x 64 tile at 1024^3; with two wave groups, whose
            // barrier is shared by twice the waves, 4-13% slower, so they keep the old order)
            multiply(j, next);
        } else {
            next();
            if (j < my_steps) multiply(j, [] {});
        }
    }

    if constexpr (KG == 2) {
        // group 1's accumulators to LDS (lane-minor: conflict-free), group 0 adds them
        __syncthreads();  // every wave is done with the stages
        typedef __attribute__((address_space(3))) float lds_f32;
        lds_f32 *x = (lds_f32 *)lds + w * (T::FM * T::FN * 16 * 64) + lane;
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[((i * T::FN + jj) * 16 + r) * 64] = acc[i][jj][r];
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][jj][r] += x[((i * T::FN + jj) * 16 + r) * 64];
    }

    // accumulator layout as for the fp32 32x32 blocks; local column c is column nb0 + c of
    // C, stored from n0 on (columns left of n0 belong to the tile column before)
    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                const int gn = nb0 + wn0 + jj * 32 + col_l;
                if (gm < p.M && gn < p.N && gn >= n0) p.C[(int64_t)gm * p.ldc + gn] = acc[i][jj][r];
            }
}

// The direct pipeline's requirements for K-steps of bk (see above).
bool direct_ok(const Gemm16Args &a, int bm, int bn, int bk)
{
    // the per-lane byte offsets from a tile's corner (below bm rows of A, bk rows of B and
    // bn columns) must fit 32 bits
    constexpr int64_t kOffMax = int64_t(1) << 32;
    return a.K >= bk && a.N >= 8 && (a.N >= bn || a.N % 8 == 0) &&
           2 * ((bm - 1) * a.lda + bk) < kOffMax && 2 * ((int64_t)(bk - 1) * a.ldb + bn) < kOffMax;
}

template <class T, bool BF16, int KG>
hipError_t launch16_direct(const Gemm16Args &a, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (!direct_ok(a, T::BM, T::BN, T::BK)) return hipErrorInvalidValue;
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    Gemm16Args arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_h16_direct_kernel<T, BF16, KG>),
                           dim3(gx, gy), dim3(T::NT * KG), args, 0, stream);
}

// A direct tile with K-steps of 64 (T64) where K >= 64, else of 32 (T32), in KG wave
// groups; shapes the pipeline cannot take (K < 32, N < BN with N % 8 != 0, offsets beyond
// 32 bits) run the register-staged tile `staged`.
template <class T32, class T64, class TS, int KG>
hipError_t launch16_direct_k(bool bf16, const Gemm16Args &a, hipStream_t stream)
{
    if (direct_ok(a, T64::BM, T64::BN, 64))
        return bf16 ? launch16_direct<T64, true, KG>(a, stream) : launch16_direct<T64, false, KG>(a, stream);
    if (direct_ok(a, T32::BM, T32::BN, 32))
        return bf16 ? launch16_direct<T32, true, KG>(a, stream) : launch16_direct<T32, false, KG>(a, stream);
    return bf16 ? launch16<TS, true>(a, stream) : launch16<TS, false>(a, stream);
}

using T16L = Tile16<256, 256, 128, 64>;
using T16M = Tile16<128, 128, 64, 64>;
using T16S = Tile16<64, 64, 32, 32>;
using T16Mp2 = Tile16<128, 128, 64, 64, 2>;
using T16Sp2 = Tile16<64, 64, 32, 32, 2>;

// direct tiles: <BM, BN, WM, WN, BK, stages>
using D16L = Direct16<256, 256, 128, 64, 32, 4>;
// 16 waves of 64 x 64: four waves per SIMD to cover each K-step's barrier and operand reads,
// against 8 waves of 128 x 64 whose LDS operand reads per MFMA are a third fewer. Measured
// with the two alternating in one process, 40-45 launches back to back each (the clock then
// settles lower under the larger LDS traffic): projection bf16 1151 against 1134 TFLOP/s,
// 8192^3 1203 against 1181, 4096^3 1031 against 1041; in short bursts, before the clock
// settles, the projection gains 7%. 4 waves of 128 x 128 were slower everywhere (4-30%).
using D16L64 = Direct16<256, 256, 64, 64, 64, 2>;
using D16M = Direct16<128, 128, 64, 64, 32, 4>;
using D16M64 = Direct16<128, 128, 64, 64, 64, 2>;
// 8 waves of 64 x 32 in one group, four stages: two waves per SIMD without splitting the
// K-steps (the two-group tile, config 10, shares each barrier between groups that cannot
// read early). Against config 10, same process: 2048^3 730 against 708 TFLOP/s,
// 4096 x 1024 x 4096 851 against 852 (fp16 831 against 802), 1000 x 4000 x 3000 716 against
// 660; against the 64 x 64 tile at 1536^3 481 against 466. With 2 stages 659 at 2048^3.
using D16M64w8 = Direct16<128, 128, 64, 32, 64, 4>;
using D16M32w8 = Direct16<128, 128, 64, 32, 32, 8>;
using D16S = Direct16<64, 64, 32, 32, 32, 4>;
using D16S64 = Direct16<64, 64, 32, 32, 64, 2>;
// deeper rings for the smaller tiles
using D16M32s8 = Direct16<128, 128, 64, 64, 32, 8>;
using D16M64s4 = Direct16<128, 128, 64, 64, 64, 4>;
using D16S32s8 = Direct16<64, 64, 32, 32, 32, 8>;
using D16S64s4 = Direct16<64, 64, 32, 32, 64, 4>;

struct Config16 {
    const char *name;
    hipError_t (*launch)(bool, const Gemm16Args &, hipStream_t);
};

template <class T>
hipError_t staged16(bool bf16, const Gemm16Args &a, hipStream_t stream)
{
    return bf16 ? launch16<T, true>(a, stream) : launch16<T, false>(a, stream);
}

template <class T32, class T64, class TS, int KG = 1>
hipError_t direct16(bool bf16, const Gemm16Args &a, hipStream_t stream)
{
    return launch16_direct_k<T32, T64, TS, KG>(bf16, a, stream);
}

const Config16 kConfigs16[] = {
    {"256x256x64 w128x64 pf1 (8 waves)", &staged16<T16L>},
    {"128x128x64 w64x64 pf1 (4 waves)", &staged16<T16M>},
    {"64x64x64 w32x32 pf1 (4 waves)", &staged16<T16S>},
    {"128x128x64 w64x64 pf2 (4 waves)", &staged16<T16Mp2>},
    {"64x64x64 w32x32 pf2 (4 waves)", &staged16<T16Sp2>},
    {"256x256x64 w64x64 direct-to-LDS 2 stages (16 waves; K < 64: K-steps of 32, 4 stages, 8 waves of 128x64)",
     &direct16<D16L, D16L64, T16L>},
    {"128x128x64 w64x64 direct-to-LDS 2 stages (4 waves; K < 64: K-steps of 32, 4 stages)",
     &direct16<D16M, D16M64, T16Mp2>},
    {"64x64x64 w32x32 direct-to-LDS 2 stages (4 waves; K < 64: K-steps of 32, 4 stages)",
     &direct16<D16S, D16S64, T16Sp2>},
    {"128x128x64 w64x64 direct-to-LDS 4 stages (4 waves; K < 64: K-steps of 32, 8 stages)",
     &direct16<D16M32s8, D16M64s4, T16Mp2>},
    {"64x64x64 w32x32 direct-to-LDS 4 stages (4 waves; K < 64: K-steps of 32, 8 stages)",
     &direct16<D16S32s8, D16S64s4, T16Sp2>},
    {"128x128x64 w64x64 direct-to-LDS 2 stages, K over 2 wave groups (8 waves; K < 64: K-steps of 32, 4 stages)",
     &direct16<D16M, D16M64, T16Mp2, 2>},
    {"128x128x64 w64x32 direct-to-LDS 4 stages (8 waves; K < 64: K-steps of 32, 8 stages)",
     &direct16<D16M32w8, D16M64w8, T16Mp2>},
};
constexpr int kNumConfigs16 = sizeof(kConfigs16) / sizeof(kConfigs16[0]);

}  // namespace

int gemm16_num_configs() { return kNumConfigs16; }

const char *gemm16_config_name(int cfg)
{
    return (cfg >= 0 && cfg < kNumConfigs16) ? kConfigs16[cfg].name : nullptr;
}

int gemm16_select_config(int64_t M, int64_t N, int64_t K)
{
    (void)K;
    // The direct pipelines (5 .. 11); on shapes they cannot take they run the register-
    // staged tile of their size. From the timed sweep of every config (bf16 and fp16,
    // 128^3 .. 8192^3, the projection and ragged shapes): the 256 x 256 tile from 144 tiles
    // on (3072^3: 788 TFLOP/s against 718 on 128 x 128); with fewer, the 128 x 128 tile on 8
    // waves of 64 x 32 from 144 tiles of 128^2 on (2048^3: 730; 4096 x 1024 x 4096: 851;
    // 1536^3: 481 against 466 on 64 x 64); below that the 64 x 64 tile, four stages deep
    // where at most two workgroups per CU are needed (1024^3: 334; 1000 x 1531 x 777: 208
    // against 193 with two stages), else two stages, which fit three workgroups per CU.
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    if (t256 >= 144) return 5;
    if (t128 >= 144) return 11;
    return t64 > 512 ? 7 : 9;
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
    if (cfg < 0 || cfg >= kNumConfigs16) return hipErrorInvalidValue;
    return kConfigs16[cfg].launch(bf16, a, stream);
}

}  // namespace mm
