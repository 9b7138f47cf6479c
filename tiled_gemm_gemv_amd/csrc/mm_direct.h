// mm_direct.h -- building blocks of the fp32 tiles whose panels the LDS DMA moves from
// HBM straight into LDS (the GEMM of mm_gemm_direct.hip and the convolution of
// mm_conv.hip): tile parameters, the LDS layout's permutations, the DMA and wait
// primitives, and the MFMA step on one stage.
//
// LDS layout of a stage (BK = 16, 32 or 64 k per K-step; 64 in the convolution only):
//   * A panel: BM rows of 4 BK bytes. The 16-byte chunk c of row r sits in slot
//     c ^ swz_a(r), so that a wave's reads of 32 rows at one k hit distinct banks; each
//     lane reads 4 consecutive k of its row with one 16-byte read.
//   * B panel: BK rows of BN floats, row-major. v_mfma_f32_32x32x2_f32 takes one B value
//     per lane per step, so a lane reads its column's value of the step's k row with a
//     4-byte read; rows r and r + BK/2 (read by the two wave halves at once) are put on
//     opposite halves of the banks by swz_b (chunk index ^ 8).
//   * k order: lanes 0-31 take k = 4 q + j and lanes 32-63 k = BK/2 + 4 q + j at step j
//     of group q (q < BK/8), so each k of the K-step is added once, in the order of the
//     register-staged kernel with the same BK (the same bits).
//   * Tiles on v_mfma_f32_16x16x4_f32 (M16): lane group g = lane / 16 takes k = (BK/4) g + t
//     at MFMA step t, so one 16-byte read of A still serves 4 steps; the four groups read B
//     rows r + g BK/4 at once, and swz_b puts groups 0/1 (and 2/3) on opposite bank halves
//     (chunk index ^ 8, which keeps each 128-byte line of B whole in the DMA).
// BK = 32 makes each A row of a K-step one whole 128-byte line (at BK = 16 a load of A
// touches 16 half-used lines, and the DMA's LDS writes of those rows count bank-conflict
// cycles) and doubles the MFMAs per barrier; with half the stages in the same LDS it
// measured 0.9% faster on the 256 x 256 tile and 1-8% on the 128 x 128 and 64 x 64 ones.
#pragma once
#include "mm_gemm_tile.h"

namespace mm {
namespace {

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) float lds_float;

// GEN: every shape (4-byte lanes where needed); otherwise K % 16 == 0 and N % 4 == 0 only
// (direct_f32_wide_ok), which keeps the narrow-lane code out of the kernel.
// KS: wave groups that split each K-step's k groups (KS = 2: 8 waves on a 4-wave tile grid;
// group g multiplies groups g QN / 2 .. of every step, and the two sums meet in LDS).
// M16: the MFMA is v_mfma_f32_16x16x4_f32 (8 passes) instead of v_mfma_f32_32x32x2_f32 (16
// passes). Both reach ~155 TFLOP/s when independent MFMAs are issued back to back; in the
// 128 x 128 tile the shorter instruction raised the matrix cores' busy share from 0.938 to
// 0.945 (its LDS reads and waits interleave with the MFMAs at a finer grain).
template <int BM_, int BN_, int WM_, int WN_, int NS_, bool GEN_, int BK_ = 16, int KS_ = 1, bool M16_ = false>
struct DirectF32 {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, NS = NS_, WM = WM_, WN = WN_, KS = KS_;
    static constexpr bool M16 = M16_;
    static constexpr int QN = BK / 8;      // groups of 4 k per wave half and K-step
    static constexpr int QW = QN / KS;     // ... that one wave multiplies
    static constexpr int TQ = BK / 4;      // M16: MFMA steps per K-step
    static constexpr int A_ROW = BK * 4;   // bytes per A row
    static constexpr bool GEN = GEN_;
    static constexpr int GRID = (BM / WM) * (BN / WN);  // waves of the tile's wave grid
    static constexpr int WAVES = GRID * KS, NT = WAVES * 64;
    static constexpr int MB = M16 ? 16 : 32;  // edge of an MFMA block
    static constexpr int FM = WM / MB, FN = WN / MB;
    static constexpr int ACC = MB * MB / 64;  // accumulator registers per block and lane
    typedef float Acc __attribute__((ext_vector_type(ACC)));
    static constexpr int A_BYTES = BM * BK * 4, B_BYTES = BK * BN * 4;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int B_ROW = BN * 4;  // bytes per B row
    // loads per wave per K-step with 16-byte (1 KB per wave) and 4-byte lanes (256 B)
    static constexpr int A16 = A_BYTES / 1024 / WAVES, B16 = B_BYTES / 1024 / WAVES;
    static constexpr int A4 = A_BYTES / 256 / WAVES, B4 = B_BYTES / 256 / WAVES;
    static constexpr int LOADS_WIDE = A16 + B16, LOADS_NARROW_B = A16 + B4;
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "whole loads");
    static_assert(B_ROW >= 256 && B_ROW <= 1024, "B rows of 64 to 256 floats");
    static_assert(NS * STAGE <= 160 * 1024, "stages must fit the 160 KB LDS");
    static_assert((NS - 2) * LOADS_NARROW_B <= 63, "vmcnt range");
    static_assert(BK == 16 || ((BK == 32 || BK == 64) && !GEN), "BK of 32 or 64 only for the lean build");
    static_assert(KS == 1 || (KS == 2 && !GEN && QN % 2 == 0), "K-step groups split in two only in the lean build");
    static_assert(!M16 || KS == 1, "the 16 x 16 MFMA tiles run each K-step in one wave group");
};

// Rows of 64 bytes: two rows per 128 bytes of banks. Rows of 128 bytes: the 8 chunk slots
// of any 8 (or, on 64 banks, 16) consecutive rows read at one k are distinct. Rows of 256
// bytes (every bank): the 16 slots of any 16 consecutive rows are distinct.
template <class T>
__device__ __forceinline__ int swz_a(int row)
{
    if constexpr (T::BK == 16) return ((row >> 1) ^ (row >> 3)) & 3;
    else if constexpr (T::BK == 32) return ((row >> 1) & 7) ^ ((row & 1) << 2);
    else return row & 15;  // rows of 256 bytes: any 16 consecutive rows, 16 distinct slots
}
// B rows: with 32 x 32 MFMAs the wave halves read rows r and r + BK/2 at once, put on
// opposite halves of the banks; with 16 x 16 MFMAs the four lane groups read rows
// r + g BK/4, put on the four quarters (16 consecutive columns of a row span 64 bytes).
template <class T>
__device__ __forceinline__ int swz_b(int krow)
{
    if constexpr (T::M16) return ((krow / (T::BK / 4)) & 1) * 8;
    else return ((krow / (T::BK / 2)) & 1) * 8;
}

// VEC bytes per lane from src into LDS at lds_addr + VEC * lane (lds_addr wave-uniform).
// The LDS address travels in M0 as an operand of the asm statement ("{m0}"), so the
// compiler writes M0 itself right before each load and knows the load reads it. A global
// load with LDS = 1 that reads M0 needs one wait state after the SALU write of M0 (CDNA's
// table of manually inserted wait states); the hazard recognizer does not look inside an
// asm string, so the s_nop is written at its start (the compiler's own builtin leaves at
// least one instruction there too).
template <int VEC>
__device__ __forceinline__ void load_to_lds(unsigned lds_addr, const float *src)
{
    if constexpr (VEC == 16)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     :: "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off"
                     :: "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

// 16 bytes per lane from base + voff into LDS at lds_addr + 16 * lane: base and lds_addr
// wave-uniform (scalar registers), voff the lane's byte offset. With the base stepped by
// scalar arithmetic and fixed lane offsets, a load takes no vector instruction (the
// pointer form above needs a 64-bit address add and a readfirstlane per load; measured
// 1.7% of the 256 x 256 tile's time at the projection shape).
__device__ __forceinline__ void load_to_lds_s16(unsigned lds_addr, const float *base, unsigned voff)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
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

// A lane's operand addresses inside a stage (bytes), fixed for the whole K loop.
//   32 x 32 MFMAs: A per group q and block i; B per group q, step j and block jj
//     (k = (BK / 2) (lane / 32) + 4 q + j, column wn0 + 32 jj + lane % 32).
//   16 x 16 MFMAs: lane group g = lane / 16 takes k = (BK / 4) g + t at MFMA step t, so a
//     16-byte read of A gives 4 steps (a[u][i]: steps 4u .. 4u + 3 of row block i, row
//     wm0 + 16 i + lane % 16), and B's value for step t and column block jj sits at
//     b[jj] + t B_ROW (column wn0 + 16 jj + lane % 16).
template <class T, bool = T::M16>
struct DirectOffsets {
    int a[T::QW][T::FM];
    int b[T::QW][4][T::FN];
};
template <class T>
struct DirectOffsets<T, true> {
    int a[T::TQ / 4][T::FM];
    int b[T::FN];
};

template <class T>
__device__ __forceinline__ void direct_operand_offsets(int lane, int wm0, int wn0, int (&a_off)[T::QW][T::FM],
                                                       int (&b_off)[T::QW][4][T::FN], int q0 = 0)
{
#pragma unroll
    for (int qq = 0; qq < T::QW; ++qq) {
        const int q = q0 + qq;
#pragma unroll
        for (int i = 0; i < T::FM; ++i) {
            const int row = wm0 + 32 * i + (lane & 31);
            a_off[qq][i] = row * T::A_ROW + 16 * ((q + T::QN * (lane >> 5)) ^ swz_a<T>(row));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int jj = 0; jj < T::FN; ++jj) {
                const int krow = (T::BK / 2) * (lane >> 5) + 4 * q + j;
                const int col = wn0 + 32 * jj + (lane & 31);
                b_off[qq][j][jj] = T::A_BYTES + krow * T::B_ROW + 16 * ((col >> 2) ^ swz_b<T>(krow)) +
                                   4 * (col & 3);
            }
    }
}

// For this wave's QW groups q = q0 + qq of each K-step (32 x 32 MFMAs), or all of its
// steps (16 x 16).
template <class T>
__device__ __forceinline__ void direct_offsets(int lane, int wm0, int wn0, DirectOffsets<T> &o, int q0 = 0)
{
    if constexpr (T::M16) {
        const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
        for (int u = 0; u < T::TQ / 4; ++u)
#pragma unroll
            for (int i = 0; i < T::FM; ++i) {
                const int row = wm0 + 16 * i + l16;
                o.a[u][i] = row * T::A_ROW + 16 * ((g * (T::TQ / 4) + u) ^ swz_a<T>(row));
            }
        const int krow = T::TQ * g;  // step 0's row; step t adds t B_ROW (same swizzle)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj) {
            const int col = wn0 + 16 * jj + l16;
            o.b[jj] = T::A_BYTES + krow * T::B_ROW + 16 * ((col >> 2) ^ swz_b<T>(krow)) + 4 * (col & 3);
        }
    } else {
        direct_operand_offsets<T>(lane, wm0, wn0, o.a, o.b, q0);
    }
}

// The MFMAs of one K-step on stage st: this wave's QW groups of 4 k per lane half.
template <class T>
__device__ __forceinline__ void direct_multiply(const lds_char *st, const int (&a_off)[T::QW][T::FM],
                                                const int (&b_off)[T::QW][4][T::FN], f32x16 (&acc)[T::FM][T::FN])
{
#pragma unroll
    for (int q = 0; q < T::QW; ++q) {
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
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][j], b[j][jj], acc[i][jj], 0, 0, 0);
    }
}

// The MFMAs of one K-step on stage st, either MFMA shape.
template <class T>
__device__ __forceinline__ void direct_mma(const lds_char *st, const DirectOffsets<T> &o,
                                           typename T::Acc (&acc)[T::FM][T::FN])
{
    if constexpr (T::M16) {
#pragma unroll
        for (int u = 0; u < T::TQ / 4; ++u) {
            f32x4 a[T::FM];
            float b[4][T::FN];
#pragma unroll
            for (int i = 0; i < T::FM; ++i)
                a[i] = *(const __attribute__((address_space(3))) f32x4 *)(st + o.a[u][i]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int jj = 0; jj < T::FN; ++jj)
                    b[t][jj] = *(const lds_float *)(st + o.b[jj] + (4 * u + t) * T::B_ROW);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < T::FM; ++i)
#pragma unroll
                    for (int jj = 0; jj < T::FN; ++jj)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][t], b[t][jj], acc[i][jj], 0, 0, 0);
        }
    } else {
        direct_multiply<T>(st, o.a, o.b, acc);
    }
}

// Accumulator layout of v_mfma_f32_32x32x2_f32: lane l, register r holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of the 32 x 32 block. The tile's columns
// start at nb0; element (gm, gn) of the product goes to C + gm * ldc + col_off(gn), for
// gm < M, gn < N and gn >= n_first (columns left of n_first belong to another tile).
// Of v_mfma_f32_16x16x4_f32: lane l, register r holds row 4 (l / 16) + r, column l % 16.
template <class T, class ColOff>
__device__ __forceinline__ void direct_store(const GemmArgs &p, int m0, int nb0, int n_first, int wm0, int wn0,
                                             int lane, const typename T::Acc (&acc)[T::FM][T::FN], ColOff col_off)
{
    if constexpr (T::M16) {
        const int col_l = lane & 15, row_l = 4 * (lane >> 4);
        int64_t coff[T::FN];
        bool cok[T::FN];
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj) {
            const int gn = nb0 + wn0 + jj * 16 + col_l;
            cok[jj] = gn < p.N && gn >= n_first;
            coff[jj] = cok[jj] ? col_off(gn) : 0;
        }
#pragma unroll
        for (int i = 0; i < T::FM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int gm = m0 + wm0 + i * 16 + row_l + r;
                if (gm >= p.M) continue;
#pragma unroll
                for (int jj = 0; jj < T::FN; ++jj)
                    if (cok[jj]) p.C[(int64_t)gm * p.ldc + coff[jj]] = acc[i][jj][r];
            }
        return;
    }
    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
    // a lane's column in each 32-column block, and its offset in C, once per block: inside
    // the guarded stores the compiler would evaluate col_off per element (for the
    // convolution's NKPQ scatter a division each: 16 per block, which on a filter of
    // 147 taps outweighed the tile's MFMAs)
    int64_t coff[T::FN];
    bool cok[T::FN];
#pragma unroll
    for (int jj = 0; jj < T::FN; ++jj) {
        const int gn = nb0 + wn0 + jj * 32 + col_l;
        cok[jj] = gn < p.N && gn >= n_first;
        coff[jj] = cok[jj] ? col_off(gn) : 0;
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                if (gm < p.M && cok[jj]) p.C[(int64_t)gm * p.ldc + coff[jj]] = acc[i][jj][r];
            }
}

// As direct_store, but adding each element to C with an atomic add (C + gm * ldc + gn):
// for two K halves of one product summed into a zeroed C, where the result does not
// depend on which half arrives first (0 + x is exact and x + y == y + x).
template <class T>
__device__ __forceinline__ void direct_store_add(const GemmArgs &p, int m0, int nb0, int n_first, int wm0, int wn0,
                                                 int lane, const typename T::Acc (&acc)[T::FM][T::FN])
{
    static_assert(!T::M16, "the atomic epilogue is built for the 32 x 32 MFMA tiles only");
    const int col_l = lane & 31, row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int gm = m0 + wm0 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
                const int gn = nb0 + wn0 + jj * 32 + col_l;
                if (gm < p.M && gn < p.N && gn >= n_first) atomicAdd(p.C + (int64_t)gm * p.ldc + gn, acc[i][jj][r]);
            }
}

}  // namespace
}  // namespace mm
