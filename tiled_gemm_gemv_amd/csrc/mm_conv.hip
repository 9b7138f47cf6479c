// mm_conv.hip -- fp32 2-D convolution as an implicit GEMM on the matrix-core tiles:
// the register-staged tiles of mm_gemm_tile.h and the direct-to-LDS tiles of mm_direct.h.
//
// The core of a convolutional layer can be recast as a matrix product, and im2col
// is the classic way to do so ("Matrix Operations", docs.vulkan.org ML-inference
// tutorial, Introduction; "GPU Matrix Multiplication: Tiling and Shared Memory",
// closing preview of the next lesson). With x an N x C x H x W batch, w a
// K x C x R x S filter bank and y the N x K x P x Q output (all packed, row-major),
//
//   y[n][k][p][q] = sum over c, r, s of w[k][c][r][s] * x[n][c][p sh + r dh - ph][q sw + s dw - pw]
//
// (x read as 0 outside the image) is the product of the K x CRS filter matrix --
// w exactly as stored, row k, column (c R + r) S + s -- with the CRS x NPQ im2col
// matrix, whose row (c, r, s) and column (n, p, q) hold that x element.
//
// The im2col matrix is never written to memory. The tiles stage it K-step by K-step
// like any B operand, but its loader computes every element's address in x, or a zero
// for the padding, as it goes: through registers on the register-staged tiles
// (Im2colOperands), by 4-byte LDS DMA lanes straight into the B panel on the direct
// ones (conv_direct_kernel); the C store scatters product column (n, p, q) to
// y[n][.][p][q]. The images are laid side by
// side along the product's columns (j = n P Q + p Q + q), so a batch of small
// feature maps still makes one wide product that fills the chip. Beyond reading w
// and x and writing y once, HBM traffic is only the x panels the L2 does not keep
// between the R S row-shifts that reuse them.
//
// A 1 x 1 filter with unit stride and no padding needs no gather: each image of x is
// then a C x HW matrix and the convolution is the strided batched GEMM of the same
// kernel with a plain B.
#include "mm_direct.h"

namespace mm {
namespace {

constexpr int kFar = -(1 << 30);  // an input row that is outside any image

// Read by the direct gather's LDS DMA, where it runs without tap masks, for every
// element of the product that is zero: a tap in the padding, a row past K (partial
// K-step) or a column past N.
__device__ float kZeros[64];

// B = the im2col matrix of a run of images of x (p.B points at the first), C = those
// images of y; p.N = images * P * Q, p.K = C * R * S, p.ldc = P * Q.
//
// Piece idx of a K-step is one column of the panel, col = idx % BN, at 16
// consecutive k rows from k0 + 16 (idx / BN). BN is a multiple of 64, so the 64
// lanes of a wave take 64 adjacent output positions at the same 16 rows: (c, r, s)
// and everything derived from them are the same in every lane (scalar registers),
// and at unit stride neighbouring lanes read neighbouring floats of x. Loads need no
// branch: an element outside the image reads x[0] and is replaced by zero.
//
// The host keeps a run of images below 2^30 elements (byte offsets fit in 32 bits)
// and the padded plane (H + 2 ph)(W + 2 pw) below 2^30, so every offset below fits
// in int32.
struct Im2colOperands {
    static constexpr bool kMatrixB = false;
    int H, W, R, S, sh, sw, ph, pw, dh, dw;
    int Q, PQ, HW, RS, CHW;
    int sK, rK, cK;  // one K-step (BK rows) of the im2col matrix: s += sK, r += rK, c += cK (with carries)
    int64_t KPQ;
    // the direct gather's tap-mask path (a run of x below 2^31 bytes): 0 if not taken, else
    // the mask words per column (1: R S <= 31, 2: R S <= 63), and the run's size in bytes
    // (the bound of its buffer loads)
    int tap_masks;
    unsigned run_bytes;
    // the tap-mask path's row table in LDS (K rounded up to whole K-steps, 8 bytes a row)
    int row_table;

    // Output column (n, p, q): input row h0 and column w0 under the filter's first
    // tap, and base = offset of x[n][0][h0][w0] (negative when in the padding).
    // Columns past the end get h0 = kFar.
    struct Cols {
        int h0, w0, base;
    };

    template <class T>
    __device__ __forceinline__ Cols columns(const GemmArgs &p, int n0, int idx) const
    {
        static_assert(T::BN % 64 == 0 && T::BK % 16 == 0, "a wave's lanes must share their rows");
        return columns_of(p, n0 + idx % T::BN);
    }

    // The state of output column j (any j; h0 = kFar past the end).
    __device__ __forceinline__ Cols columns_of(const GemmArgs &p, int j) const
    {
        Cols c;
        if (j < p.N) {
            const int n = (unsigned)j / (unsigned)PQ, pq = j - n * PQ;
            const int op = (unsigned)pq / (unsigned)Q, oq = pq - op * Q;
            c.h0 = op * sh - ph;
            c.w0 = oq * sw - pw;
            c.base = n * CHW + c.h0 * W + c.w0;
        } else {
            c.h0 = kFar;
            c.w0 = 0;
            c.base = 0;
        }
        return c;
    }

    template <class T, bool VEC>
    __device__ __forceinline__ void load_b(const GemmArgs &p, const Cols &cl, int k0, int, int idx,
                                           bool, f32x4 (&b)[4]) const
    {
        // first row of the piece: (c, r, s) by division once, then stepped
        const int gk0 = __builtin_amdgcn_readfirstlane(k0 + 16 * (idx / T::BN));
        const int c = gk0 / RS;  // channel of the first row
        const int rem = gk0 - c * RS;
        int r = rem / S;
        int s = rem - r * S;
        int dy = r * dh, dx = s * dw;
        int rowoff = c * HW + dy * W + dx;  // offset of (c, dy, dx) from (0, h0, w0)
        const char *x = reinterpret_cast<const char *>(p.B);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int h = cl.h0 + dy, w = cl.w0 + dx;
            const bool ok = (gk0 + i < p.K) && (unsigned)h < (unsigned)H && (unsigned)w < (unsigned)W;
            const unsigned off = ok ? (unsigned)(cl.base + rowoff) * 4u : 0u;
            const float v = *reinterpret_cast<const float *>(x + off);
            b[i >> 2][i & 3] = ok ? v : 0.f;
            // next row: s + 1, carrying into r and then c (uniform branches, mostly
            // not taken: cheaper here than selects evaluated on every row)
            dx += dw;
            rowoff += dw;
            if (++s == S) {
                s = 0;
                dx = 0;
                dy += dh;
                rowoff += dh * W - S * dw;
                if (++r == R) {
                    r = 0;
                    dy = 0;
                    rowoff += HW - R * dh * W;
                }
            }
        }
    }

    // b[j] holds k rows 4j .. 4j + 3 of the piece: one 16-byte LDS write each
    template <class T>
    __device__ __forceinline__ void store_b(float *Bs, int idx, const f32x4 (&b)[4]) const
    {
        float *dst = Bs + (idx % T::BN) * T::PITCH + 16 * (idx / T::BN);
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4 *>(dst + 4 * j) = b[j];
    }

    // Column (n, p, q) of the product is y[n][.][p][q]: image offset + p Q + q.
    __device__ __forceinline__ int64_t c_column(const GemmArgs &, int gn) const
    {
        const int n = (unsigned)gn / (unsigned)PQ;
        return (int64_t)n * KPQ + (gn - n * PQ);
    }
};

// The implicit GEMM on the direct-to-LDS tiles of mm_direct.h: filters (A) by 16-byte DMA
// lanes, the im2col matrix (B) gathered by 4-byte DMA lanes straight into the B panel.
// A lane of a B load lands at a fixed column of one k row of the panel, so it keeps that
// column's state (h0, w0, image offset) for the whole K loop; the row's (c, r, s) and
// offset are the same in every lane (scalar registers), found by one division per
// workgroup and stepped across the wave's ROWS consecutive rows. An element that is zero
// (padding, k >= K, column >= N) is read from kZeros, so a partial last K-step needs
// no clearing. A's partial step takes 4-byte lanes with the same rule.
// MASK (1 or 2 words): each lane also keeps, per column, a bit per filter tap r S + s that
// is set where the tap falls in the padding; the last bit of the last word (31 or 63, above
// every tap) is always set and stands for the rows past K. A B element is then read by a
// buffer load of x (the run's size as the bound) at byte offset (column base + row offset)
// * 4, or at 2^31 for a padded tap or a row past K: that offset is beyond the run (runs are
// kept below 2^31 bytes), so the load returns 0. Three vector instructions per element
// (shift-add, bit extract, bit select; one more, the word select, with two words) instead
// of the bounds tests and a 64-bit pointer select.
// TABLE (with MASK): the row offset and tap of every k come from a table the workgroup
// writes into LDS before its first load, one wave-uniform LDS read per row instead of the
// scalar stepping.
template <class T, int MASK, bool TABLE>
__global__ __launch_bounds__(T::NT) void conv_direct_kernel(GemmArgs p, Im2colOperands o)
{
    static_assert(MASK > 0 || !TABLE, "the row table feeds the tap-mask path");
    static_assert(T::KS == 1, "one wave group per K-step");
    static_assert(MASK >= 0 && MASK <= 2, "one or two mask words");
    constexpr int kPastK = MASK == 2 ? 63 : 31;  // the mask bit of a row past K
    static_assert(T::B_ROW <= 1024 && (T::B4 * 256) % T::B_ROW == 0, "a wave's B loads cover whole rows");
    constexpr int ROWS = T::B4 * 256 / T::B_ROW;      // k rows of a K-step one wave loads
    constexpr int PER_ROW = T::B_ROW / 256;           // loads per row
    static_assert(ROWS * T::WAVES == T::BK, "the waves split the k rows");
    __shared__ __attribute__((aligned(1024))) char lds[T::NS * T::STAGE];
    const int tiles_m = (p.M + T::BM - 1) / T::BM;
    const int tiles_n = (p.N + T::BN - 1) / T::BN;
    const int64_t tiles = (int64_t)tiles_m * tiles_n;
    const int64_t bid = linear_block();
    if (bid >= tiles) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    int tm, tn;
    tile_of_block((int)bid, (int)tiles, tiles_m, tiles_n, 8, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int lane = threadIdx.x & 63;
    // the wave index in a scalar register: the rows a wave gathers, their (c, r, s) and
    // offsets, and the branches that step them are then scalar work
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm0 = (w / (T::BN / T::WN)) * T::WM, wn0 = (w % (T::BN / T::WN)) * T::WN;
    const int nk = (p.K + T::BK - 1) / T::BK;
    const float *zeros = kZeros + lane;
    const char *x = reinterpret_cast<const char *>(p.B);
    // TABLE: per im2col row k, its offset in x from the column's base and its filter tap
    // (kPastK past K: the tap masks' always-set bit), built once per workgroup
    extern __shared__ int2 ktab[];
    if constexpr (TABLE) {
        for (int e = threadIdx.x; e < nk * T::BK; e += T::NT) {
            int2 t = {0, kPastK};
            if (e < p.K) {
                const int c = e / o.RS, rs = e - c * o.RS, r = rs / o.S, s = rs - r * o.S;
                t.x = c * o.HW + r * o.dh * o.W + s * o.dw;
                t.y = rs;
            }
            ktab[e] = t;
        }
        __syncthreads();
    }

    // A: 16-byte lanes on full K-steps (sources at k0 = 0)
    const float *asrc[T::A16];
#pragma unroll
    for (int i = 0; i < T::A16; ++i) {
        const int ob = (T::A16 * w + i) * 1024 + 16 * lane;
        const int row = ob / T::A_ROW, chunk = (ob % T::A_ROW) / 16;
        asrc[i] = p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + 4 * (chunk ^ swz_a<T>(row));
    }
    // B: the wave loads rows ROWS * w .. ROWS * w + ROWS - 1 of each K-step, PER_ROW loads
    // per row; this lane's column in load h of a row, and that column's state
    const int krow0 = ROWS * w;
    Im2colOperands::Cols cols[PER_ROW];
#pragma unroll
    for (int h = 0; h < PER_ROW; ++h) {
        const int slot = 64 * h + lane;  // 4-byte slot in the row
        const int col = n0 + 4 * ((slot >> 2) ^ swz_b<T>(krow0)) + (slot & 3);
        cols[h] = o.columns_of(p, col);
    }
    static_assert((T::BK / 2) % ROWS == 0, "a wave's rows lie in one half of the K-step: they share swz_b");
    // the tap-mask path: per column, bit r S + s set where that tap is in the padding (or the
    // column is past N), and the column's base offset in bytes
    unsigned pad_lo[PER_ROW], pad_hi[PER_ROW], base4[PER_ROW];
    __amdgpu_buffer_rsrc_t xrsrc;
    if constexpr (MASK > 0) {
        xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.B), (short)0, (int)o.run_bytes, 0x00020000);
        // tap (r, s) is in the padding when its filter row r or its filter column s is:
        // the mask is the S bits of the padded columns, or all S bits for a padded row,
        // at r S for each r (R + S steps rather than R S)
        const uint64_t full_row = (uint64_t(1) << o.S) - 1;  // S <= 63
#pragma unroll
        for (int h = 0; h < PER_ROW; ++h) {
            uint64_t col_pad = 0;
            for (int ss = 0; ss < o.S; ++ss)
                if ((unsigned)(cols[h].w0 + ss * o.dw) >= (unsigned)o.W) col_pad |= uint64_t(1) << ss;
            uint64_t m = uint64_t(1) << kPastK;
            for (int r = 0; r < o.R; ++r) {
                const bool hin = (unsigned)(cols[h].h0 + r * o.dh) < (unsigned)o.H;
                m |= (hin ? col_pad : full_row) << (r * o.S);
            }
            pad_lo[h] = (unsigned)m;
            pad_hi[h] = (unsigned)(m >> 32);
            base4[h] = (unsigned)cols[h].base * 4u;
        }
    }
    // all ones where tap `bit` of column h is in the padding (or the row is past K), else 0
    auto pad_of = [&](int h, int bit) -> unsigned {
        unsigned word = pad_lo[h];
        if constexpr (MASK == 2) word = bit < 32 ? pad_lo[h] : pad_hi[h];
        return (unsigned)__builtin_amdgcn_sbfe((int)word, bit & 31, 1);
    };

    const unsigned lds0 = (unsigned)(uintptr_t)(lds_char *)lds;
    // (c, r, s) of row krow0 of the next K-step to issue (one division, here)
    int fc = krow0 / o.RS, fr = (krow0 - fc * o.RS) / o.S;
    int fs = krow0 - fc * o.RS - fr * o.S;
    auto issue = [&](int kt) {
        const unsigned st = lds0 + (kt % T::NS) * T::STAGE;
        const int k0 = kt * T::BK;
        if (k0 + T::BK <= p.K) {
#pragma unroll
            for (int i = 0; i < T::A16; ++i) load_to_lds<16>(st + (T::A16 * w + i) * 1024, asrc[i] + k0);
        } else {
#pragma unroll
            for (int i = 0; i < T::A4; ++i) {
                const int ob = (T::A4 * w + i) * 256 + 4 * lane;
                const int row = ob / T::A_ROW, slot = (ob % T::A_ROW) / 4;
                const int k = k0 + 4 * ((slot >> 2) ^ swz_a<T>(row)) + (slot & 3);
                const float *src = k < p.K ? p.A + (int64_t)min(m0 + row, p.M - 1) * p.lda + k : zeros;
                load_to_lds<4>(st + (T::A4 * w + i) * 256, src);
            }
        }
        if constexpr (TABLE) {
#pragma unroll
            for (int rr = 0; rr < ROWS; ++rr) {
                const int2 t = ktab[k0 + krow0 + rr];
#pragma unroll
                for (int h = 0; h < PER_ROW; ++h) {
                    const unsigned dst = st + T::A_BYTES + (krow0 + rr) * T::B_ROW + 256 * h;
                    const unsigned pad = pad_of(h, t.y);
                    const unsigned v = base4[h] + (unsigned)t.x * 4u;
                    const unsigned off = (pad & 0x80000000u) | (~pad & v);
                    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                                 :: "v"(off), "s"(xrsrc), "{m0}"(dst) : "memory");
                }
            }
            return;
        }
        // (c, r, s) of the wave's first row: carried over from the previous issue (the
        // steps are issued in order), then stepped across the wave's rows
        int k = k0 + krow0;
        int r = fr, s = fs;
        int dy = r * o.dh, dx = s * o.dw;
        int rowoff = fc * o.HW + dy * o.W + dx;
        // advance the first row by one K-step (BK rows) for the next issue
        fs += o.sK;
        const int cs = fs >= o.S;
        fs -= cs ? o.S : 0;
        fr += o.rK + cs;
        const int cr = fr >= o.R;
        fr -= cr ? o.R : 0;
        fc += o.cK + cr;
        int tap = r * o.S + s;  // the row's filter tap (scalar)
#pragma unroll
        for (int rr = 0; rr < ROWS; ++rr) {
#pragma unroll
            for (int h = 0; h < PER_ROW; ++h) {
                const unsigned dst = st + T::A_BYTES + (krow0 + rr) * T::B_ROW + 256 * h;
                if constexpr (MASK > 0) {
                    // a padded tap or a row past K (bit kPastK) reads at 2^31, past the run
                    const int bit = k < p.K ? tap : kPastK;
                    const unsigned pad = pad_of(h, bit);
                    const unsigned v = base4[h] + (unsigned)rowoff * 4u;
                    const unsigned off = (pad & 0x80000000u) | (~pad & v);
                    asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                                 :: "v"(off), "s"(xrsrc), "{m0}"(dst) : "memory");
                } else {
                    const int hh = cols[h].h0 + dy, ww = cols[h].w0 + dx;
                    const bool ok = k < p.K && (unsigned)hh < (unsigned)o.H && (unsigned)ww < (unsigned)o.W;
                    const float *src = ok ? reinterpret_cast<const float *>(x + (unsigned)(cols[h].base + rowoff) * 4u)
                                          : zeros;
                    load_to_lds<4>(dst, src);
                }
            }
            ++tap;
            ++k;
            dx += o.dw;
            rowoff += o.dw;
            if (++s == o.S) {
                s = 0;
                dx = 0;
                dy += o.dh;
                rowoff += o.dh * o.W - o.S * o.dw;
                if (++r == o.R) {
                    r = 0;
                    dy = 0;
                    tap = 0;
                    rowoff += o.HW - o.R * o.dh * o.W;
                }
            }
        }
    };

    DirectOffsets<T> off;
    direct_offsets<T>(lane, wm0, wn0, off);
    typename T::Acc acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < T::FN; ++jj)
#pragma unroll
            for (int r = 0; r < T::ACC; ++r) acc[i][jj][r] = 0.f;

    // loads per wave per K-step (a partial step issues more: the count is then conservative)
    constexpr int L = T::A16 + T::B4;
    static_assert((T::NS - 2) * L <= 63, "vmcnt range");
    // The step NS - 1 ahead goes into the stage read in the previous step, free once every
    // wave is past the barrier. With two waves per SIMD it is issued before this step's
    // MFMAs, which then cover its latency while the other wave fills the matrix core (3 x 3
    // layers +2-6%); with one, the MFMAs go first and the gather's address work runs
    // while they execute (the 64 x 64 tile on the 3 x 3 layer: 70.3 against 68.3).
    constexpr bool kIssueFirst = T::WAVES >= 8;
    for (int st = 0; st < T::NS - 1 && st < nk; ++st) issue(st);
    for (int kt = 0; kt < nk; ++kt) {
        wait_steps<L, T::NS - 2>(nk - 1 - kt);
        __syncthreads();
        if (kIssueFirst && kt + T::NS - 1 < nk) issue(kt + T::NS - 1);
        direct_mma<T>((const lds_char *)lds + (kt % T::NS) * T::STAGE, off, acc);
        if (!kIssueFirst && kt + T::NS - 1 < nk) issue(kt + T::NS - 1);
    }
    direct_store<T>(p, m0, n0, n0, wm0, wn0, lane, acc, [&](int gn) { return o.c_column(p, gn); });
}

template <class T>
hipError_t launch_conv_direct(const GemmArgs &a, const Im2colOperands &o, hipStream_t stream)
{
    const int64_t tiles = (int64_t)((a.M + T::BM - 1) / T::BM) * ((a.N + T::BN - 1) / T::BN);
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    unsigned gx, gy;
    if (!grid_for(tiles, gx, gy)) return hipErrorInvalidConfiguration;
    GemmArgs ga = a;
    Im2colOperands oa = o;
    void *args[] = {&ga, &oa};
    const void *fn = o.tap_masks == 0 ? reinterpret_cast<const void *>(&conv_direct_kernel<T, 0, false>)
                     : o.tap_masks == 1
                         ? (o.row_table ? reinterpret_cast<const void *>(&conv_direct_kernel<T, 1, true>)
                                        : reinterpret_cast<const void *>(&conv_direct_kernel<T, 1, false>))
                         : (o.row_table ? reinterpret_cast<const void *>(&conv_direct_kernel<T, 2, true>)
                                        : reinterpret_cast<const void *>(&conv_direct_kernel<T, 2, false>));
    const size_t table = o.row_table ? (size_t)((a.K + T::BK - 1) / T::BK) * T::BK * 8 : 0;
    return hipLaunchKernel(fn, dim3(gx, gy), dim3(T::NT), args, table, stream);
}

struct ConvConfig {
    const char *name;
    hipError_t (*launch)(const GemmArgs &, const Im2colOperands &, hipStream_t);
    int gemm_cfg;       // the same tile shape as a GEMM config (used for 1 x 1 filters)
    int bm, bn;
    int waves;          // per workgroup
    int wg_per_cu;      // workgroups one CU holds (registers and LDS)
    double tflops;      // rate of the tile on the gather, for the choice below
    int bk;             // K-step depth
    bool direct = false;  // the direct-to-LDS gather (conv_direct_kernel)
    double fill_waves = 8;  // waves per CU at which the tile reaches its rate
    bool row_table = false; // the tap-mask gather reads its rows' offsets from an LDS table
};

template <class T>
hipError_t launch_im2col(const GemmArgs &a, const Im2colOperands &o, hipStream_t stream)
{
    return launch_tile_ops<T>(a, o, stream);
}

// Tile shapes of the fp32 GEMM. The 256 x 256 tile is left out: with the gather's
// per-column state it no longer fits its 256 registers per lane. Rates: fitted to a timed
// sweep of image-network layers (3 x 3 at strides 1 and 2, dilated 3 x 3, 7 x 7 input
// layer), gather included.
const ConvConfig kConvConfigs[] = {
    {"128x128x32 w64x64 pf2 ks1 (4 waves)", &launch_im2col<T128x128k32p2>, 1, 128, 128, 4, 2, 100, 32},
    {"128x128x32 w64x64 pf1 ks2 (8 waves)", &launch_im2col<T128x128k32s2>, 2, 128, 128, 8, 1, 100, 32},
    {"64x64x64 w32x32 pf2 ks1 (4 waves)", &launch_im2col<T64x64k64p2>, 3, 64, 64, 4, 2, 90, 64},
    {"64x64x64 w32x32 pf2 ks2 (8 waves)", &launch_im2col<T64x64k64p2s2>, 4, 64, 64, 8, 2, 86, 64},
    {"128x64x64 w64x32 pf1 ks2 (8 waves)", &launch_im2col<T128x64k64s2>, 5, 128, 64, 8, 1, 80, 64},
    // The direct gather (timed on the tap-mask path, TFLOP/s). 64 x 64: K-steps of 32 in 2
    // stages (5 workgroups per CU) beat 16 in 4 stages (dilated 3 x 3 layer 70.0 against
    // 65.4, 3 x 3 70.2 against 68.7). 128 x 128 and 64 x 128 on 8 waves (wave tiles of
    // 64 x 32 and 32 x 32, two waves per SIMD) beat 4 waves: 3 x 3 layer 79.4 against 73.1,
    // 3 x 3 at 256 filters 85.4 against 83.0, dilated 3 x 3 (64 filters: 256 tiles of
    // 64 x 128) 74.0. The 128 x 128 tiles: K-steps of 32 in 2 stages where a CU holds one
    // workgroup (196 tiles), 16 in 4 stages (fill_waves 16) where it holds two.
    {"64x64x32 w32x32 direct-to-LDS gather 2 stages (4 waves)",
     &launch_conv_direct<DirectF32<64, 64, 32, 32, 2, false, 32>>, 13, 64, 64, 4, 5, 95, 32, true, 4},
    {"128x128x16 w64x32 direct-to-LDS gather 4 stages (8 waves)",
     &launch_conv_direct<DirectF32<128, 128, 64, 32, 4, false>>, 11, 128, 128, 8, 2, 122, 16, true, 16, true},
    {"128x128x32 w64x32 direct-to-LDS gather 2 stages (8 waves)",
     &launch_conv_direct<DirectF32<128, 128, 64, 32, 2, false, 32>>, 11, 128, 128, 8, 2, 120, 32, true, 8, true},
    {"64x128x32 w32x32 direct-to-LDS gather 2 stages (8 waves)",
     &launch_conv_direct<DirectF32<64, 128, 32, 32, 2, false, 32>>, 13, 64, 128, 8, 3, 105, 32, true, 8, true},
    // K-steps of 64 (96 KB of LDS: one workgroup per CU) for layers of about one 64 x 128 tile
    // per CU: twice the MFMAs per barrier and per gather issue. Dilated 3 x 3 layer (256
    // tiles) 82.0 against 78.9; the 128 x 128 tile gains nothing from them (82.1 against
    // 83.1 on the 3 x 3 layer).
    {"64x128x64 w32x32 direct-to-LDS gather 2 stages (8 waves)",
     &launch_conv_direct<DirectF32<64, 128, 32, 32, 2, false, 64>>, 13, 64, 128, 8, 1, 110, 64, true, 8, true},
};
constexpr int kNumConvConfigs = sizeof(kConvConfigs) / sizeof(kConvConfigs[0]);
constexpr int64_t kMaxI32 = 0x7fffffff;
constexpr int64_t kMaxRun = (int64_t(1) << 30) - 1;      // elements of x per launch
constexpr int64_t kMaxMaskRun = (int64_t(1) << 29) - 1;  // ... with the direct gather's tap masks
constexpr int64_t kMaxRowTable = 16 * 1024;                // bytes of LDS for the row table

}  // namespace

int conv_num_configs() { return kNumConvConfigs; }

const char *conv_config_name(int cfg)
{
    return (cfg >= 0 && cfg < kNumConvConfigs) ? kConvConfigs[cfg].name : nullptr;
}

// The product is M = K filters by N columns by CRS. Filter counts are often 64-256, so a
// tall tile can be mostly padding, and CRS is often small, so a deep K-step can be mostly
// padding too; the choice is the least modelled time (tile_time: padded tile area, the
// busiest CU's tiles and its occupancy, the tile's rate on the gather; k_steps_factor).
int conv_select_config(int64_t M, int64_t N, int64_t K)
{
    int best = 0;
    double best_t = 0;
    for (int c = 0; c < kNumConvConfigs; ++c) {
        const ConvConfig &k = kConvConfigs[c];
        const int64_t tiles = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn);
        const double t = tile_time(tiles, k.bm, k.bn, k.waves, k.wg_per_cu, k.tflops, k.fill_waves) *
                         k_steps_factor(K, k.bk);
        if (c == 0 || t < best_t) {
            best = c;
            best_t = t;
        }
    }
    return best;
}

// 1 x 1 layers on large maps run the batched GEMM: the config whose GEMM tile the GEMM's
// own model times fastest.
int conv_select_batched_gemm(int64_t M, int64_t N, int64_t K, int64_t batch)
{
    int best = 0;
    double best_t = 0;
    for (int c = 0; c < kNumConvConfigs; ++c) {
        const double t = gemm_config_time(kConvConfigs[c].gemm_cfg, M, N, K, batch);
        if (c == 0 || t < best_t) {
            best = c;
            best_t = t;
        }
    }
    return best;
}

// 1 x 1 filters, unit stride, no padding, feature maps large enough that per-image
// products waste little of their last tile: y[n] (K x HW) = w (K x C) x[n] (C x HW),
// the images as one strided batch of the plain GEMM.
bool conv_is_batched_gemm(const ConvArgs &a)
{
    return a.R == 1 && a.S == 1 && a.sh == 1 && a.sw == 1 && a.ph == 0 && a.pw == 0 &&
           a.H * a.W >= 1024;
}

int conv_choose_config(const ConvArgs &a)
{
    if (conv_is_batched_gemm(a)) return conv_select_batched_gemm(a.K, a.H * a.W, a.C, a.N < 65535 ? a.N : 65535);
    return conv_select_config(a.K, a.N * a.P * a.Q, a.C * a.R * a.S);
}

// Shapes are validated by the caller: N, K, P, Q >= 1, P and Q as the definition gives
// them, and the limits stated for Im2colOperands. C, H or W may be 0: every tap of the
// sum then reads padding (or there is none), so y is zeroed.
hipError_t conv_launch(int cfg, const ConvArgs &a, hipStream_t stream)
{
    const int64_t PQ = a.P * a.Q, HW = a.H * a.W, CHW = a.C * HW, KPQ = a.K * PQ;
    if (CHW == 0) return zero_fill_launch(a.y, a.N * a.K, PQ, PQ, stream);

    if (cfg < 0) cfg = conv_choose_config(a);
    if (conv_is_batched_gemm(a)) {
        const int gcfg = kConvConfigs[cfg].gemm_cfg;
        for (int64_t n0 = 0; n0 < a.N; n0 += 65535) {
            GemmArgs g;
            g.A = a.w;
            g.B = a.x + n0 * CHW;
            g.C = a.y + n0 * KPQ;
            g.lda = a.C;
            g.ldb = HW;
            g.ldc = HW;
            g.M = (int)a.K;
            g.N = (int)HW;
            g.K = (int)a.C;
            g.batch = (int)(a.N - n0 < 65535 ? a.N - n0 : 65535);
            g.sa = 0;
            g.sb = CHW;
            g.sc = KPQ;
            const hipError_t e = gemm_launch(gcfg, g, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }

    Im2colOperands o;
    o.H = (int)a.H;
    o.W = (int)a.W;
    o.R = (int)a.R;
    o.S = (int)a.S;
    o.sh = (int)a.sh;
    o.sw = (int)a.sw;
    o.ph = (int)a.ph;
    o.pw = (int)a.pw;
    o.dh = (int)a.dh;
    o.dw = (int)a.dw;
    o.Q = (int)a.Q;
    o.PQ = (int)PQ;
    o.HW = (int)HW;
    o.RS = (int)(a.R * a.S);
    o.CHW = (int)CHW;
    const int bk = kConvConfigs[cfg].bk;  // the direct gather steps (c, r, s) by whole K-steps
    o.sK = (int)(bk % a.S);
    o.rK = (int)((bk / a.S) % a.R);
    o.cK = (int)(bk / (a.R * a.S));
    o.KPQ = KPQ;
    // images per launch: x offsets below 2^30, product columns below 2^31; the direct
    // gather's tap masks need a filter of at most 63 taps and runs below 2^31 bytes
    const bool masks = kConvConfigs[cfg].direct && a.R * a.S <= 63 && CHW <= kMaxMaskRun;
    o.tap_masks = masks ? (a.R * a.S <= 31 ? 1 : 2) : 0;
    o.row_table = masks && kConvConfigs[cfg].row_table && (a.C * a.R * a.S + bk - 1) / bk * bk * 8 <= kMaxRowTable;
    int64_t per = (masks ? kMaxMaskRun : kMaxRun) / CHW;
    if (kMaxI32 / PQ < per) per = kMaxI32 / PQ;
    for (int64_t n0 = 0; n0 < a.N; n0 += per) {
        const int64_t nb = (a.N - n0 < per) ? a.N - n0 : per;
        GemmArgs g;
        g.A = a.w;
        g.B = a.x + n0 * CHW;
        g.C = a.y + n0 * KPQ;
        g.lda = a.C * a.R * a.S;
        g.ldb = 0;
        g.ldc = PQ;
        g.M = (int)a.K;
        g.N = (int)(nb * PQ);
        g.K = (int)(a.C * a.R * a.S);
        o.run_bytes = (unsigned)(nb * CHW * 4);
        const hipError_t e = kConvConfigs[cfg].launch(g, o, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mm
