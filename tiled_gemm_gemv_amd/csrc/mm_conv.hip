// mm_conv.hip -- fp32 2-D convolution as an implicit GEMM on the tiled matrix-core
// kernel of mm_gemm_tile.h.
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
// The im2col matrix is never written to memory. The tiled kernel stages it K-step
// by K-step like any B operand, but its loader (Im2colOperands) computes every
// element's address in x, or a zero for the padding, as it goes; the C store
// scatters product column (n, p, q) to y[n][.][p][q]. The images are laid side by
// side along the product's columns (j = n P Q + p Q + q), so a batch of small
// feature maps still makes one wide product that fills the chip. Beyond reading w
// and x and writing y once, HBM traffic is only the x panels the L2 does not keep
// between the R S row-shifts that reuse them.
//
// A 1 x 1 filter with unit stride and no padding needs no gather: each image of x is
// then a C x HW matrix and the convolution is the strided batched GEMM of the same
// kernel with a plain B.
#include "mm_gemm_tile.h"

namespace mm {
namespace {

constexpr int kFar = -(1 << 30);  // an input row that is outside any image

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
    int64_t KPQ;

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
        const int j = n0 + idx % T::BN;
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

struct ConvConfig {
    const char *name;
    hipError_t (*launch)(const GemmArgs &, const Im2colOperands &, hipStream_t);
    int gemm_cfg;       // the same tile shape as a GEMM config (used for 1 x 1 filters)
    int bm, bn;
    int waves;          // per workgroup
    int wg_per_cu;      // workgroups one CU holds (registers and LDS)
    double tflops;      // rate of the tile on large dense shapes, for the choice below
};

template <class T>
hipError_t launch_im2col(const GemmArgs &a, const Im2colOperands &o, hipStream_t stream)
{
    return launch_tile_ops<T>(a, o, stream);
}

// Tile shapes of the fp32 GEMM. The 256 x 256 tile is left out: with the gather's
// per-column state it no longer fits its 256 registers per lane.
const ConvConfig kConvConfigs[] = {
    {"128x128x32 w64x64 pf2 ks1 (4 waves)", &launch_im2col<T128x128k32p2>, 1, 128, 128, 4, 2, 122},
    {"128x128x32 w64x64 pf1 ks2 (8 waves)", &launch_im2col<T128x128k32s2>, 2, 128, 128, 8, 1, 122},
    {"64x64x64 w32x32 pf2 ks1 (4 waves)", &launch_im2col<T64x64k64p2>, 3, 64, 64, 4, 2, 113},
    {"64x64x64 w32x32 pf2 ks2 (8 waves)", &launch_im2col<T64x64k64p2s2>, 4, 64, 64, 8, 2, 94},
    {"128x64x64 w64x32 pf1 ks2 (8 waves)", &launch_im2col<T128x64k64s2>, 5, 128, 64, 8, 1, 111},
};
constexpr int kNumConvConfigs = sizeof(kConvConfigs) / sizeof(kConvConfigs[0]);
constexpr int64_t kMaxI32 = 0x7fffffff;
constexpr int64_t kMaxRun = (int64_t(1) << 30) - 1;  // elements of x per launch

}  // namespace

int conv_num_configs() { return kNumConvConfigs; }

const char *conv_config_name(int cfg)
{
    return (cfg >= 0 && cfg < kNumConvConfigs) ? kConvConfigs[cfg].name : nullptr;
}

// The product is M = K filters by N columns (batch such products side by side).
// Filter counts are often 64-256, so a tall tile can be mostly padding; the choice is
// the least modelled time (tile_time: padded tile area, rounds over the 256 CUs,
// waves per CU, the tile's own rate).
int conv_select_config(int64_t M, int64_t N, int64_t batch)
{
    int best = 0;
    double best_t = 0;
    for (int c = 0; c < kNumConvConfigs; ++c) {
        const ConvConfig &k = kConvConfigs[c];
        const int64_t tiles = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn) * batch;
        const double t = tile_time(tiles, k.bm, k.bn, k.waves, k.wg_per_cu, k.tflops);
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
    if (conv_is_batched_gemm(a)) return conv_select_config(a.K, a.H * a.W, a.N < 65535 ? a.N : 65535);
    return conv_select_config(a.K, a.N * a.P * a.Q, 1);
}

// Shapes are validated by the caller: every size >= 1 (C may be 0: then y is zeroed),
// P and Q as the definition gives them, and the limits stated for Im2colOperands.
hipError_t conv_launch(int cfg, const ConvArgs &a, hipStream_t stream)
{
    const int64_t PQ = a.P * a.Q, HW = a.H * a.W, CHW = a.C * HW, KPQ = a.K * PQ;
    if (a.C == 0) return zero_fill_launch(a.y, a.N * a.K, PQ, PQ, stream);

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
    o.KPQ = KPQ;
    // images per launch: x offsets below 2^30, product columns below 2^31
    int64_t per = kMaxRun / CHW;
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
        const hipError_t e = kConvConfigs[cfg].launch(g, o, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mm
