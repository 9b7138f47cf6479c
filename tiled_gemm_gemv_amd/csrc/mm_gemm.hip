// mm_gemm.hip -- fp32 GEMM C = A x B on the gfx950 matrix cores: the tile
// configurations, the choice among them, and their launch. The tiled kernel
// itself is in mm_gemm_tile.h; the narrow-C kernel in mm_gemm_skinny.hip.
#include "mm_gemm_tile.h"

namespace mm {
namespace {

template <class T>
hipError_t launch_tile(const GemmArgs &a, hipStream_t stream)
{
    return launch_tile_ops<T>(a, DenseOperands{}, stream);
}

// The direct-to-LDS pipelines (mm_gemm_direct.hip). The 256 x 256 one needs 16-byte DMA
// lanes; on other shapes the register-staged kernel of that tile size runs instead.
hipError_t direct_or_staged_256(const GemmArgs &a, hipStream_t stream)
{
    return direct_f32_wide_ok(a, 256) ? gemm_direct_launch(DirectTile::T256, a, stream)
                                 : launch_tile<T256x256k32>(a, stream);
}

template <DirectTile T>
hipError_t direct(const GemmArgs &a, hipStream_t stream)
{
    return gemm_direct_launch(T, a, stream);
}

struct ConfigEntry {
    const char *name;
    hipError_t (*launch)(const GemmArgs &, hipStream_t);
    int bm, bn;
    int waves;       // per workgroup
    int wg_per_cu;   // workgroups a CU holds (registers and LDS)
    double tflops;   // measured on large shapes, for the choice below
    int bk;          // K-step depth
    double fill_waves = 8;  // waves per CU at which the tile runs at `tflops` (tile_time)
};

// name: BMxBNxBK, wave tile, prefetch depth, waves per output block (K split).
const ConfigEntry kConfigs[] = {
    {"256x256x32 w128x64 pf1 ks1 (8 waves)", &launch_tile<T256x256k32>, 256, 256, 8, 1, 137, 32},
    {"128x128x32 w64x64 pf2 ks1 (4 waves)", &launch_tile<T128x128k32p2>, 128, 128, 4, 2, 122, 32},
    {"128x128x32 w64x64 pf1 ks2 (8 waves)", &launch_tile<T128x128k32s2>, 128, 128, 8, 1, 122, 32},
    {"64x64x64 w32x32 pf2 ks1 (4 waves)", &launch_tile<T64x64k64p2>, 64, 64, 4, 2, 113, 64},
    {"64x64x64 w32x32 pf2 ks2 (8 waves)", &launch_tile<T64x64k64p2s2>, 64, 64, 8, 1, 94, 64},
    {"128x64x64 w64x32 pf1 ks2 (8 waves)", &launch_tile<T128x64k64s2>, 128, 64, 8, 1, 111, 64},
    {"narrow 16x64 (16x16x4 MFMA), K over 8 waves, 16/NB chunks", &gemm_skinny_launch<8, 16>, 16, 64, 8, 1, 0, 16},
    {"narrow 16x64 (16x16x4 MFMA), K over 4 waves, 16/NB chunks", &gemm_skinny_launch<4, 16>, 16, 64, 4, 1, 0, 16},
    {"narrow 16x64 (16x16x4 MFMA), K over 16 waves, 4/NB chunks", &gemm_skinny_launch<16, 4>, 16, 64, 16, 1, 0, 16},
    {"columns <= 4: one wave per row, B rounds in LDS (8 x 4 per workgroup)", &gemm_cols_launch, 8, 4, 4, 1, 0, 16},
    {"256x256x32 w128x64 direct-to-LDS 2 stages (8 waves; K % 32 != 0: K-steps of 16, 4 stages)", &direct_or_staged_256, 256, 256, 8, 1, 146, 32, 4},
    {"128x128x16 w64x64 direct-to-LDS 4 stages (4 waves; K % 32 == 0: K-steps of 32, 2 stages)", &direct<DirectTile::T128>, 128, 128, 4, 2, 148, 16, 5},
    {"64x64x16 w32x32 direct-to-LDS 8 stages (4 waves; K % 32 == 0: K-steps of 32, 4 stages)", &direct<DirectTile::T64S8>, 64, 64, 4, 2, 136, 16, 5.5},
    {"64x64x16 w32x32 direct-to-LDS 4 stages (4 waves; K % 32 == 0: K-steps of 32, 2 stages)", &direct<DirectTile::T64S4>, 64, 64, 4, 5, 140, 16, 5.5},
    {"64x64x32 w32x32 direct-to-LDS 4 stages, K-step over 2 wave groups (8 waves; K % 32 != 0: config 13's kernel)",
     &direct<DirectTile::T64K2>, 64, 64, 8, 2, 140, 16, 5.5},
    {"narrow 16x64 (16x16x4 MFMA), A and B moved into LDS in whole row segments (N % 4 == 0, K a multiple of 256 or 128; else config 8's kernel)",
     &gemm_narrow_launch, 16, 64, 16, 1, 0, 16},
    {"128x128x16 w64x64 16x16x4 MFMA direct-to-LDS 4 stages (4 waves; K % 32 == 0: K-steps of 32, 2 stages)",
     &direct<DirectTile::T128M16>, 128, 128, 4, 2, 150, 16, 5},
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

// A big tile reuses each staged element more often; a small one fills the chip on
// small shapes and leaves a shorter last round. Among the macro-tile configs the
// choice is the least modelled time (tile_time: padded tile area, rounds over the
// 256 CUs, waves per CU; rates from a timed sweep of every config, 128^3 .. 8192^2).
int gemm_select_config(int64_t M, int64_t N, int64_t K, int64_t batch)
{
    if (N <= 4) return 9;   // a GEMV with a few vectors (mm_gemm_cols.hip)
    // a few columns: stream A once, moved into LDS in whole row segments where the shape
    // allows (mm_gemm_narrow.hip), else in 16-row pieces (mm_gemm_skinny.hip)
    if (N <= 64) return 15;
    if (batch * tiles_for(4, M, N) < 128) return 6;  // few 64 x 64 tiles: 16-row tiles fill more CUs
    // the macro-tile configs (10 runs 0's kernel on shapes its 16-byte DMA does not take;
    // alignment is not known here). The 256 and 128 direct tiles fill 3 stages of a big
    // tile before their first MFMA; below K = 2048 that costs more than the deeper
    // pipeline saves (measured: K = 512 and 1024 slower by 10% and 3%, K = 4096 faster
    // by 5%). 14 is 13's tile on 8 waves (each K-step's k split over two wave groups) where
    // K % 32 == 0: the model rates it above 13 where a CU holds one tile (1024^3: 99 against
    // 97 TFLOP/s), and the two tie where it holds several, which 13 (listed first) takes
    // (1536^3: 100 against 92, 3072^3: 138 against 133, 8192 x 1792 x 4096: 141 against 136).
    // 16 is 11's tile on v_mfma_f32_16x16x4_f32 (rated above it: 149.5 against 147.1 at
    // 8192 x 14336 x 4096, 148.0 against 145.2 at 4096^3), so 11 is never chosen.
    static const int kTileConfigs[] = {0, 1, 2, 3, 4, 5, 10, 11, 12, 13, 14, 16};
    int best = 0;
    double best_t = 0;
    for (int c : kTileConfigs) {
        if ((c == 10 || c == 11 || c == 16) && K < 2048) continue;
        const double t = gemm_config_time(c, M, N, K, batch);
        if (c == 0 || t < best_t) {
            best = c;
            best_t = t;
        }
    }
    return best;
}

double gemm_config_time(int cfg, int64_t M, int64_t N, int64_t K, int64_t batch)
{
    if (cfg < 0 || cfg >= kNumConfigs || kConfigs[cfg].tflops <= 0) return 1e300;
    const ConfigEntry &e = kConfigs[cfg];
    return tile_time(batch * tiles_for(cfg, M, N), e.bm, e.bn, e.waves, e.wg_per_cu, e.tflops, e.fill_waves) *
           k_steps_factor(K, e.bk);
}

hipError_t gemm_launch(int cfg, const GemmArgs &a, hipStream_t stream)
{
    return kConfigs[cfg].launch(a, stream);
}

// ---------------------------------------------------------------------------
// K split across workgroups, for products with few output tiles and long K (the
// fully-connected layer on a batch of 25 to 256 vectors). With at most 256 tiles of
// 64 x 64 the chip holds under one workgroup per CU, and the narrow kernel (16 rows and
// all of K per workgroup) reads all of B from L2 in each workgroup. Split into `chunks`
// K ranges, the product is a strided batch of GEMMs over the chunks (A + c Kc columns,
// B + c Kc rows) on the 64 x 64 direct tile, each writing its own M x N4 slice of the
// workspace (N4 = N rounded up to a multiple of 4); a second kernel adds the slices in
// chunk order and writes the N columns of C. Measured against mm_gemm_f32 (TFLOP/s):
// 4096 x 64 x 4096 58 -> 87, 4096 x 128 x 4096 55 -> 102, 4096 x 256 x 4096 109 -> 118,
// 1024 x 128 x 4096 28 -> 63, 4096 x 32 x 4096 42 -> 45.
// With N % 4 != 0, B's rows are not whole 16-byte lanes: run directly, the chunks took the
// tile's general (4-byte lane) build and the split lost (4096 x 25 x 4096: 33 -> 28). B
// is first copied into the workspace as K x N4 with zero columns after N (one more
// launch, K N4 floats), so the chunks run the lean build; below 33 columns that copy
// eats the gain and such shapes are not split.
namespace {

constexpr int kSplitCfg = 14;  // 64 x 64 direct tile, 4 stages, K-steps over two wave groups

int64_t round4(int64_t n) { return (n + 3) & ~int64_t(3); }

// Bp (K x N4, packed) = B (K x N, leading dimension ldb) with zeros in columns N .. N4 - 1.
__global__ __launch_bounds__(256) void pad_columns_kernel(const float *B, int64_t ldb, float *Bp, int K, int N,
                                                          int N4)
{
    const int64_t total = (int64_t)K * N4;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = e / N4, j = e - k * N4;
        Bp[e] = j < N ? B[k * ldb + j] : 0.f;
    }
}

// C (M x N, leading dimension ldc) = the sum of the `chunks` M x N4 slices of ws, in
// slice order.
__global__ __launch_bounds__(256) void sum_chunks_kernel(const float *ws, float *C, int64_t ldc, int M, int N,
                                                         int N4, int chunks)
{
    const int64_t MN = (int64_t)M * N, slice = (int64_t)M * N4;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < MN; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = e / N, j = e - i * N, w = i * N4 + j;
        float s = ws[w];
        for (int c = 1; c < chunks; ++c) s += ws[c * slice + w];
        C[i * ldc + j] = s;
    }
}

int64_t grid_blocks(int64_t elements)
{
    const int64_t blocks = (elements + 255) / 256;
    return blocks < 4096 ? blocks : 4096;
}

}  // namespace

int gemm_split_chunks(int64_t M, int64_t N, int64_t K)
{
    if (N <= 24 || N > 256 || (N % 4 != 0 && N <= 32) || K < 2048 || M < 1) return 0;
    const int64_t tiles = (M + 63) / 64 * ((N + 63) / 64);
    if (tiles > 256) return 0;  // at least one workgroup per CU without a split
    int chunks = 1;
    while (chunks < 8 && tiles * chunks < 512) chunks *= 2;
    while (chunks > 1 && (K % (16 * chunks) != 0)) chunks /= 2;  // whole 16-k steps per chunk
    return chunks >= 2 ? chunks : 0;
}

// Layout: the chunks' M x N4 slices, then (N % 4 != 0 only) the padded copy of B, which
// starts 16-byte aligned (the slices hold a multiple of 4 floats).
int64_t gemm_split_ws_floats(int64_t M, int64_t N, int64_t K)
{
    const int chunks = gemm_split_chunks(M, N, K);
    if (!chunks) return 0;
    const int64_t N4 = round4(N);
    return chunks * M * N4 + (N4 != N ? K * N4 : 0);
}

hipError_t gemm_split_launch(const GemmArgs &a, float *ws, hipStream_t stream)
{
    const int chunks = gemm_split_chunks(a.M, a.N, a.K);
    if (!chunks) return hipErrorInvalidValue;
    const int N4 = (int)round4(a.N);
    const int kc = a.K / chunks;
    GemmArgs b = a;
    if (N4 != a.N) {
        float *Bp = ws + (int64_t)chunks * a.M * N4;
        const float *B = a.B;
        int64_t ldb = a.ldb;
        int K = a.K, N = a.N, n4 = N4;
        void *pargs[] = {&B, &ldb, &Bp, &K, &N, &n4};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&pad_columns_kernel),
                                             dim3((unsigned)grid_blocks((int64_t)a.K * N4)), dim3(256), pargs, 0,
                                             stream);
        if (e != hipSuccess) return e;
        b.B = Bp;
        b.ldb = N4;
        b.N = N4;
    }
    b.K = kc;
    b.C = ws;
    b.ldc = N4;
    b.batch = chunks;
    b.sa = kc;
    b.sb = (int64_t)kc * b.ldb;
    b.sc = (int64_t)a.M * N4;
    hipError_t e = gemm_launch(kSplitCfg, b, stream);
    if (e != hipSuccess) return e;
    const float *wsc = ws;
    float *C = a.C;
    int64_t ldc = a.ldc;
    int M = a.M, N = a.N, n4 = N4, ch = chunks;
    void *args[] = {&wsc, &C, &ldc, &M, &N, &n4, &ch};
    return hipLaunchKernel(reinterpret_cast<const void *>(&sum_chunks_kernel),
                           dim3((unsigned)grid_blocks((int64_t)a.M * a.N)), dim3(256), args, 0, stream);
}

// Without a workspace, K split in two halves added into C: C is zeroed (a fill kernel over
// its M x N elements), then the two halves run as a batch of two products on the 64 x 64
// direct tile that both add their tiles into C atomically. With exactly two partial sums
// the result does not depend on their order (0 + x == x exactly, x + y == y + x), so it
// is deterministic. Taken where C has 128 to 256 tiles of 64 x 64 (half a workgroup to
// one per CU unsplit) and each half is long. Measured against the unsplit choice
// (TFLOP/s): 4096 x 128 x 4096 53 -> 90, 8192 x 64 x 8192 60 -> 93, 16384 x 64 x 4096
// 60 -> 109, 1024 x 512 x 8192 56 -> 102, 1024 x 1024 x 4096 109 -> 119, 2048 x 512 x 8192
// 112 -> 129. At 64 tiles or fewer two halves still leave most CUs idle (forced through
// the workspace path, 4096 x 64 x 4096 lost, 58 -> 50).
bool gemm_split2_ok(int64_t M, int64_t N, int64_t K)
{
    // N < 64 stays on the narrow kernels; N % 4 != 0 runs the halves on the general build
    // (4-byte B lanes in the last tile column)
    if (K < 2048 || K % 32 != 0 || N < 64) return false;
    const int64_t tiles = (M + 63) / 64 * ((N + 63) / 64);
    // halves of 1024-1040 k on 129-256 tiles measured 1-2% slower (4096 x 256 x 2048,
    // 2000 x 300 x 2080); on 128 tiles still faster (1000 x 500 x 2048: 51 -> 72)
    if (K < 4096 && tiles > 128) return false;
    return tiles >= 128 && tiles <= 256;
}

int gemm_split2_config() { return kSplitCfg; }

hipError_t gemm_split2_launch(const GemmArgs &a, hipStream_t stream)
{
    hipError_t e = zero_fill_launch(a.C, a.M, a.N, a.ldc, stream);
    if (e != hipSuccess) return e;
    GemmArgs b = a;
    b.K = a.K / 2;
    b.batch = 2;
    b.sa = b.K;
    b.sb = (int64_t)b.K * a.ldb;
    b.sc = 0;
    return gemm_direct64_add_launch(b, stream);
}

}  // namespace mm
