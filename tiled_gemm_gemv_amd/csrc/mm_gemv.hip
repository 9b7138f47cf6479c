// mm_gemv.hip -- fp32 GEMV y = A x, bound by HBM bandwidth.
//
// y[i] is the dot product of row i of A with x ("Matrix Operations",
// docs.vulkan.org ML-inference tutorial, "Matrix-Vector Multiplication"). Every
// element of A is used once, so the kernel's speed is the rate at which A
// streams from HBM (0.5 FLOP per byte). The pages give each output row to one
// thread and stage x in shared memory. On CDNA4 one thread per row would make
// neighbouring lanes read addresses a whole row apart; here one 64-lane wave
// owns a row instead: its lanes read the row in 16-byte pieces (1 KB per wave
// instruction, fully coalesced), multiply by the matching pieces of x, and
// combine the 64 partial sums with a cross-lane reduction.
//
// Launch shape and memory-level parallelism, sized by measurement on MI355X:
//   * a wave issues the loads for up to 16 KB of its row (16 pieces per lane)
//     before it does any arithmetic, so a 4096-column row is one round trip;
//   * A is read with non-temporal loads (it is used once);
//   * rows whose 16-byte pieces are aligned go four to a workgroup, and the
//     workgroup stages each 16 KB round of x in LDS once (the pages' shared-memory
//     x, per round so that any N fits): read from L2 by every wave instead, x would
//     cost as many L2 bytes as A. Measured at 4096 x 4096: 11.6 us per cold launch
//     against 12.0 us with x from L2 and 11.25 us for a bare 64 MiB read stream;
//   * the order in which a wave visits its 16 pieces is rotated by the row
//     index, so the waves in flight spread over different column offsets and
//     hence over more HBM channels than rows of a power-of-two length would.
// Other rows (N % 4 != 0 or unaligned A or x) take one wave per row with 4-byte
// pieces. Longer rows take several rounds. The summation order (per-lane partial
// sums over the row's pieces, then a butterfly across lanes) is fixed for a given
// N, so results are deterministic.
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPieces = 16;  // 16-byte (or 4-byte) pieces per lane per round

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

constexpr int kRows = 4;               // rows (waves) per workgroup, 16-byte path
constexpr int kRound = 64 * kPieces;   // float4 pieces of x per round: 16 KB

// One round of a row: pieces base .. base + kRound - 1 of the row (float4 units).
// Every load is issued before any arithmetic; x comes through LDS buffer xb, which
// the workgroup fills here (one barrier). FULL: the round lies inside the row.
template <bool FULL>
__device__ __forceinline__ void gemv_round(const f32x4 *ar, const f32x4 *x4, int n4, int base,
                                           int rot, f32x4 *xb, float &acc)
{
    const int lane = threadIdx.x & 63;
    constexpr int XPT = kRound / (kRows * 64);  // x pieces each thread stages
    f32x4 xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int e = base + threadIdx.x + i * kRows * 64;
        xv[i] = (FULL || e < n4) ? x4[e] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // An opaque copy of the lane index: stops the compiler from hoisting the
    // per-piece addresses out of the rounds loop, which would hold them in
    // registers for the whole kernel and cut the waves a SIMD can hold.
    int l = lane;
    asm volatile("" : "+v"(l));
    f32x4 va[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int idx = base + ((u + rot) & (kPieces - 1)) * 64 + l;
        va[u] = (FULL || idx < n4) ? __builtin_nontemporal_load(ar + idx) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // x was requested first, so writing it waits for x alone
#pragma unroll
    for (int i = 0; i < XPT; ++i) xb[threadIdx.x + i * kRows * 64] = xv[i];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const f32x4 xx = xb[((u + rot) & (kPieces - 1)) * 64 + lane];
        acc += va[u][0] * xx[0];
        acc += va[u][1] * xx[1];
        acc += va[u][2] * xx[2];
        acc += va[u][3] * xx[3];
    }
}

// A and x 16-byte aligned, N % 4 == 0. A workgroup of kRows waves takes kRows
// consecutive rows, one per wave, and stages each 16 KB round of x in LDS once for
// all of them (x would otherwise be read from L2 by every wave: as many bytes as A).
// The two LDS buffers alternate between rounds: buffer r & 1 is written in round r
// only after the barrier of round r - 1, by which time every wave has finished
// reading it in round r - 2. TAIL: the last round of a row is partial.
template <bool TAIL>
__device__ __forceinline__ void gemv_vec_rows(const GemvArgs &p)
{
    __shared__ f32x4 xs[2][kRound];
    const int64_t groups = ((int64_t)p.M + kRows - 1) / kRows;
    const int64_t bid = linear_block();
    if (bid >= groups) return;  // padding of a 2-D grid (whole workgroup, before any barrier)
    const int lane = threadIdx.x & 63;
    const int row = (int)bid * kRows + (threadIdx.x >> 6);
    const bool row_ok = row < p.M;  // the last workgroup's spare waves read row 0
    const int rot = row & (kPieces - 1);
    const f32x4 *ar = reinterpret_cast<const f32x4 *>(p.A + (int64_t)(row_ok ? row : 0) * p.N);
    const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x);
    const int n4 = p.N >> 2;
    const int full = n4 / kRound;
    float acc = 0.f;
    int r = 0;
    for (; r < full; ++r) gemv_round<true>(ar, x4, n4, r * kRound, rot, xs[r & 1], acc);
    if (TAIL) gemv_round<false>(ar, x4, n4, r * kRound, rot, xs[r & 1], acc);
    acc = wave_sum(acc);
    if (row_ok && lane == 0) p.y[row] = acc;
}

// N a multiple of 4096 (every round full). At most 128 VGPRs, so that a SIMD holds 4
// of these waves and a CU 4 workgroups: the 1024 workgroups of a 4096 x 4096 A then
// all start at once. With the partial-round code in the same kernel it took 130 VGPRs
// (3 workgroups per CU: a quarter of them waited for a second pass, 3% slower).
__global__ __launch_bounds__(kRows * 64) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_f32_vec_kernel(GemvArgs p)
{
    gemv_vec_rows<false>(p);
}

// Other N (N % 4 == 0): the last round of each row is partial.
__global__ __launch_bounds__(kRows * 64) void gemv_f32_vec_tail_kernel(GemvArgs p)
{
    gemv_vec_rows<true>(p);
}

// Any alignment: one wave (workgroup) per row, 4-byte pieces, x from L1/L2.
__global__ __launch_bounds__(64) void gemv_f32_kernel(GemvArgs p)
{
    const int64_t bid = linear_block();
    if (bid >= p.M) return;  // padding of a 2-D grid
    const int lane = threadIdx.x;
    const int row = (int)bid;
    float acc = 0.f;
    const float *a = p.A + (int64_t)row * p.N;
    for (int base = 0; base < p.N; base += 64 * kPieces) {
        float va[kPieces], vx[kPieces];
#pragma unroll
        for (int u = 0; u < kPieces; ++u) {
            const int idx = base + u * 64 + lane;
            const bool ok = idx < p.N;
            va[u] = ok ? __builtin_nontemporal_load(a + idx) : 0.f;
            vx[u] = ok ? p.x[idx] : 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kPieces; ++u) acc += va[u] * vx[u];
    }
    acc = wave_sum(acc);
    if (lane == 0) p.y[row] = acc;
}

__global__ void zero_fill_kernel(float *p, int64_t rows, int64_t cols, int64_t ld)
{
    const int64_t total = rows * cols;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = e / cols, c = e - r * cols;
        p[r * ld + c] = 0.f;
    }
}

}  // namespace

hipError_t gemv_launch(const GemvArgs &a, hipStream_t stream)
{
    const bool vec = (a.N % 4 == 0) && ((uintptr_t)a.A % 16 == 0) && ((uintptr_t)a.x % 16 == 0);
    GemvArgs arg = a;
    void *args[] = {&arg};
    unsigned gx, gy;
    if (vec) {
        if (!grid_for(((int64_t)a.M + kRows - 1) / kRows, gx, gy)) return hipErrorInvalidConfiguration;
        const void *fn = (a.N % (4 * kRound) == 0) ? reinterpret_cast<const void *>(&gemv_f32_vec_kernel)
                                                    : reinterpret_cast<const void *>(&gemv_f32_vec_tail_kernel);
        return hipLaunchKernel(fn, dim3(gx, gy), dim3(kRows * 64), args, 0, stream);
    }
    if (!grid_for(a.M, gx, gy)) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_f32_kernel), dim3(gx, gy), dim3(64),
                           args, 0, stream);
}

hipError_t zero_fill_launch(float *ptr, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream)
{
    const int64_t total = rows * cols;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    void *args[] = {&ptr, &rows, &cols, &ld};
    return hipLaunchKernel(reinterpret_cast<const void *>(&zero_fill_kernel), dim3((unsigned)blocks),
                           dim3(256), args, 0, stream);
}

}  // namespace mm
