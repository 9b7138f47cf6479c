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
//   * a workgroup is a single wave, so waves start as soon as a CU has room;
//   * a wave issues the loads for up to 16 KB of its row (16 pieces per lane)
//     before it does any arithmetic, so a 4096-column row is one round trip;
//   * A is read with non-temporal loads (it is used once); x (16 KB at the
//     fully-connected-layer size) is read with ordinary loads and stays in the
//     CU's L1 and the L2 for the other waves;
//   * the order in which a wave visits its 16 pieces is rotated by the row
//     index, so the waves in flight spread over different column offsets and
//     hence over more HBM channels than rows of a power-of-two length would.
// Longer rows take several rounds. The summation order (per-lane partial sums
// over the row's pieces, then a butterfly across lanes) is fixed for a given N,
// so results are deterministic.
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

// VEC: A and x 16-byte aligned and N % 4 == 0. One wave (workgroup) per row.
template <bool VEC>
__global__ __launch_bounds__(64) void gemv_f32_kernel(GemvArgs p)
{
    const int64_t bid = linear_block();
    if (bid >= p.M) return;  // padding of a 2-D grid
    const int lane = threadIdx.x;
    const int row = (int)bid;
    const int rot = row & (kPieces - 1);
    float acc = 0.f;
    if constexpr (VEC) {
        const f32x4 *a4 = reinterpret_cast<const f32x4 *>(p.A + (int64_t)row * p.N);
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x);
        const int n4 = p.N >> 2;
        const int rounds = n4 / (64 * kPieces);
        // full rounds: 16 pieces of 64 float4 each, no masking
        for (int r = 0; r < rounds; ++r) {
            const f32x4 *ar = a4 + r * (64 * kPieces);
            const f32x4 *xr = x4 + r * (64 * kPieces);
            // An opaque copy of the lane index: stops the compiler from hoisting
            // the 32 per-piece addresses out of the loop, which would hold them in
            // registers for the whole kernel and halve the waves a SIMD can hold.
            int l = lane;
            asm volatile("" : "+v"(l));
            f32x4 va[kPieces], vx[kPieces];
#pragma unroll
            for (int u = 0; u < kPieces; ++u) {
                const int idx = ((u + rot) & (kPieces - 1)) * 64 + l;
                va[u] = __builtin_nontemporal_load(ar + idx);
                vx[u] = xr[idx];
            }
            // keep every load above ahead of the arithmetic below
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kPieces; ++u) {
                acc += va[u][0] * vx[u][0];
                acc += va[u][1] * vx[u][1];
                acc += va[u][2] * vx[u][2];
                acc += va[u][3] * vx[u][3];
            }
        }
        const int base = rounds * (64 * kPieces);
        // last, partial round
        if (base < n4) {
            f32x4 va[kPieces], vx[kPieces];
#pragma unroll
            for (int u = 0; u < kPieces; ++u) {
                const int idx = base + u * 64 + lane;
                if (idx < n4) {
                    va[u] = __builtin_nontemporal_load(a4 + idx);
                    vx[u] = x4[idx];
                } else {
                    va[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                    vx[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kPieces; ++u) {
                acc += va[u][0] * vx[u][0];
                acc += va[u][1] * vx[u][1];
                acc += va[u][2] * vx[u][2];
                acc += va[u][3] * vx[u][3];
            }
        }
    } else {
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
    const void *fn = vec ? reinterpret_cast<const void *>(&gemv_f32_kernel<true>)
                         : reinterpret_cast<const void *>(&gemv_f32_kernel<false>);
    unsigned gx, gy;
    if (!grid_for(a.M, gx, gy)) return hipErrorInvalidConfiguration;
    return hipLaunchKernel(fn, dim3(gx, gy), dim3(64), args, 0, stream);
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
