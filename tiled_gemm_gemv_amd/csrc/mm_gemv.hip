// mm_gemv.hip -- fp32 GEMV y = A x, bound by HBM bandwidth.
//
// y[i] is the dot product of row i of A with x ("Matrix Operations",
// docs.vulkan.org ML-inference tutorial, "Matrix-Vector Multiplication"). Every
// element of A is used once, so the kernel's speed is the rate at which A
// streams from HBM (0.5 FLOP per byte). The pages give each output row to one
// thread and stage x in shared memory. On CDNA4 one thread per row would make
// neighbouring lanes read addresses a whole row apart; here one 64-lane wave
// owns a row instead: its lanes read the row front to back in 16-byte pieces
// (1 KB per wave instruction, fully coalesced), multiply by the matching pieces
// of x, and combine the 64 partial sums with a cross-lane reduction. x is read
// in the same pattern; at 16 KB it stays in the CU's L1 / the L2, so HBM traffic
// is A plus one copy of x and y. Up to 16 row pieces per lane are in flight at
// once, which covers the 4096-column rows of the fully-connected layer in one
// round trip; longer rows loop.
#include "mm_internal.h"

namespace mm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemvThreads = 256;          // 4 waves, one row each
constexpr int kRowsPerBlock = kGemvThreads / 64;
constexpr int kUnroll = 16;                // 16-byte pieces per lane per round

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// VEC: rows and x are 16-byte aligned and N % 4 == 0.
template <bool VEC>
__global__ __launch_bounds__(kGemvThreads) void gemv_f32_kernel(GemvArgs p)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= p.M) return;  // whole wave leaves; the kernel has no barrier
    const float *a = p.A + (int64_t)row * p.N;
    float acc = 0.f;
    if constexpr (VEC) {
        const f32x4 *a4 = reinterpret_cast<const f32x4 *>(a);
        const f32x4 *x4 = reinterpret_cast<const f32x4 *>(p.x);
        const int n4 = p.N >> 2;
        int c = 0;
        for (; c + 64 * kUnroll <= n4; c += 64 * kUnroll) {
            f32x4 va[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) va[u] = a4[c + u * 64 + lane];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const f32x4 vx = x4[c + u * 64 + lane];
                acc += va[u][0] * vx[0];
                acc += va[u][1] * vx[1];
                acc += va[u][2] * vx[2];
                acc += va[u][3] * vx[3];
            }
        }
        for (; c < n4; c += 64) {
            const int idx = c + lane;
            if (idx < n4) {
                const f32x4 va = a4[idx];
                const f32x4 vx = x4[idx];
                acc += va[0] * vx[0];
                acc += va[1] * vx[1];
                acc += va[2] * vx[2];
                acc += va[3] * vx[3];
            }
        }
    } else {
        int c = 0;
        for (; c + 64 * kUnroll <= p.N; c += 64 * kUnroll) {
            float va[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) va[u] = a[c + u * 64 + lane];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) acc += va[u] * p.x[c + u * 64 + lane];
        }
        for (; c < p.N; c += 64) {
            const int idx = c + lane;
            if (idx < p.N) acc += a[idx] * p.x[idx];
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
    const unsigned blocks = (unsigned)((a.M + kRowsPerBlock - 1) / kRowsPerBlock);
    GemvArgs arg = a;
    void *args[] = {&arg};
    const void *fn = vec ? reinterpret_cast<const void *>(&gemv_f32_kernel<true>)
                         : reinterpret_cast<const void *>(&gemv_f32_kernel<false>);
    return hipLaunchKernel(fn, dim3(blocks), dim3(kGemvThreads), args, 0, stream);
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
