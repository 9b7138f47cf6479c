// mm_internal.h -- declarations shared by the HIP sources of libmm (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

// Arguments of one GEMM launch, already validated on the host. Sizes fit in
// int32; offsets are formed in int64.
struct GemmArgs {
    const float *A;
    const float *B;
    float *C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    // strided batch: problem b uses A + b * sa, B + b * sb, C + b * sc (elements)
    int batch = 1;
    int64_t sa = 0, sb = 0, sc = 0;
};

// Arguments of one GEMV launch (A has packed rows: leading dimension N).
struct GemvArgs {
    const float *A;
    const float *x;
    float *y;
    int M, N;
};

// GEMM tile configurations, in the order of the public config index.
int gemm_num_configs();
const char *gemm_config_name(int cfg);
// batch: number of independent problems launched together (tiles are counted over all).
int gemm_select_config(int64_t M, int64_t N, int64_t K, int64_t batch = 1);
// Enqueue config `cfg` of the GEMM (K >= 1, M >= 1, N >= 1).
hipError_t gemm_launch(int cfg, const GemmArgs &a, hipStream_t stream);

// Narrow-C GEMM (mm_gemm_skinny.hip): 16 x 64 tiles of C, K split over W waves
// per workgroup, L / (column blocks) 16-deep chunks per wave per round. Correct for
// any shape.
template <int W, int L>
hipError_t gemm_skinny_launch(const GemmArgs &a, hipStream_t stream);

// GEMM with 16-bit inputs (mm_gemm_h16.hip); A and B hold bf16 (bf16 = true) or
// binary16 bit patterns, C is fp32. M, N, K >= 1.
int gemm16_num_configs();
const char *gemm16_config_name(int cfg);
int gemm16_select_config(int64_t M, int64_t N, int64_t K);
hipError_t gemm16_launch(int cfg, bool bf16, const void *A, int64_t lda, const void *B, int64_t ldb,
                         float *C, int64_t ldc, int M, int N, int K, hipStream_t stream);

// Enqueue the GEMV (M >= 1, N >= 1).
hipError_t gemv_launch(const GemvArgs &a, hipStream_t stream);

// Enqueue the transposed GEMV y = A^T x (mm_gemv_t.hip); x has M entries, y has N.
// M >= 1, N >= 1.
hipError_t gemv_t_launch(const GemvArgs &a, hipStream_t stream);

// Enqueue a fill of the rows x cols matrix at p (row stride ld) with zeros.
hipError_t zero_fill_launch(float *p, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

}  // namespace mm
