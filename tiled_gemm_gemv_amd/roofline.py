"""Work and traffic accounting for the GEMM and GEMV, and MI355X roofline peaks.

Counts follow the pages' own analyses:
* multiply-adds: M*N for GEMV, M*N*K for GEMM ("Matrix Operations",
  docs.vulkan.org ML-inference tutorial, "Why Matrix Operations Matter /
  Computational Intensity"); 2 FLOP each.
* naive global reads 2MNK and tiled reads 2MNK / T ("Matrix Operations",
  "Tiled Implementation with Shared Memory / Performance Analysis"; "CUDA
  Programming (6)", section 3.1 "Memory Traffic Analysis of the Baseline" and
  section 3.2 "Memory Reduction Benefit");
* arithmetic intensity 0.25 FLOP/byte naive, T times that tiled ("CUDA
  Programming (6)", section 3.4);
* per-output-tile reads B^2 * 2N naive and 2NB tiled ("GPU Matrix
  Multiplication: Tiling and Shared Memory", section 4);
* shared-memory footprint 2 * T^2 * 4 bytes for two fp32 tiles ("Matrix
  Operations", "Optimizing Tile Size").

Algorithmic bytes (what a roofline divides by) are each operand moved once:
4(MK + KN + MN) for GEMM and 4(MN + N + M) for GEMV. The macro-tile traffic
model 4(MK * ceil(N/BN) + KN * ceil(M/BM) + MN) is the most a tiled GEMM reads
and writes if no panel is ever reused across workgroups.

Peaks are AMD's published MI355X figures (not from the pages).
"""

FP32 = 4

MI355X_FP32_MFMA_PEAK = 157.3e12      # FLOP/s, dense fp32 matrix
MI355X_16BIT_MFMA_PEAK = 2.5e15       # FLOP/s, dense bf16 / fp16 matrix
MI355X_HBM_PEAK = 8.0e12              # bytes/s, HBM3E
MI355X_CUS = 256
MI355X_PEAK_SCLK_HZ = 2.4e9


def ceil_div(a, b):
    return -(-a // b)


# ------------------------------------------------------------------- work counts

def gemv_macs(M, N):
    return M * N


def gemm_macs(M, N, K):
    return M * N * K


def gemm_flops(M, N, K):
    return 2 * M * N * K


def gemv_flops(M, N):
    return 2 * M * N


# --------------------------------------------------------------- traffic models

def gemm_algorithmic_bytes(M, N, K):
    """A, B read once, C written once."""
    return FP32 * (M * K + K * N + M * N)


def gemv_algorithmic_bytes(M, N):
    """A and x read once, y written once."""
    return FP32 * (M * N + N + M)


def gemm_tile_model_bytes(M, N, K, BM, BN):
    """Every workgroup reads its whole A row panel and B column panel from HBM."""
    return FP32 * (M * K * ceil_div(N, BN) + K * N * ceil_div(M, BM) + M * N)


def naive_element_reads(M, N, K):
    """One thread per output, each reading a row of A and a column of B."""
    return 2 * M * N * K


def tiled_element_reads(M, N, K, T):
    """T x T shared-memory tiles: every loaded element serves T outputs."""
    return 2 * M * N * K // T


def two_tile_bytes(T):
    """Shared memory for one T x T fp32 tile of A and one of B."""
    return 2 * T * T * FP32


def naive_intensity():
    """FLOP per global byte when each multiply-add loads both operands."""
    return 2 / (2 * FP32)


def tiled_intensity(T):
    return naive_intensity() * T


def output_tile_reads_naive(B, N):
    return B * B * 2 * N


def output_tile_reads_tiled(B, N):
    return (N // B) * 2 * B * B


def conv_out_hw(H, W, R, S, stride=(1, 1), pad=(0, 0), dil=(1, 1)):
    P = (H + 2 * pad[0] - dil[0] * (R - 1) - 1) // stride[0] + 1
    Q = (W + 2 * pad[1] - dil[1] * (S - 1) - 1) // stride[1] + 1
    return P, Q


def conv_flops(N, C, K, R, S, P, Q):
    """2 FLOP per multiply-add of the implicit GEMM: K x (N P Q) outputs, C R S terms each."""
    return 2 * N * K * P * Q * C * R * S


def conv_algorithmic_bytes(N, C, H, W, K, R, S, P, Q):
    """x and the filters read once, y written once (the im2col matrix is never stored)."""
    return FP32 * (N * C * H * W + K * C * R * S + N * K * P * Q)


def im2col_matrix_bytes(N, C, R, S, P, Q):
    """What an explicit im2col matrix (C R S x N P Q) would take, written and read back."""
    return FP32 * C * R * S * N * P * Q


# ----------------------------------------------------------------- roofline use

def gemm_bound_time(M, N, K):
    """Seconds at the fp32 MFMA peak."""
    return gemm_flops(M, N, K) / MI355X_FP32_MFMA_PEAK


def gemv_bound_time(M, N):
    """Seconds at the HBM peak."""
    return gemv_algorithmic_bytes(M, N) / MI355X_HBM_PEAK
