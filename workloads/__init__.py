"""Seeded synthetic inputs for the fp32 GEMM / GEMV workloads.

This module is the only code that both sides of a parity check share: it draws
the input matrices (and lays them out in memory), and it holds none of the
products' arithmetic. The same host arrays are handed to the GPU library and to
the oracle, so the choice of generator cannot affect parity.

Workloads (shapes and value distributions; the pages' own example sizes are the
4096-in x 4096-out fully-connected layer and the 1024 x 1024 square product of
"Matrix Operations", docs.vulkan.org ML-inference tutorial, "Why Matrix Operations
Matter / Computational Intensity"):

  gemm128      C = A B, M = N = K = 128, A, B ~ U[-1, 1)   (+ integer variant)
  gemv4096     y = A x, A 4096 x 4096, x of 4096, A, x ~ U[-1, 1)
  gemm1024     C = A B, M = N = K = 1024, A, B ~ U[-1, 1)
  gemm_ragged  C = A B, M = 1000, K = 777, N = 1531, A, B ~ N(0, 1)
  gemm_proj    C = A B, M = 8192, K = 4096, N = 14336, A ~ N(0, 1), B ~ N(0, 1/K)

Convolution workloads (x N x C x H x W, filters K x C x R x S; the pages name im2col
as the way a convolution maps onto the GEMM but give no layer sizes, so these are
the usual shapes of an image network's layers):

  conv_small   N=2  C=5   13x11  K=7   3x3 stride 1 pad 1        (oracle-sized, ragged)
  conv3x3      N=32 C=128 28x28  K=128 3x3 stride 1 pad 1        (a middle layer)
  conv3x3_s2   N=32 C=128 56x56  K=256 3x3 stride 2 pad 1        (a downsampling layer)
  conv7x7_s2   N=32 C=3   224x224 K=64 7x7 stride 2 pad 3        (the input layer)
  conv1x1      N=32 C=256 56x56  K=64  1x1                       (a pointwise layer)
  conv3x3_d2   N=8  C=64  64x64  K=64  3x3 stride 1 pad 2 dil 2  (a dilated layer)

x ~ U[-1, 1) (operand id 0); w ~ N(0, 1/(C R S)) (operand id 1), the usual scale of
an initialised filter bank; same generator as below.

Every operand comes from numpy's PCG64 seeded with [workload seed, operand id];
operand ids: A = 0, B = 1, x = 2, row sample = 3. Readings where the workload
text is silent: U[-1, 1) is half-open and drawn as 2u - 1 with u a float32 in
[0, 1) (exact in fp32, never 1.0); N(0, 1/K) has variance 1/K (std 1/sqrt(K),
exactly 1/64 at K = 4096); the integer variant draws integers uniformly from
[-4, 4].
"""
from dataclasses import dataclass, field

import numpy as np

OPERAND_A, OPERAND_B, OPERAND_X, OPERAND_ROWS = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                 # "gemm" or "gemv"
    M: int
    N: int
    K: int                  # GEMV: K is unused (0); A is M x N
    dist_a: str             # "u11", "normal", "int4"
    dist_b: str             # for GEMV the distribution of x
    seed: int
    b_std: float = 1.0      # scale of B for "normal" (1/sqrt(K) for N(0, 1/K))
    spot_rows: int = 0      # >0: verify this many sampled rows instead of all
    note: str = field(default="", compare=False)

    def with_dist(self, dist: str) -> "Workload":
        """The same shape and seed with every operand drawn from `dist`."""
        return Workload(self.name + "_" + dist, self.op, self.M, self.N, self.K, dist, dist,
                        self.seed, 1.0, self.spot_rows, self.note)

    def describe(self) -> str:
        if self.op == "gemv":
            return f"gemv fp32 M={self.M} N={self.N}"
        return f"gemm fp32 M={self.M} N={self.N} K={self.K}"


WORKLOADS = {
    "gemm128": Workload("gemm128", "gemm", 128, 128, 128, "u11", "u11", 1001,
                        note="square GEMM 128^3; launch-latency regime"),
    "gemv4096": Workload("gemv4096", "gemv", 4096, 4096, 0, "u11", "u11", 1002,
                         note="fully-connected layer, 4096 inputs x 4096 outputs"),
    "gemm1024": Workload("gemm1024", "gemm", 1024, 1024, 1024, "u11", "u11", 1003,
                         note="square GEMM 1024^3"),
    "gemm_ragged": Workload("gemm_ragged", "gemm", 1000, 1531, 777, "normal", "normal", 1004,
                            note="ragged, non-tile-multiple shape; exercises edge masking"),
    "gemm_proj": Workload("gemm_proj", "gemm", 8192, 14336, 4096, "normal", "normal", 1005,
                          b_std=1.0 / 64.0, spot_rows=64,
                          note="transformer projection: 8192 tokens, 4096 -> 14336"),
}


@dataclass(frozen=True)
class ConvWorkload:
    name: str
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    stride: tuple = (1, 1)
    pad: tuple = (0, 0)
    dilation: tuple = (1, 1)
    seed: int = 0
    dist_x: str = "u11"
    dist_w: str = "normal"    # N(0, 1/(C R S)) for "normal"
    sample_images: int = 0    # >0: verify this many sampled images instead of all
    note: str = field(default="", compare=False)

    def out_hw(self):
        P = (self.H + 2 * self.pad[0] - self.dilation[0] * (self.R - 1) - 1) // self.stride[0] + 1
        Q = (self.W + 2 * self.pad[1] - self.dilation[1] * (self.S - 1) - 1) // self.stride[1] + 1
        return P, Q

    def geometry(self):
        """(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw), the order of the C entry points."""
        return (self.N, self.C, self.H, self.W, self.K, self.R, self.S, *self.stride, *self.pad,
                *self.dilation)

    def with_dist(self, dist: str) -> "ConvWorkload":
        return ConvWorkload(self.name + "_" + dist, self.N, self.C, self.H, self.W, self.K, self.R,
                            self.S, self.stride, self.pad, self.dilation, self.seed, dist, dist,
                            self.sample_images, self.note)

    def describe(self) -> str:
        return (f"conv2d fp32 N={self.N} C={self.C} H={self.H} W={self.W} K={self.K} "
                f"{self.R}x{self.S} stride={self.stride} pad={self.pad} dil={self.dilation}")


CONV_WORKLOADS = {
    "conv_small": ConvWorkload("conv_small", 2, 5, 13, 11, 7, 3, 3, (1, 1), (1, 1), (1, 1), 1101,
                               note="oracle-sized, ragged everywhere"),
    "conv3x3": ConvWorkload("conv3x3", 32, 128, 28, 28, 128, 3, 3, (1, 1), (1, 1), (1, 1), 1102,
                            sample_images=2, note="3x3 middle layer of an image network"),
    "conv3x3_s2": ConvWorkload("conv3x3_s2", 32, 128, 56, 56, 256, 3, 3, (2, 2), (1, 1), (1, 1),
                               1103, sample_images=2, note="3x3 stride-2 downsampling layer"),
    "conv7x7_s2": ConvWorkload("conv7x7_s2", 32, 3, 224, 224, 64, 7, 7, (2, 2), (3, 3), (1, 1),
                               1104, sample_images=2, note="7x7 stride-2 input layer"),
    "conv1x1": ConvWorkload("conv1x1", 32, 256, 56, 56, 64, 1, 1, (1, 1), (0, 0), (1, 1), 1105,
                            sample_images=2, note="pointwise layer"),
    "conv3x3_d2": ConvWorkload("conv3x3_d2", 8, 64, 64, 64, 64, 3, 3, (1, 1), (2, 2), (2, 2), 1106,
                               sample_images=2, note="3x3 dilated layer"),
}


def conv_inputs(w: ConvWorkload):
    """(x, filters): N x C x H x W and K x C x R x S, C-contiguous float32."""
    x = draw(rng_for(w.seed, OPERAND_A), (w.N, w.C, w.H, w.W), w.dist_x)
    std = 1.0 / np.sqrt(max(1, w.C * w.R * w.S)) if w.dist_w == "normal" else 1.0
    f = draw(rng_for(w.seed, OPERAND_B), (w.K, w.C, w.R, w.S), w.dist_w, std)
    return x, f


def sample_images(w: ConvWorkload, n: int = 0) -> np.ndarray:
    """n distinct image indices in [0, N), always with the first and the last."""
    n = n or w.sample_images or w.N
    if n >= w.N:
        return np.arange(w.N, dtype=np.int64)
    mid = rng_for(w.seed, OPERAND_ROWS).choice(np.arange(1, w.N - 1), size=max(0, n - 2),
                                               replace=False)
    return np.sort(np.concatenate([[0, w.N - 1], mid]).astype(np.int64))


def rng_for(seed: int, operand: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(operand)])


def draw(rng: np.random.Generator, shape, dist: str, std: float = 1.0) -> np.ndarray:
    """fp32 array of `shape` with values from `dist`."""
    if dist == "u11":
        u = rng.random(shape, dtype=np.float32)
        return u * np.float32(2.0) - np.float32(1.0)
    if dist == "normal":
        z = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        return z
    if dist == "int4":
        return rng.integers(-4, 5, size=shape, dtype=np.int32).astype(np.float32)
    if dist == "ones":
        return np.ones(shape, dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def gemm_inputs(w: Workload):
    """(A, B): A is M x K, B is K x N, both C-contiguous float32."""
    assert w.op == "gemm"
    A = draw(rng_for(w.seed, OPERAND_A), (w.M, w.K), w.dist_a)
    B = draw(rng_for(w.seed, OPERAND_B), (w.K, w.N), w.dist_b, w.b_std)
    return A, B


def gemv_inputs(w: Workload):
    """(A, x): A is M x N C-contiguous float32, x has N entries."""
    assert w.op == "gemv"
    A = draw(rng_for(w.seed, OPERAND_A), (w.M, w.N), w.dist_a)
    x = draw(rng_for(w.seed, OPERAND_X), (w.N,), w.dist_b)
    return A, x


def sample_rows(w: Workload, n: int = 0) -> np.ndarray:
    """n distinct row indices in [0, M), drawn without replacement, sorted."""
    n = n or w.spot_rows or w.M
    if n >= w.M:
        return np.arange(w.M, dtype=np.int64)
    r = rng_for(w.seed, OPERAND_ROWS).choice(w.M, size=n, replace=False)
    return np.sort(r.astype(np.int64))


def random_matrix(seed: int, rows: int, cols: int, dist: str = "u11", std: float = 1.0):
    """A free-standing seeded matrix, for tests that build their own shapes."""
    return draw(rng_for(seed, OPERAND_A), (rows, cols), dist, std)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), rounding to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the same values as float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns (uint16), rounding to nearest even."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """binary16 bit patterns -> the same values as float32 (exact)."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def embed(a: np.ndarray, ld: int, fill=np.nan, extra_rows: int = 0):
    """Place a (rows x cols) in a buffer with row stride ld >= cols.

    Returns (buf, view): buf is (rows + extra_rows) x ld, filled with `fill` outside
    the matrix (the row gaps and any extra rows), and view is buf[:rows, :cols].
    """
    rows, cols = a.shape
    if ld < cols:
        raise ValueError("ld must be >= cols")
    buf = np.full((rows + extra_rows, ld), fill, dtype=np.float32)
    buf[:rows, :cols] = a
    return buf, buf[:rows, :cols]
