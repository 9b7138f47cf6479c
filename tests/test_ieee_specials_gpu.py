"""IEEE special values through every GPU path, element by element against the oracle.

The defining sums ("Matrix Operations", Matrix-Matrix and Matrix-Vector Multiplication)
propagate NaN and infinities as IEEE arithmetic does: a NaN input makes every sum it
enters NaN, an infinity times a zero is NaN, +inf + -inf is NaN, and an infinity plus
finite values stays infinite. With integer-valued finite inputs every output is then NaN,
an infinity of a fixed sign, or an exact integer, whatever the order of the additions,
so the GPU result must match the oracle's pattern exactly. The specials sit at the edges
the kernels treat apart: the last row and column (clamped or shifted tiles), the last k
(partial or overlapping K-steps, zero-filled stages), the two K halves, the K chunks of
the workspace split, the x rounds of the GEMV, and the padding of the convolution.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_gemm_gemv_amd as mm
import workloads as wl
from gpu_helpers import require_gpu, to_device

pytestmark = pytest.mark.gpu

NAN, INF = np.float32(np.nan), np.float32(np.inf)


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def assert_same_ieee(got, ref64, what):
    """NaN exactly where the oracle has NaN; every other element equal to the oracle's
    value rounded to fp32 (infinities with their sign)."""
    got = np.asarray(got)
    want = np.asarray(ref64).astype(np.float32)
    gn, wn = np.isnan(got), np.isnan(want)
    bad = (gn != wn) | (~wn & (got != want))
    assert wn.any() and np.isinf(want).any(), f"{what}: the case plants no special values"
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} differ, first at {i}: "
                             f"got {got[i]!r}, want {want[i]!r}")


def plant(A, B):
    """Integer-valued A (M x K) and B (K x N) with specials planted (copies)."""
    A, B = A.copy(), B.copy()
    M, K = A.shape
    N = B.shape[1]
    A[M - 1, K - 1] = NAN                 # last row, last k: that row of C is NaN
    A[::3, 0] = 0                         # zeros against an infinity: NaN in those rows
    B[0, N - 1] = INF                     # last column
    B[K // 2, N - 1] = -INF               # +inf - inf in rows where both terms are non-zero
    B[K // 3, ::2] = 0
    A[M // 2, K // 3] = INF               # inf * 0 in every other column of row M/2
    return A, B


def ints(seed, rows, cols):
    return wl.random_matrix(seed, rows, cols, "int4")


def gemm_case(M, N, K, seed):
    return plant(ints(seed, M, K), ints(seed + 1, K, N))


def n_configs():
    try:
        return mm.mm_gemm_f32_num_configs()
    except OSError:
        return 14


# a ragged shape (partial K-steps, N % 4 != 0: the general builds and 4-byte lanes) and an
# aligned one (the lean builds, the 256 x 256 direct tile)
GEMM_SHAPES = [(130, 99, 77), (200, 264, 512)]


@pytest.mark.parametrize("cfg", list(range(n_configs())) + [None])
@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gemm_f32_every_config(dev, shape, cfg):
    M, N, K = shape
    A, B = gemm_case(M, N, K, 5100)
    C = mm.gemm(to_device(A, dev), to_device(B, dev), config=cfg)
    torch.cuda.synchronize()
    assert_same_ieee(C.cpu().numpy(), oracle.gemm(A, B)[0], f"{shape} config {cfg}")


# the default call's special paths: two K halves added into a zeroed C, the narrow and
# few-column kernels
@pytest.mark.parametrize("shape", [(1000, 500, 2048), (4096, 128, 4096), (300, 40, 1000), (257, 3, 700)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_f32_default_paths(dev, shape):
    M, N, K = shape
    A, B = gemm_case(M, N, K, 5200)
    C = mm.gemm(to_device(A, dev), to_device(B, dev))
    torch.cuda.synchronize()
    assert_same_ieee(C.cpu().numpy(), oracle.gemm(A, B)[0], f"{shape} default")


@pytest.mark.parametrize("shape", [(1000, 99, 2048), (4096, 64, 4096)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_f32_k_split(dev, shape):
    M, N, K = shape
    A, B = gemm_case(M, N, K, 5300)
    ref = oracle.gemm(A, B)[0]
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    for ws in (mm.gemm_workspace(M, N, K, dev), "static"):
        assert ws is not None
        C = mm.gemm(Ad, Bd, workspace=ws)
        torch.cuda.synchronize()
        assert_same_ieee(C.cpu().numpy(), ref, f"{shape} K split ({'static' if isinstance(ws, str) else 'caller'})")


def test_gemm_f32_batched(dev):
    M, N, K, batch = 70, 90, 300, 3
    pairs = [gemm_case(M, N, K, 5400 + 10 * b) for b in range(batch)]
    A = np.stack([p[0] for p in pairs])
    B = np.stack([p[1] for p in pairs])
    C = mm.gemm_batched(to_device(A, dev), to_device(B, dev))
    torch.cuda.synchronize()
    for b in range(batch):
        assert_same_ieee(C[b].cpu().numpy(), oracle.gemm(A[b], B[b])[0], f"batch {b}")


def gemv_case(M, N, seed):
    A = ints(seed, M, N)
    x = ints(seed + 1, 1, N)[0]
    A[M - 1, N - 1] = NAN        # last row, last column
    A[::3, 0] = 0
    x[0] = INF                   # against zeros: NaN in every third row
    x[N // 2] = -INF
    A[M // 2, N // 3] = INF
    return A, x


@pytest.mark.parametrize("shape", [(300, 1000), (77, 20003)], ids=lambda s: "x".join(map(str, s)))
def test_gemv(dev, shape):
    M, N = shape
    A, x = gemv_case(M, N, 5500)
    y = mm.gemv(to_device(A, dev), to_device(x, dev))
    torch.cuda.synchronize()
    assert_same_ieee(y.cpu().numpy(), oracle.gemv(A, x)[0], f"gemv {shape}")


@pytest.mark.parametrize("shape", [(300, 1000), (2048, 1000)], ids=lambda s: "x".join(map(str, s)))
def test_gemv_t(dev, shape):
    # y = A^T x is the GEMV of A^T: plant in A^T's terms
    M, N = shape
    At, x = gemv_case(N, M, 5600)
    A = np.ascontiguousarray(At.T)
    ref = oracle.gemv(At, x)[0]
    Ad, xd = to_device(A, dev), to_device(x, dev)
    for ws in (None, mm.gemv_t_workspace(M, N, dev)):
        y = mm.gemv_t(Ad, xd, workspace=ws)
        torch.cuda.synchronize()
        assert_same_ieee(y.cpu().numpy(), ref, f"gemv_t {shape} workspace={ws is not None}")


def n16():
    try:
        return mm.mm_gemm_h16_num_configs()
    except OSError:
        return 11


FORMATS16 = {"bf16": (wl.to_bf16_bits, torch.bfloat16), "f16": (wl.to_f16_bits, torch.float16)}


def to16(a, fmt, dev):
    to_bits, tdtype = FORMATS16[fmt]
    return torch.from_numpy(to_bits(a).view(np.int16)).to(dev).view(tdtype)


# K = 777: the direct tiles end with a K-step over k in [713, 777) that overlaps the whole
# steps on [713, 768) and is zeroed there in both panels; an infinity of A in that range
# must not meet a zeroed B value (that would make its whole row NaN)
@pytest.mark.parametrize("fmt", list(FORMATS16))
@pytest.mark.parametrize("cfg", list(range(n16())) + [None])
@pytest.mark.parametrize("shape", [(130, 99, 777), (300, 264, 777)], ids=lambda s: "x".join(map(str, s)))
def test_gemm_16bit(dev, shape, cfg, fmt):
    M, N, K = shape
    A, B = gemm_case(M, N, K, 5700)
    A[M // 4, 720] = INF
    B[720, 1::2] = 0
    C = mm.gemm16(to16(A, fmt, dev), to16(B, fmt, dev), config=cfg)
    torch.cuda.synchronize()
    assert_same_ieee(C.cpu().numpy(), oracle.gemm(A, B)[0], f"{fmt} {shape} config {cfg}")


def n_conv():
    try:
        return mm.mm_conv2d_f32_num_configs()
    except OSError:
        return 5


@pytest.mark.parametrize("cfg", list(range(n_conv())) + [None])
def test_conv2d(dev, cfg):
    N, C, H, W, K, R, S = 2, 5, 13, 11, 7, 3, 3
    x = wl.random_matrix(5800, N * C * H, W, "int4").reshape(N, C, H, W)
    w = wl.random_matrix(5801, K, C * R * S, "int4").reshape(K, C, R, S)
    x[1, 2, 6, 5] = NAN             # a NaN pixel: the windows that hold it
    x[0, 4, 12, 10] = INF           # the last pixel, against zero filter taps
    w[:, 4, 0, 0] = 0
    w[3, 1, 0, 0] = INF             # a corner tap: in the padding for the border outputs
    w[5, 0, 1, 1] = -INF            # the centre tap
    y = mm.conv2d(to_device(x, dev), to_device(w, dev), (1, 1), (1, 1), (1, 1), config=cfg)
    torch.cuda.synchronize()
    assert_same_ieee(y.cpu().numpy(), oracle.conv2d(x, w, (1, 1), (1, 1), (1, 1))[0], f"conv config {cfg}")
