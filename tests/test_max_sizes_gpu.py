"""Element offsets beyond 2^31: the kernels must form every address in 64 bits.

GEMM: A, B and C are views with leading dimensions near 2^25, so their last rows
start more than 2^31 elements (8 GiB) into NaN-filled buffers.
GEMV: a packed 65539 x 32772 matrix (2.15e9 elements, 8.6 GB) whose rows repeat a
block of 64 seeded rows (built on the device by copying, no arithmetic), so every
one of the 65539 outputs can be checked exactly against the oracle's 64 rows.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import verify
import tiled_gemm_gemv_amd as mm
import workloads as wl
from gpu_helpers import require_gpu, to_device

pytestmark = pytest.mark.gpu

BIG = 1 << 31


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def huge_view(a: np.ndarray, ld: int, dev):
    """Device view of `a` with row stride ld inside a NaN-filled buffer."""
    rows, cols = a.shape
    extent = (rows - 1) * ld + cols
    buf = torch.full((extent + 16,), float("nan"), dtype=torch.float32, device=dev)
    view = torch.as_strided(buf, (rows, cols), (ld, 1))
    view.copy_(to_device(a, dev))
    return buf, view


@pytest.mark.parametrize("pad", [3, 4])  # odd leading dimensions, then multiples of 4
def test_gemm_offsets_beyond_2_31(dev, pad):
    M, N, K = 96, 300, 200
    lda, ldb, ldc = (1 << 25) + pad, (1 << 24) + pad, (1 << 25) + 2 * pad
    assert (M - 1) * lda > BIG and (K - 1) * ldb > BIG and (M - 1) * ldc > BIG
    A = wl.random_matrix(71, M, K, "int4")
    B = wl.random_matrix(72, K, N, "int4")
    _, Av = huge_view(A, lda, dev)
    _, Bv = huge_view(B, ldb, dev)
    Cbuf = torch.full(((M - 1) * ldc + N + 16,), float("nan"), dtype=torch.float32, device=dev)
    Cv = torch.as_strided(Cbuf, (M, N), (ldc, 1))
    for cfg in (None, 0, mm.mm_gemm_f32_num_configs() - 1):
        Cv.fill_(float("nan"))
        mm.gemm(Av, Bv, out=Cv, config=cfg)
        torch.cuda.synchronize()
        C64, _ = oracle.gemm(A, B)
        r = verify.exact(Cv.cpu().numpy(), C64)
        assert r, f"config {cfg}: {r}"
    # nothing written between the rows of C: sample the gaps after a few rows
    for i in (0, M // 2, M - 2):
        gap = Cbuf[i * ldc + N: i * ldc + N + 1024]
        assert torch.isnan(gap).all().item()
    del Cbuf, Cv, Av, Bv
    torch.cuda.empty_cache()


def test_gemv_offsets_beyond_2_31(dev):
    M, N, R = 65539, 32772, 64
    assert M * N > BIG
    block = wl.random_matrix(81, R, N, "int4")
    x = wl.random_matrix(82, 1, N, "int4")[0]
    reps = -(-M // R)
    A = to_device(block, dev).repeat(reps, 1)[:M].contiguous()
    assert A.shape == (M, N) and A.is_contiguous()
    y = torch.full((M + 1,), float("nan"), dtype=torch.float32, device=dev)
    mm.gemv(A, to_device(x, dev), out=y[:M])
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    del A
    assert np.isnan(got[M])
    torch.cuda.empty_cache()
    y64, _ = oracle.gemv(block, x)
    want = y64[np.arange(M) % R]
    r = verify.exact(got[:M], want)
    assert r, str(r)
