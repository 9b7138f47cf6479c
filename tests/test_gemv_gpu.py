"""GPU parity of the GEMV (libmm via its C ABI) against the CPU oracle.

Same bars as the GEMM: integer-valued inputs bit-exact, random inputs within
1e-5 * sum_j |A_ij x_j| per output.
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

REL_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def gpu_gemv(A, x, dev, x_offset=0, a_offset=0):
    """Run the GEMV with A and x placed `a_offset` / `x_offset` floats into their
    buffers; y gets a NaN canary after its last entry."""
    M, N = A.shape
    abuf = to_device(np.concatenate([np.full(a_offset, np.nan, np.float32), A.ravel()]), dev)
    xbuf = to_device(np.concatenate([np.full(x_offset, np.nan, np.float32), x]), dev)
    Ad = abuf[a_offset:].view(M, N)
    xd = xbuf[x_offset:]
    ybuf = torch.full((M + 1,), float("nan"), dtype=torch.float32, device=dev)
    mm.gemv(Ad, xd, out=ybuf[:M])
    torch.cuda.synchronize()
    y = ybuf.cpu().numpy()
    assert np.isnan(y[M]), "GEMV wrote past the end of y"
    return y[:M]


def test_fc_layer_tolerance(dev):
    w = wl.WORKLOADS["gemv4096"]
    A, x = wl.gemv_inputs(w)
    y64, s64 = oracle.gemv(A, x)
    r = verify.within_tol(gpu_gemv(A, x, dev), y64, s64, REL_TOL)
    assert r, str(r)


def test_fc_layer_integer_exact(dev):
    w = wl.WORKLOADS["gemv4096"].with_dist("int4")
    A, x = wl.gemv_inputs(w)
    y64, _ = oracle.gemv(A, x)
    r = verify.exact(gpu_gemv(A, x, dev), y64)
    assert r, str(r)


SHAPES = [(1, 1), (3, 5), (7, 4093), (100, 4097), (64, 1), (5, 1024), (33, 8191), (4097, 4100),
          (2, 65536 + 12), (9, 20000), (1000, 64), (513, 257), (6, 12288), (4095, 4096)]


@pytest.mark.parametrize("M,N", SHAPES)
@pytest.mark.parametrize("offsets", [(0, 0), (1, 0), (0, 3)])
def test_ragged_shapes(dev, M, N, offsets):
    """Row lengths that are not multiples of 4 or of the 1024-float wave stride, and
    starts that are only 4-byte aligned; integer inputs exact, random within tolerance."""
    A = wl.random_matrix(300 + M, M, N, "int4")
    x = wl.random_matrix(400 + N, 1, N, "int4")[0]
    y64, _ = oracle.gemv(A, x)
    r = verify.exact(gpu_gemv(A, x, dev, a_offset=offsets[0], x_offset=offsets[1]), y64)
    assert r, f"{(M, N)}: {r}"
    A = wl.random_matrix(500 + M, M, N, "u11")
    x = wl.random_matrix(600 + N, 1, N, "u11")[0]
    y64, s64 = oracle.gemv(A, x)
    r = verify.within_tol(gpu_gemv(A, x, dev, a_offset=offsets[0], x_offset=offsets[1]),
                          y64, s64, REL_TOL)
    assert r, f"{(M, N)}: {r}"


def test_gemv_equals_gemm_column(dev):
    """GEMV(A, x) and GEMM(A, x as N x 1) agree exactly on integer inputs."""
    A = wl.random_matrix(51, 777, 1531, "int4")
    x = wl.random_matrix(52, 1, 1531, "int4")[0]
    y = gpu_gemv(A, x, dev)
    C = mm.gemm(to_device(A, dev), to_device(x.reshape(-1, 1), dev))
    torch.cuda.synchronize()
    assert np.array_equal(y, C.cpu().numpy()[:, 0])


def test_n_zero_writes_zeros(dev):
    y = torch.full((11,), float("nan"), dtype=torch.float32, device=dev)
    mm.gemv(torch.empty((10, 0), dtype=torch.float32, device=dev),
            torch.empty(0, dtype=torch.float32, device=dev), out=y[:10])
    torch.cuda.synchronize()
    assert (y[:10] == 0).all().item() and torch.isnan(y[10]).item()


def test_deterministic(dev):
    w = wl.WORKLOADS["gemv4096"]
    A, x = wl.gemv_inputs(w)
    Ad, xd = to_device(A, dev), to_device(x, dev)
    y1 = mm.gemv(Ad, xd)
    y2 = mm.gemv(Ad, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_host_tensors_rejected(dev):
    """A host x or out is refused by the binding before any launch (its address would be
    a host pointer)."""
    A = torch.zeros((64, 32), device=dev)
    with pytest.raises(ValueError, match="out is on cpu"):
        mm.gemv(A, torch.zeros(32, device=dev), out=torch.empty(64))
    with pytest.raises(ValueError, match="x is on cpu"):
        mm.gemv(A, torch.zeros(32))
    with pytest.raises(ValueError, match="out is on cpu"):
        mm.gemv_t(A, torch.zeros(64, device=dev), out=torch.empty(32))
    with pytest.raises(ValueError, match="x is on cpu"):
        mm.gemv_t(A, torch.zeros(64))
