"""GPU parity of the strided batched fp32 GEMM: every problem of the batch against
the oracle (integer inputs exact, random inputs within 1e-5 * sum|a b|)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import verify
import tiled_gemm_gemv_amd as mm
import workloads as wl
from gpu_helpers import require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def check_batch(C, As, Bs, exact):
    for b in range(len(As)):
        C64, S64 = oracle.gemm(As[b], Bs[b])
        r = verify.exact(C[b], C64) if exact else verify.within_tol(C[b], C64, S64, 1e-5)
        assert r, f"problem {b}: {r}"


@pytest.mark.parametrize("shape", [(7, 100, 130, 77), (5, 300, 40, 257), (3, 513, 257, 129),
                                   (9, 64, 64, 64), (4, 1000, 1531, 777)])
@pytest.mark.parametrize("dist", ["int4", "normal"])
def test_packed_batches(dev, shape, dist):
    batch, M, N, K = shape
    A = np.stack([wl.random_matrix(10 + b, M, K, dist) for b in range(batch)])
    B = np.stack([wl.random_matrix(50 + b, K, N, dist) for b in range(batch)])
    C = mm.gemm_batched(to_device(A, dev), to_device(B, dev))
    torch.cuda.synchronize()
    check_batch(C.cpu().numpy(), A, B, dist == "int4")


def test_shared_operand_and_gapped_strides(dev):
    """stride_b = 0 shares B; A and C batches sit in NaN-filled buffers with gaps
    between problems and between rows."""
    batch, M, N, K = 6, 150, 90, 70
    lda, ldc = K + 3, N + 5
    sa, sc = M * lda + 11, M * ldc + 13
    A = np.stack([wl.random_matrix(70 + b, M, K, "int4") for b in range(batch)])
    B = wl.random_matrix(80, K, N, "int4")
    Abuf = torch.full((batch * sa,), float("nan"), device=dev)
    Av = torch.as_strided(Abuf, (batch, M, K), (sa, lda, 1))
    Av.copy_(to_device(A, dev))
    Cbuf = torch.full((batch * sc,), float("nan"), device=dev)
    Cv = torch.as_strided(Cbuf, (batch, M, N), (sc, ldc, 1))
    Bd = to_device(B, dev)
    mm.mm_gemm_f32_batched(batch, M, N, K, Av, lda, sa, Bd, N, 0, Cv, ldc, sc)
    torch.cuda.synchronize()
    check_batch(Cv.cpu().numpy(), A, [B] * batch, True)
    host = Cbuf.cpu().numpy()
    mask = np.ones(host.shape, bool)
    for b in range(batch):
        for i in range(M):
            mask[b * sc + i * ldc: b * sc + i * ldc + N] = False
    assert np.isnan(host[mask]).all(), "the batched GEMM wrote outside its problems"


def test_narrow_batches(dev):
    """N <= 64 takes the narrow kernel; its batch index is the third grid dimension."""
    batch, M, N, K = 5, 700, 24, 333
    A = np.stack([wl.random_matrix(90 + b, M, K, "int4") for b in range(batch)])
    B = np.stack([wl.random_matrix(95 + b, K, N, "int4") for b in range(batch)])
    C = mm.gemm_batched(to_device(A, dev), to_device(B, dev))
    torch.cuda.synchronize()
    check_batch(C.cpu().numpy(), A, B, True)


@pytest.mark.parametrize("N,K", [(24, 512), (60, 384), (8, 256)])
def test_narrow_lds_batches(dev, N, K):
    """Narrow shapes that the kernel moving A into LDS in whole row segments takes (N % 4
    == 0, K a multiple of its round): the batch index is the third grid dimension."""
    batch, M = 4, 333
    A = np.stack([wl.random_matrix(110 + b, M, K, "int4") for b in range(batch)])
    B = np.stack([wl.random_matrix(115 + b, K, N, "int4") for b in range(batch)])
    C = mm.gemm_batched(to_device(A, dev), to_device(B, dev))
    torch.cuda.synchronize()
    check_batch(C.cpu().numpy(), A, B, True)


def test_large_batches_sampled_rows(dev):
    """16 problems of 1024^3: enough tiles for the 256 x 256 direct-to-LDS tile (batch on
    the third grid dimension); 8 sampled rows of every problem checked exactly."""
    batch, M, N, K = 16, 1024, 1024, 1024
    A = np.stack([wl.random_matrix(140 + b, M, K, "int4") for b in range(batch)])
    B = np.stack([wl.random_matrix(160 + b, K, N, "int4") for b in range(batch)])
    C = mm.gemm_batched(to_device(A, dev), to_device(B, dev))
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    rows = np.array([0, 1, 255, 256, 511, 700, 1022, 1023])
    for b in range(batch):
        C64, _ = oracle.gemm(A[b], B[b], rows=rows)
        r = verify.exact(got[b][rows], C64)
        assert r, f"problem {b}: {r}"


@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_few_column_batches(dev, N):
    """N <= 4 takes the few-columns kernel; batch index on the third grid dimension,
    odd K and M, and one A shared by every problem (batch stride 0)."""
    batch, M, K = 4, 301, 1031
    A = wl.random_matrix(120 + N, M, K, "int4")
    B = np.stack([wl.random_matrix(130 + b, K, N, "int4") for b in range(batch)])
    Ad = to_device(A, dev).unsqueeze(0).expand(batch, M, K)
    C = mm.gemm_batched(Ad, to_device(B, dev))
    torch.cuda.synchronize()
    check_batch(C.cpu().numpy(), np.stack([A] * batch), B, True)


def test_empty_and_k_zero(dev):
    C = torch.full((3, 4, 5), float("nan"), device=dev)
    mm.gemm_batched(torch.empty((3, 4, 0), device=dev), torch.empty((3, 0, 5), device=dev), out=C)
    torch.cuda.synchronize()
    assert (C == 0).all().item()
    C0 = torch.full((0, 4, 5), float("nan"), device=dev)
    mm.gemm_batched(torch.empty((0, 4, 3), device=dev), torch.empty((0, 3, 5), device=dev), out=C0)
    torch.cuda.synchronize()


def test_rejects_bad_batch_arguments(dev):
    A = torch.zeros((2, 4, 4), device=dev)
    with pytest.raises(mm.MMError):
        mm.mm_gemm_f32_batched(-1, 4, 4, 4, A, 4, 16, A, 4, 16, A, 4, 16)
    with pytest.raises(mm.MMError):
        mm.mm_gemm_f32_batched(2, 4, 4, 4, A, 4, -16, A, 4, 16, A, 4, 16)
    with pytest.raises(mm.MMError):
        mm.mm_gemm_f32_batched(70000, 4, 4, 4, A, 4, 16, A, 4, 16, A, 4, 16)
