"""GPU parity of the transposed GEMV y = A^T x against the oracle (which computes
A^T x as the GEMM x^T A: the same sums, y[j] = sum_i x_i A[i][j])."""
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


def run(A, x, dev, a_offset=0):
    M, N = A.shape
    abuf = to_device(np.concatenate([np.full(a_offset, np.nan, np.float32), A.ravel()]), dev)
    Ad = abuf[a_offset:].view(M, N)
    y = torch.full((N + 1,), float("nan"), device=dev)
    mm.gemv_t(Ad, to_device(x, dev), out=y[:N])
    torch.cuda.synchronize()
    h = y.cpu().numpy()
    assert np.isnan(h[N]), "wrote past the end of y"
    return h[:N]


def reference(A, x):
    C64, S64 = oracle.gemm(x.reshape(1, -1), A)
    return C64[0], S64[0]


# strips of 16 columns up to N = 6144, of 32 up to 12288, of 64 beyond (ragged last strips
# at 8200 and 12292)
@pytest.mark.parametrize("M,N", [(4096, 4096), (1, 1), (3, 5), (1000, 1531), (4097, 17),
                                 (20000, 64), (17, 4100), (333, 4095), (300, 8200),
                                 (1000, 12288), (130, 12292), (70, 16384), (257, 6144),
                                 (257, 6148), (65, 12284)])
@pytest.mark.parametrize("a_offset", [0, 1])
def test_shapes(dev, M, N, a_offset):
    A = wl.random_matrix(500 + M, M, N, "int4")
    x = wl.random_matrix(600 + N, 1, M, "int4")[0]
    y64, _ = reference(A, x)
    r = verify.exact(run(A, x, dev, a_offset), y64)
    assert r, f"{(M, N)}: {r}"
    A = wl.random_matrix(700 + M, M, N, "u11")
    x = wl.random_matrix(800 + N, 1, M, "u11")[0]
    y64, s64 = reference(A, x)
    r = verify.within_tol(run(A, x, dev, a_offset), y64, s64, 1e-5)
    assert r, f"{(M, N)}: {r}"


def test_matches_gemv_of_transpose(dev):
    """A^T x equals the row GEMV of the explicitly transposed matrix, exactly on integers."""
    A = wl.random_matrix(91, 777, 1531, "int4")
    x = wl.random_matrix(92, 1, 777, "int4")[0]
    y = run(A, x, dev)
    yr = mm.gemv(to_device(np.ascontiguousarray(A.T), dev), to_device(x, dev))
    torch.cuda.synchronize()
    assert np.array_equal(y, yr.cpu().numpy())


def test_deterministic_and_m_zero(dev):
    A = to_device(wl.random_matrix(93, 4096, 4096, "u11"), dev)
    x = to_device(wl.random_matrix(94, 1, 4096, "u11")[0], dev)
    y1 = mm.gemv_t(A, x)
    y2 = mm.gemv_t(A, x)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    y = torch.full((9,), float("nan"), device=dev)
    mm.gemv_t(torch.empty((0, 8), device=dev), torch.empty(0, device=dev), out=y[:8])
    torch.cuda.synchronize()
    assert (y[:8] == 0).all().item() and torch.isnan(y[8]).item()


def run_ws(A, x, dev, a_offset=0, ws=None):
    """mm_gemv_t_f32_ws through the binding, with a NaN-filled workspace (its contents on
    entry must not matter) and a canary after y."""
    M, N = A.shape
    abuf = to_device(np.concatenate([np.full(a_offset, np.nan, np.float32), A.ravel()]), dev)
    Ad = abuf[a_offset:].view(M, N)
    if ws is None:
        ws = mm.gemv_t_workspace(M, N, dev)
        if ws is not None:
            ws.view(torch.float32).fill_(float("nan"))
    y = torch.full((N + 1,), float("nan"), device=dev)
    mm.gemv_t(Ad, to_device(x, dev), out=y[:N], workspace=ws)
    torch.cuda.synchronize()
    h = y.cpu().numpy()
    assert np.isnan(h[N]), "wrote past the end of y"
    return h[:N]


# row blocks (several sizes of block and strip, a ragged last strip and block) and shapes
# that fall back to the strips kernel (too few rows, N % 4 != 0, tiny)
WS_SHAPES = [(4096, 4096), (512, 4096), (1000, 4096), (4096, 16384), (5000, 1000), (1300, 260),
             (2600, 8), (511, 4096), (4096, 1001), (300, 8)]


@pytest.mark.parametrize("M,N", WS_SHAPES)
@pytest.mark.parametrize("a_offset", [0, 1])   # 1: rows not 16-byte aligned (strips kernel)
def test_workspace_variant(dev, M, N, a_offset):
    A = wl.random_matrix(520 + M, M, N, "int4")
    x = wl.random_matrix(620 + N, 1, M, "int4")[0]
    y64, _ = reference(A, x)
    r = verify.exact(run_ws(A, x, dev, a_offset), y64)
    assert r, f"{(M, N)}: {r}"
    A = wl.random_matrix(720 + M, M, N, "u11")
    x = wl.random_matrix(820 + N, 1, M, "u11")[0]
    y64, s64 = reference(A, x)
    r = verify.within_tol(run_ws(A, x, dev, a_offset), y64, s64, 1e-5)
    assert r, f"{(M, N)}: {r}"


def test_workspace_reuse_and_determinism(dev):
    """One workspace for calls in a row (the second smaller): each overwrites what it
    needs; repeated calls give the same bits."""
    ws = mm.gemv_t_workspace(4096, 4096, dev)
    for M, N in [(4096, 4096), (1000, 4096), (4096, 4096)]:
        A = wl.random_matrix(930 + M, M, N, "int4")
        x = wl.random_matrix(940 + N, 1, M, "int4")[0]
        y64, _ = reference(A, x)
        r = verify.exact(run_ws(A, x, dev, ws=ws), y64)
        assert r, f"{(M, N)}: {r}"
    A = to_device(wl.random_matrix(95, 4096, 4096, "u11"), dev)
    x = to_device(wl.random_matrix(96, 1, 4096, "u11")[0], dev)
    y1 = mm.gemv_t(A, x, workspace=ws)
    y2 = mm.gemv_t(A, x, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_workspace_binding_checks(dev):
    """The binding rejects a workspace on the host or not contiguous before any launch."""
    A = torch.zeros((4096, 4096), device=dev)
    x = torch.zeros(4096, device=dev)
    n = mm.mm_gemv_t_f32_workspace_bytes(4096, 4096)
    with pytest.raises(ValueError, match="workspace is on"):
        mm.gemv_t(A, x, workspace=torch.empty(n, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous"):
        mm.gemv_t(A, x, workspace=torch.empty(2 * n, dtype=torch.uint8, device=dev)[::2])
    with pytest.raises(mm.MMError, match="smaller"):
        mm.gemv_t(A, x, workspace=torch.empty(n - 16, dtype=torch.uint8, device=dev))
