"""GPU checks of mm_gemm_f32_ws_static (the K split in the library's static device
scratch, for callers that cannot allocate) against mm_gemm_f32_ws with a caller
workspace: the same kernels in the same order, so the bits must be identical. Calls run
in a row with different shapes (the second smaller), so the scratch holds the previous
call's partial sums when the next one starts. Integer-valued inputs are also checked
against the oracle, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import verify
import tiled_gemm_gemv_amd as mm
import workloads as wl
from gpu_helpers import nan_output, outside_untouched, require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def run_both(A, B, dev):
    """C from mm_gemm_f32_ws_static and from mm_gemm_f32_ws, each into a NaN-filled buffer
    with gaps (ldc = N + 3); checks that neither wrote outside C."""
    M, K = A.shape
    N = B.shape[1]
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    out = []
    for ws in ("static", mm.gemm_workspace(M, N, K, dev)):
        buf, view = nan_output(M, N, N + 3, dev)
        if isinstance(ws, str) or ws is not None:
            mm.gemm(Ad, Bd, out=view, workspace=ws)
        else:
            mm.gemm(Ad, Bd, out=view)
        torch.cuda.synchronize()
        assert outside_untouched(buf, M, N), "wrote outside C"
        out.append(view.cpu().numpy())
    return out


# calls in a row: each split shape is followed by a smaller one, so the scratch still
# holds larger partial sums of the call before
SEQUENCE = [(4096, 64, 4096), (1000, 40, 2048), (4096, 128, 4096), (1000, 99, 2048), (520, 36, 2048)]


@pytest.mark.parametrize("dist", ["int4", "u11"])
def test_static_scratch_matches_caller_workspace(dev, dist):
    for i, (M, N, K) in enumerate(SEQUENCE):
        need = mm.mm_gemm_f32_workspace_bytes(M, N, K)
        assert 0 < need <= mm.MM_STATIC_SCRATCH_BYTES, (M, N, K, need)
        A = wl.random_matrix(3100 + i, M, K, dist)
        B = wl.random_matrix(3200 + i, K, N, dist)
        c_static, c_ws = run_both(A, B, dev)
        assert np.array_equal(c_static.view(np.int32), c_ws.view(np.int32)), (M, N, K)
        C64, S64 = oracle.gemm(A, B)
        r = verify.exact(c_static, C64) if dist == "int4" else verify.within_tol(c_static, C64, S64, 1e-5)
        assert r, f"{M}x{N}x{K} ({dist}): {r}"


def test_shapes_without_a_split_run_the_plain_gemm(dev):
    # no scratch needed: the result is mm_gemm_f32's, bit for bit
    for M, N, K in [(300, 16, 4096), (128, 128, 128), (1000, 1531, 777)]:
        assert mm.mm_gemm_f32_workspace_bytes(M, N, K) == 0
        A = wl.random_matrix(3300, M, K, "u11")
        B = wl.random_matrix(3301, K, N, "u11")
        c_static, c_plain = run_both(A, B, dev)
        assert np.array_equal(c_static.view(np.int32), c_plain.view(np.int32)), (M, N, K)


def test_larger_than_the_scratch_is_rejected(dev):
    # N % 4 != 0 pads B into the scratch: 4096 x 255 x 16384 needs 24 MiB
    M, N, K = 4096, 255, 16384
    assert mm.mm_gemm_f32_workspace_bytes(M, N, K) > mm.MM_STATIC_SCRATCH_BYTES
    A = torch.zeros((M, K), device=dev)
    B = torch.zeros((K, N), device=dev)
    C = torch.full((M, N), float("nan"), device=dev)
    with pytest.raises(mm.MMError, match="static scratch"):
        mm.gemm(A, B, out=C, workspace="static")
    torch.cuda.synchronize()
    assert torch.isnan(C).all().item(), "a rejected call wrote C"


def test_on_a_caller_stream(dev):
    M, N, K = 2048, 56, 4096
    A = wl.random_matrix(3400, M, K, "int4")
    B = wl.random_matrix(3401, K, N, "int4")
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = torch.empty((M, N), dtype=torch.float32, device=dev)
        mm.mm_gemm_f32_ws_static(M, N, K, Ad, K, Bd, N, C, N, stream=s)
    s.synchronize()
    r = verify.exact(C.cpu().numpy(), oracle.gemm(A, B)[0])
    assert r, r
