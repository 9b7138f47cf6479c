"""GPU parity of the GEMM (libmm via its C ABI) against the CPU oracle.

Bars: integer-valued inputs must match the oracle bit for bit (every fp32
operation is exact on them, in any order); random inputs must satisfy
|C - C_ref| <= 1e-5 * sum_k |A_ik B_kj| per element. Every tile configuration is
run on the same cases, so the shape-based choice cannot hide a broken one.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import verify
import tiled_gemm_gemv_amd as mm
import workloads as wl
from gpu_helpers import (nan_output, outside_untouched, require_gpu, strided_on_device,
                         to_device)

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def n_configs():
    try:
        return mm.mm_gemm_f32_num_configs()
    except OSError:
        return 3


CONFIGS = list(range(n_configs()))


def gpu_gemm(A, B, dev, cfg=None):
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    C = mm.gemm(Ad, Bd, config=cfg)
    torch.cuda.synchronize()
    return C.cpu().numpy()


def assert_exact(C, A, B):
    C64, _ = oracle.gemm(A, B)
    r = verify.exact(C, C64)
    assert r, str(r)


def assert_tol(C, A, B):
    C64, S64 = oracle.gemm(A, B)
    r = verify.within_tol(C, C64, S64, REL_TOL)
    assert r, str(r)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_permutation_rows(dev, cfg):
    """P B for a permutation P and unique integers in B: pins the MFMA operand and
    accumulator lane layouts (a swapped row or column shows up as a mismatch)."""
    M = K = 96
    N = 80
    perm = np.random.default_rng(5).permutation(K)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1
    B = (np.arange(K * N, dtype=np.float32).reshape(K, N) - 1000)
    C = gpu_gemm(P, B, dev, cfg)
    assert np.array_equal(C, B[perm])


@pytest.mark.parametrize("cfg", CONFIGS)
def test_one_hot_positions(dev, cfg):
    """A single 1 in A at (i, k) copies row k of B into row i of C and nothing else;
    positions cover both lane halves, several 32-blocks and the K tail."""
    M, K, N = 150, 70, 170
    B = wl.random_matrix(77, K, N)
    for (i, k) in [(0, 0), (31, 33), (32, 1), (100, 69), (149, 35), (64, 16)]:
        A = np.zeros((M, K), np.float32)
        A[i, k] = 1
        C = gpu_gemm(A, B, dev, cfg)
        want = np.zeros((M, N), np.float32)
        want[i] = B[k]
        assert np.array_equal(C, want), (i, k)


@pytest.mark.parametrize("cfg", CONFIGS + [None])
@pytest.mark.parametrize("name", ["gemm128", "gemm1024", "gemm_ragged"])
def test_workload_tolerance(dev, name, cfg):
    w = wl.WORKLOADS[name]
    A, B = wl.gemm_inputs(w)
    assert_tol(gpu_gemm(A, B, dev, cfg), A, B)


@pytest.mark.parametrize("cfg", CONFIGS + [None])
@pytest.mark.parametrize("name", ["gemm128", "gemm1024", "gemm_ragged"])
def test_workload_integer_exact(dev, name, cfg):
    w = wl.WORKLOADS[name].with_dist("int4")
    A, B = wl.gemm_inputs(w)
    assert_exact(gpu_gemm(A, B, dev, cfg), A, B)


EDGE = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def edge_shapes(seed, count):
    rng = np.random.default_rng(seed)
    shapes = [(1, 1, 1), (257, 257, 257), (1, 257, 33), (257, 1, 65), (33, 65, 1)]
    while len(shapes) < count:
        shapes.append(tuple(int(v) for v in rng.choice(EDGE, 3)))
    return shapes


# Shapes the direct-to-LDS pipelines take (K % 16 == 0, N % 4 == 0, aligned): one, two,
# three, four and many K-steps (the prologue fills up to three stages), M and N that are
# not tile multiples (clamped loads, masked stores).
# K % 32 == 0 takes the 256 x 256 tile's K-steps of 32 (two stages; one, two, three and
# many steps), other K its K-steps of 16.
DIRECT_SHAPES = [(1, 4, 16), (37, 8, 32), (300, 264, 48), (257, 520, 64), (300, 264, 96),
                 (513, 260, 160), (129, 136, 4096), (1000, 1532, 800)]


@pytest.mark.parametrize("cfg", [10, 11, 12, 13, 16, None])
@pytest.mark.parametrize("shape", DIRECT_SHAPES)
def test_direct_pipeline_shapes(dev, cfg, shape):
    M, N, K = shape
    A = wl.random_matrix(1100 + M, M, K, "int4")
    B = wl.random_matrix(1200 + N, K, N, "int4")
    assert_exact(gpu_gemm(A, B, dev, cfg), A, B)
    A = wl.random_matrix(1300 + M, M, K, "normal")
    B = wl.random_matrix(1400 + N, K, N, "normal")
    assert_tol(gpu_gemm(A, B, dev, cfg), A, B)


@pytest.mark.parametrize("shape", [(300, 264, 96), (513, 260, 4096)])
def test_direct_256_same_bits_as_staged_256(dev, shape):
    """With K-steps of 32 the 256 x 256 direct tile adds each output's k terms in the
    order of the register-staged 256 x 256 x 32 tile (configuration 0), so the two give
    the same bits on random inputs."""
    M, N, K = shape
    A = wl.random_matrix(1900 + M, M, K, "normal")
    B = wl.random_matrix(1950 + N, K, N, "normal")
    C10 = gpu_gemm(A, B, dev, 10)
    C0 = gpu_gemm(A, B, dev, 0)
    assert np.array_equal(C10.view(np.int32), C0.view(np.int32))


def test_16x16_tile_builds(dev):
    """Configuration 16 (the 128 x 128 tile on 16 x 16 MFMAs) in each of its builds: K = 96
    (lean, K-steps of 32), 112 (lean, K-steps of 16) and 100 (general, a partial last
    K-step zero-filled in LDS): exact on integers, within tolerance on normal inputs."""
    M, N = 300, 264
    for K in (96, 112, 100):
        A = wl.random_matrix(61 + K, M, K, "int4")
        B = wl.random_matrix(62 + K, K, N, "int4")
        assert_exact(gpu_gemm(A, B, dev, 16), A, B)
        A = wl.random_matrix(63 + K, M, K, "normal")
        B = wl.random_matrix(64 + K, K, N, "normal")
        assert_tol(gpu_gemm(A, B, dev, 16), A, B)


# Shapes that only the 4-byte DMA lanes take (K % 16 != 0, odd leading dimensions, N < 4):
# a partial K-step alone (K < 16), after one or many full steps, with a pipeline deeper
# than the K loop, and the ragged shape of the benchmark set (lda 777, ldb 1531).
DIRECT_RAGGED = [(1, 1, 1), (5, 3, 7), (64, 64, 15), (130, 70, 33), (257, 2, 1), (65, 129, 113),
                 (1000, 1531, 777), (129, 67, 4099)]


@pytest.mark.parametrize("cfg", [11, 12, 13, 16])
@pytest.mark.parametrize("shape", DIRECT_RAGGED)
def test_direct_pipeline_ragged(dev, cfg, shape):
    M, N, K = shape
    A = wl.random_matrix(1500 + M, M, K, "int4")
    B = wl.random_matrix(1600 + N, K, N, "int4")
    assert_exact(gpu_gemm(A, B, dev, cfg), A, B)
    A = wl.random_matrix(1700 + M, M, K, "normal")
    B = wl.random_matrix(1800 + N, K, N, "normal")
    assert_tol(gpu_gemm(A, B, dev, cfg), A, B)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_edge_shape_sweep(dev, cfg):
    """Shapes around tile multiples in every dimension; integer inputs, exact."""
    for t, (M, N, K) in enumerate(edge_shapes(100 + cfg, 30)):
        A = wl.random_matrix(1000 + t, M, K, "int4")
        B = wl.random_matrix(2000 + t, K, N, "int4")
        C = gpu_gemm(A, B, dev, cfg)
        C64, _ = oracle.gemm(A, B)
        r = verify.exact(C, C64)
        assert r, f"shape {(M, N, K)}: {r}"


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("offsets", [(0, 0), (1, 2), (3, 0)])
def test_strided_poisoned_views(dev, cfg, offsets):
    """Leading dimensions beyond the width with NaN in every gap, a NaN row past each
    input and a start that is only 4-byte aligned: any read outside a matrix turns
    its outputs into NaN, and every C element outside the view must stay NaN."""
    M, N, K = 203, 181, 97
    A = wl.random_matrix(31, M, K, "int4")
    B = wl.random_matrix(32, K, N, "int4")
    _, Av = strided_on_device(A, K + 3, dev, offset=offsets[0])
    _, Bv = strided_on_device(B, N + 5, dev, offset=offsets[1])
    Cbuf, Cv = nan_output(M, N, N + 7, dev)
    mm.gemm(Av, Bv, out=Cv, config=cfg)
    torch.cuda.synchronize()
    assert_exact(Cv.cpu().numpy(), A, B)
    assert outside_untouched(Cbuf, M, N)


@pytest.mark.parametrize("cfg", [10, 11, 12, 13, 16])
@pytest.mark.parametrize("K", [96, 112])
@pytest.mark.parametrize("offsets", [(0, 0), (1, 2)])
def test_direct_lean_strided_poisoned_views(dev, cfg, K, offsets):
    """The lean direct builds (K % 16 == 0, N % 4 == 0; K-steps of 32 at K = 96, of 16 at
    K = 112) address their loads from the tile's corner plus a fixed offset per lane:
    leading dimensions beyond the width with NaN in every gap and starts that are only
    4-byte aligned must still read only the matrices."""
    M, N = 300, 264
    A = wl.random_matrix(41, M, K, "int4")
    B = wl.random_matrix(42, K, N, "int4")
    _, Av = strided_on_device(A, K + 5, dev, offset=offsets[0])
    _, Bv = strided_on_device(B, N + 12, dev, offset=offsets[1])
    Cbuf, Cv = nan_output(M, N, N + 7, dev)
    mm.gemm(Av, Bv, out=Cv, config=cfg)
    torch.cuda.synchronize()
    assert_exact(Cv.cpu().numpy(), A, B)
    assert outside_untouched(Cbuf, M, N)


@pytest.mark.parametrize("cfg", [10, 11, 12, 13, 16])
def test_direct_huge_leading_dimension(dev, cfg):
    """lda of 5M floats: 255 rows of it exceed the 32-bit lane offsets the lean builds
    use, so those shapes take the general build (or, for the 256 x 256 tile, the
    register-staged one); the result is still exact."""
    M, N, K, lda = 3, 64, 32, 5_000_000
    A = wl.random_matrix(43, M, K, "int4")
    B = wl.random_matrix(44, K, N, "int4")
    _, Av = strided_on_device(A, lda, dev)
    Bd = to_device(B, dev)
    C = mm.gemm(Av, Bd, config=cfg)
    torch.cuda.synchronize()
    assert_exact(C.cpu().numpy(), A, B)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_k_zero_writes_zeros_and_empty_is_noop(dev, cfg):
    Cbuf, Cv = nan_output(37, 45, 50, dev)
    A = torch.empty((37, 0), dtype=torch.float32, device=dev)
    B = torch.empty((0, 45), dtype=torch.float32, device=dev)
    mm.gemm(A, B, out=Cv, config=cfg)
    torch.cuda.synchronize()
    assert (Cv == 0).all().item()
    assert outside_untouched(Cbuf, 37, 45)
    Cbuf2, Cv2 = nan_output(0, 45, 45, dev)
    mm.gemm(torch.empty((0, 3), dtype=torch.float32, device=dev),
            torch.ones((3, 45), dtype=torch.float32, device=dev), out=Cv2, config=cfg)
    torch.cuda.synchronize()
    assert torch.isnan(Cbuf2).all().item()


def test_non_default_stream(dev):
    w = wl.WORKLOADS["gemm_ragged"].with_dist("int4")
    A, B = wl.gemm_inputs(w)
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = torch.empty((A.shape[0], B.shape[1]), dtype=torch.float32, device=dev)
        mm.gemm(Ad, Bd, out=C)
    s.synchronize()
    assert_exact(C.cpu().numpy(), A, B)


def test_deterministic(dev):
    w = wl.WORKLOADS["gemm1024"]
    A, B = wl.gemm_inputs(w)
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    C1 = mm.gemm(Ad, Bd)
    C2 = mm.gemm(Ad, Bd)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_transpose_identity(dev):
    """(A B)^T == B^T A^T, exact on integers, from two GPU calls."""
    A = wl.random_matrix(41, 300, 130, "int4")
    B = wl.random_matrix(42, 130, 210, "int4")
    C = gpu_gemm(A, B, dev)
    Ct = gpu_gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), dev)
    assert np.array_equal(C.T, Ct)


@pytest.mark.parametrize("dist", ["normal", "int4"])
def test_projection_spot_rows(dev, dist):
    """The 8192 x 4096 x 14336 projection in the configuration the benchmark times:
    64 sampled rows checked in full against the oracle."""
    w = wl.WORKLOADS["gemm_proj"]
    if dist == "int4":
        w = w.with_dist("int4")
    A, B = wl.gemm_inputs(w)
    rows = wl.sample_rows(wl.WORKLOADS["gemm_proj"], 64)
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    C = mm.gemm(Ad, Bd)
    torch.cuda.synchronize()
    got = C[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del C, Ad, Bd
    C64, S64 = oracle.gemm(A, B, rows=rows)
    r = verify.exact(got, C64) if dist == "int4" else verify.within_tol(got, C64, S64, REL_TOL)
    assert r, str(r)


@pytest.mark.parametrize("N", [1, 2, 3, 7, 16, 33, 64])
def test_fc_layer_small_batch(dev, N):
    """The 4096 x 4096 fully-connected layer applied to N input vectors at once
    (C = A X with X of N columns): integer inputs exact, random within tolerance,
    in the configuration mm_gemm_f32 selects."""
    M = K = 4096
    A = wl.random_matrix(91, M, K, "int4")
    X = wl.random_matrix(92 + N, K, N, "int4")
    assert_exact(gpu_gemm(A, X, dev), A, X)
    A = wl.random_matrix(93, M, K, "u11")
    X = wl.random_matrix(94 + N, K, N, "u11")
    assert_tol(gpu_gemm(A, X, dev), A, X)


# The narrow kernel that moves A into LDS in whole row segments (config 15): one, two and
# four column blocks (rounds of 256 k, 256 k and 128 k), ragged M (rows clamped), N below
# the tile's width (B's chunks past N clamped), a single round; then shapes it does not
# take (N % 4 != 0, K not a multiple of its round), which run config 8's kernel.
NARROW_SHAPES = [(16, 4, 256), (37, 16, 512), (100, 12, 768), (33, 20, 256), (130, 32, 1024),
                 (50, 36, 128), (255, 64, 384), (300, 60, 640), (20, 18, 256), (20, 16, 200),
                 (70, 44, 96)]


@pytest.mark.parametrize("M,N,K", NARROW_SHAPES)
@pytest.mark.parametrize("offsets", [(0, 0), (1, 2)])
def test_narrow_lds_kernel(dev, M, N, K, offsets):
    """Config 15 on strided views with NaN in every gap and starts that are only 4-byte
    aligned: exact on integers, within tolerance on random inputs, nothing written outside C."""
    for dist, check in (("int4", assert_exact), ("u11", assert_tol)):
        A = wl.random_matrix(61 + M, M, K, dist)
        B = wl.random_matrix(62 + N, K, N, dist)
        _, Av = strided_on_device(A, K + 3, dev, offset=offsets[0])
        _, Bv = strided_on_device(B, N + 5, dev, offset=offsets[1])
        Cbuf, Cv = nan_output(M, N, N + 7, dev)
        mm.gemm(Av, Bv, out=Cv, config=15)
        torch.cuda.synchronize()
        check(Cv.cpu().numpy(), A, B)
        assert outside_untouched(Cbuf, M, N)


def test_small_batch_columns_equal_gemv(dev):
    """Each column of A X equals the GEMV A x_j, exactly on integers."""
    A = wl.random_matrix(95, 1000, 777, "int4")
    X = wl.random_matrix(96, 777, 24, "int4")
    Ad = to_device(A, dev)
    C = gpu_gemm(A, X, dev)
    for j in (0, 5, 23):
        y = mm.gemv(Ad, to_device(np.ascontiguousarray(X[:, j]), dev))
        torch.cuda.synchronize()
        assert np.array_equal(C[:, j], y.cpu().numpy()), j


def run_gemm_ws(A, B, dev, ws=None, a_offset=0, ldb_pad=0):
    """mm_gemm_f32_ws through the binding: a NaN-filled workspace (its contents on entry
    must not matter), A possibly only 4-byte aligned, B possibly with padded rows, and C
    inside a NaN buffer that must stay untouched outside the product."""
    M, K = A.shape
    N = B.shape[1]
    _, Ad = strided_on_device(A, K, dev, offset=a_offset)
    _, Bd = strided_on_device(B, N + ldb_pad, dev)
    if ws is None:
        ws = mm.gemm_workspace(M, N, K, dev)
        if ws is not None:
            ws.view(torch.float32).fill_(float("nan"))
    Cbuf, Cv = nan_output(M, N, N + 3, dev)
    mm.gemm(Ad, Bd, out=Cv, workspace=ws)
    torch.cuda.synchronize()
    assert outside_untouched(Cbuf, M, N)
    return Cv.cpu().numpy()


# K split into 2-8 chunks (N of 28-256, ragged M and N % 64 != 0, K % 32 != 0 per chunk;
# N % 4 != 0 through the padded copy of B) and shapes that need no workspace (N <= 24,
# N % 4 != 0 up to 32, N > 256, more than 256 tiles, K < 2048, K with no whole 16-k
# chunks) and take mm_gemm_f32's kernels
WS_SHAPES = [(4096, 64, 4096), (4096, 32, 4096), (1000, 48, 2048), (777, 60, 2080), (4096, 40, 8192),
             (130, 28, 3072), (4096, 128, 4096), (1000, 200, 2048), (4096, 256, 4096), (64, 256, 8192),
             (4096, 45, 4096), (777, 61, 2080), (1000, 99, 2048), (130, 33, 3072), (4096, 255, 4096),
             (4096, 24, 4096), (4096, 25, 4096), (4096, 31, 4096), (512, 260, 2048), (8192, 256, 2048),
             (300, 64, 1024), (300, 64, 2064)]


@pytest.mark.parametrize("M,N,K", WS_SHAPES)
@pytest.mark.parametrize("layout", [(0, 0), (1, 8)])  # (A offset in floats, B row padding)
def test_split_k_workspace(dev, M, N, K, layout):
    A = wl.random_matrix(1100 + M, M, K, "int4")
    B = wl.random_matrix(1200 + N, K, N, "int4")
    assert_exact(run_gemm_ws(A, B, dev, a_offset=layout[0], ldb_pad=layout[1]), A, B)
    A = wl.random_matrix(1300 + M, M, K, "u11")
    B = wl.random_matrix(1400 + N, K, N, "u11")
    assert_tol(run_gemm_ws(A, B, dev, a_offset=layout[0], ldb_pad=layout[1]), A, B)


def test_split_k_workspace_reuse_and_determinism(dev):
    """One workspace for calls in a row (the second smaller, the third needing none):
    each overwrites what it reads; repeated calls give the same bits."""
    ws = mm.gemm_workspace(4096, 64, 4096, dev)
    assert ws is not None
    for M, N, K in [(4096, 64, 4096), (1000, 40, 2048), (1000, 99, 2048), (300, 16, 4096), (4096, 64, 4096)]:
        A = wl.random_matrix(1500 + M, M, K, "int4")
        B = wl.random_matrix(1600 + N, K, N, "int4")
        assert_exact(run_gemm_ws(A, B, dev, ws=ws), A, B)
    A = to_device(wl.random_matrix(97, 4096, 4096, "u11"), dev)
    B = to_device(wl.random_matrix(98, 4096, 48, "u11"), dev)
    C1 = mm.gemm(A, B, workspace=ws)
    C2 = mm.gemm(A, B, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int32), C2.view(torch.int32))


def test_split_k_workspace_on_stream(dev):
    """Both kernels of the split run on the caller's stream, in order."""
    A = wl.random_matrix(99, 2048, 4096, "int4")
    B = wl.random_matrix(100, 4096, 56, "int4")
    Ad, Bd = to_device(A, dev), to_device(B, dev)
    ws = mm.gemm_workspace(2048, 56, 4096, dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        C = torch.empty((2048, 56), dtype=torch.float32, device=dev)
        mm.gemm(Ad, Bd, out=C, workspace=ws)
    s.synchronize()
    assert_exact(C.cpu().numpy(), A, B)


def test_split_k_workspace_binding_checks(dev):
    """The binding rejects a workspace on the host or not contiguous before any launch."""
    A = torch.zeros((4096, 4096), device=dev)
    B = torch.zeros((4096, 64), device=dev)
    n = mm.mm_gemm_f32_workspace_bytes(4096, 64, 4096)
    with pytest.raises(ValueError, match="workspace is on"):
        mm.gemm(A, B, workspace=torch.empty(n, dtype=torch.uint8))
    with pytest.raises(ValueError, match="contiguous"):
        mm.gemm(A, B, workspace=torch.empty(2 * n, dtype=torch.uint8, device=dev)[::2])
    with pytest.raises(ValueError, match="forced config"):
        mm.gemm(A, B, workspace=torch.empty(n, dtype=torch.uint8, device=dev), config=0)
    with pytest.raises(mm.MMError, match="smaller"):
        mm.gemm(A, B, workspace=torch.empty(n - 16, dtype=torch.uint8, device=dev))


# mm_gemm_f32's two-K-halves path (C zeroed, then both halves added into it atomically):
# 128 to 256 tiles of 64 x 64, ragged M and N, K of 2048 at 128 tiles
SPLIT2_SHAPES = [(4096, 128, 4096), (1000, 500, 2048), (2000, 300, 4096), (1024, 1024, 4096),
                 (8192, 64, 8192), (520, 1000, 4096)]


def run_default(A, B, dev, a_offset=0):
    M, K = A.shape
    N = B.shape[1]
    _, Ad = strided_on_device(A, K, dev, offset=a_offset)
    Bd = to_device(B, dev)
    Cbuf, Cv = nan_output(M, N, N + 3, dev)
    mm.gemm(Ad, Bd, out=Cv)
    torch.cuda.synchronize()
    assert outside_untouched(Cbuf, M, N), "wrote into the gaps of C"
    return Cv.cpu().numpy()


@pytest.mark.parametrize("M,N,K", SPLIT2_SHAPES)
@pytest.mark.parametrize("a_offset", [0, 1])
def test_two_k_halves(dev, M, N, K, a_offset):
    assert mm.mm_gemm_f32_select(M, N, K) == 14  # the halves' tile: 64 x 64 direct, two wave groups
    A = wl.random_matrix(1700 + M, M, K, "int4")
    B = wl.random_matrix(1800 + N, K, N, "int4")
    assert_exact(run_default(A, B, dev, a_offset), A, B)
    A = wl.random_matrix(1900 + M, M, K, "u11")
    B = wl.random_matrix(2000 + N, K, N, "u11")
    assert_tol(run_default(A, B, dev, a_offset), A, B)


def test_two_k_halves_deterministic_on_stream(dev):
    """Random inputs: repeated calls on a non-default stream give the same bits, whichever
    half adds first."""
    A = to_device(wl.random_matrix(2101, 4096, 4096, "normal"), dev)
    B = to_device(wl.random_matrix(2102, 4096, 128, "normal"), dev)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        outs = [mm.gemm(A, B) for _ in range(4)]
    s.synchronize()
    for C in outs[1:]:
        assert torch.equal(C.view(torch.int32), outs[0].view(torch.int32))
