"""Element offsets beyond 2^31: the kernels must form every address in 64 bits.

GEMM: A, B and C are views with leading dimensions near 2^25, so their last rows
start more than 2^31 elements (8 GiB) into NaN-filled buffers.
GEMV: a packed 65539 x 32772 matrix (2.15e9 elements, 8.6 GB) whose rows repeat a
block of 64 seeded rows (built on the device by copying, no arithmetic), so every
one of the 65539 outputs can be checked exactly against the oracle's 64 rows.
Convolution: a batch of four 27000 x 27000 images, split by the library into runs
whose 32-bit offsets fit.
Grids: launches of more workgroups than a 1-D grid can hold, for every kernel.
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


def test_conv_batch_split_beyond_2_31(dev):
    """Convolution over 4 images of 27000 x 27000 (x: 2.92e9 elements, y: 5.83e9): the
    library splits the batch into runs of one image (a run of x stays below 2^30
    elements), so the last run starts beyond element 2^31 of x and y. Image n repeats a block of
    64 seeded integer rows starting at row 7 n (built on the device by indexing, no
    arithmetic on values), so images differ; sampled outputs are checked exactly against
    the oracle applied to their receptive field, zero-padded on the host."""
    N, C, H, W, K, R = 4, 1, 27000, 27000, 2, 3
    assert N * C * H * W > BIG and N * K * H * W > BIG
    rows = 64
    block = wl.random_matrix(91, rows, W, "int4")
    filt = wl.random_matrix(92, K, C * R * R, "int4").reshape(K, C, R, R)
    blk = to_device(block, dev)
    x = torch.empty((N, C, H, W), dtype=torch.float32, device=dev)
    for n in range(N):
        idx = (torch.arange(H, device=dev) + 7 * n) % rows
        x[n, 0] = blk[idx]
    y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device=dev)
    mm.conv2d(x, to_device(filt, dev), pad=(1, 1), out=y)
    torch.cuda.synchronize()
    del x
    torch.cuda.empty_cache()

    rng = np.random.default_rng(93)
    spots = [(n, p, q) for n in range(N) for p in (0, 1, H // 2, H - 2, H - 1)
             for q in (0, 1, W // 2, W - 1)]
    spots += [(int(rng.integers(N)), int(rng.integers(H)), int(rng.integers(W))) for _ in range(40)]
    ns = torch.tensor([s[0] for s in spots], device=dev)
    ps = torch.tensor([s[1] for s in spots], device=dev)
    qs = torch.tensor([s[2] for s in spots], device=dev)
    got = torch.stack([y[ns, k, ps, qs] for k in range(K)], 1).cpu().numpy()   # spots x K
    assert torch.isfinite(y[:, :, ::997, ::991]).all().item()
    del y
    torch.cuda.empty_cache()

    want = np.empty((len(spots), K))
    for i, (n, p, q) in enumerate(spots):
        field = np.zeros((1, C, R, R), np.float32)   # receptive field, zero outside the image
        for r in range(R):
            for s in range(R):
                h, v = p + r - 1, q + s - 1
                if 0 <= h < H and 0 <= v < W:
                    field[0, 0, r, s] = block[(h + 7 * n) % rows, v]
        y64, _ = oracle.conv2d(field, filt)
        want[i] = y64[0, :, 0, 0]
    r = verify.exact(got, want)
    assert r, str(r)


# ------------------------------------------- grids past 2^32 work-items (2-D grids)
# A launch of more than 4,194,296 workgroups does not fit a 1-D grid (the dispatch
# packet counts work-items in 32 bits); the library then launches a 2-D grid and each
# kernel numbers its workgroups itself. Outputs are NaN-filled first, so a workgroup
# that never ran leaves NaN behind. Inputs repeat a seeded integer block (device-side
# copies only), so every output is known exactly from the oracle on the block.
TWO_D = 4_194_296 + 1


def _equal_to_repeated(out: torch.Tensor, want: np.ndarray, dim: int) -> bool:
    """out (on the device) equals `want` tiled along `dim`, element by element."""
    w = torch.from_numpy(want.astype(np.float32)).to(out.device)
    reps = out.shape[dim] // want.shape[dim]
    assert reps * want.shape[dim] == out.shape[dim]
    rep = [1] * out.dim()
    rep[dim] = reps
    return torch.equal(out, w.repeat(*rep))


@pytest.mark.parametrize("cfg", [3, 4, 5, 12, 13])   # the tiles 64 columns wide
def test_gemm_grid_beyond_2_32_work_items(dev, cfg):
    M, K, blk = 3, 2, 1024
    N = 293 << 20                              # 307,232,768 columns
    assert -(-N // 64) >= TWO_D
    A = wl.random_matrix(101, M, K, "int4")
    Bb = wl.random_matrix(102, K, blk, "int4")
    B = to_device(Bb, dev).repeat(1, N // blk)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    mm.gemm(to_device(A, dev), B, out=C, config=cfg)
    torch.cuda.synchronize()
    C64, _ = oracle.gemm(A, Bb)
    assert _equal_to_repeated(C, C64, 1)
    del B, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [2, 4])      # the 16-bit tiles 64 columns wide
def test_gemm16_grid_beyond_2_32_work_items(dev, cfg):
    M, K, blk = 3, 2, 1024
    N = 293 << 20
    A = wl.random_matrix(103, M, K, "int4")
    Bb = wl.random_matrix(104, K, blk, "int4")   # small integers are exact in bf16
    Ad = to_device(A, dev).to(torch.bfloat16)
    B = to_device(Bb, dev).to(torch.bfloat16).repeat(1, N // blk)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    mm.gemm16(Ad, B, out=C, config=cfg)
    torch.cuda.synchronize()
    C64, _ = oracle.gemm(A, Bb)
    assert _equal_to_repeated(C, C64, 1)
    del B, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg", [None, 6, 7, 8, 9])   # narrow-C kernels: 16-row, 8-row blocks
def test_narrow_gemm_grid_beyond_2_32_work_items(dev, cfg):
    K, N, blk = 2, 3, 1024
    M = 70_000_640                                 # 4,375,040 blocks of 16 rows
    assert -(-M // 16) >= TWO_D
    Ab = wl.random_matrix(105, blk, K, "int4")
    B = wl.random_matrix(106, K, N, "int4")
    A = to_device(Ab, dev).repeat(M // blk, 1)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    mm.gemm(A, to_device(B, dev), out=C, config=cfg)
    torch.cuda.synchronize()
    C64, _ = oracle.gemm(Ab, B)
    assert _equal_to_repeated(C, C64, 0)
    del A, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("N,M", [(8, 17_000_448),     # 16-byte rows: 4 rows per workgroup
                                 (3, 4_500_480)])     # 4-byte rows: one row per workgroup
def test_gemv_grid_beyond_2_32_work_items(dev, N, M):
    blk = 1024
    assert -(-M // (4 if N % 4 == 0 else 1)) >= TWO_D
    Ab = wl.random_matrix(107, blk, N, "int4")
    x = wl.random_matrix(108, 1, N, "int4")[0]
    A = to_device(Ab, dev).repeat(M // blk, 1)
    y = torch.full((M,), float("nan"), dtype=torch.float32, device=dev)
    mm.gemv(A, to_device(x, dev), out=y)
    torch.cuda.synchronize()
    y64, _ = oracle.gemv(Ab, x)
    assert _equal_to_repeated(y, y64, 0)
    del A, y
    torch.cuda.empty_cache()


def test_gemv_t_grid_beyond_2_32_work_items(dev):
    M, blk = 2, 1024
    N = 70_000_640                                 # 4,375,040 strips of 16 columns
    assert -(-N // 16) >= TWO_D
    Ab = wl.random_matrix(109, M, blk, "int4")
    x = wl.random_matrix(110, 1, M, "int4")
    A = to_device(Ab, dev).repeat(1, N // blk)
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=dev)
    mm.gemv_t(A, to_device(x[0], dev), out=y)
    torch.cuda.synchronize()
    y64, _ = oracle.gemm(x, Ab)                    # x^T A as a 1 x M by M x blk product
    assert _equal_to_repeated(y, y64[0], 0)
    del A, y
    torch.cuda.empty_cache()
