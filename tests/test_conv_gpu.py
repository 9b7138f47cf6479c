"""GPU parity of the implicit-GEMM convolution (mm_conv2d_f32 through the C ABI)
against the oracle's direct definition of the convolution.

Bars as for the GEMM: integer-valued inputs (|x|, |w| <= 4) must match the oracle
bit for bit, since every partial sum is an integer below 2^24 and so exact in fp32
in any order; random inputs must satisfy |y - y_ref| <= 1e-5 * sum |x w| over the
same terms, per element. Every tile configuration runs every geometry, so the
shape-based choice cannot hide a broken one.
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


def n_configs():
    try:
        return mm.mm_conv2d_f32_num_configs()
    except OSError:
        return 5


CONFIGS = list(range(n_configs()))

# name, N, C, H, W, K, R, S, stride, pad, dilation
GEOMETRIES = [
    ("3x3 pad 1, ragged map", 2, 5, 13, 11, 7, 3, 3, (1, 1), (1, 1), (1, 1)),
    ("3x3 stride 2 pad 1, odd map", 3, 4, 15, 14, 9, 3, 3, (2, 2), (1, 1), (1, 1)),
    ("3x2, mixed strides, pads, dilations", 2, 3, 17, 19, 5, 3, 2, (2, 3), (2, 0), (2, 3)),
    ("1x1 on small maps (gathered)", 3, 6, 9, 7, 10, 1, 1, (1, 1), (0, 0), (1, 1)),
    ("1x1 stride 2", 2, 6, 9, 9, 4, 1, 1, (2, 2), (0, 0), (1, 1)),
    ("1x1 with padding", 2, 3, 5, 6, 4, 1, 1, (1, 1), (1, 2), (1, 1)),
    ("filter as large as the input", 2, 3, 6, 5, 4, 6, 5, (1, 1), (0, 0), (1, 1)),
    ("padding beyond the filter's reach", 1, 2, 4, 4, 3, 3, 3, (1, 1), (4, 4), (1, 1)),
    ("one channel, one filter", 1, 1, 10, 10, 1, 3, 3, (1, 1), (1, 1), (1, 1)),
    ("5x5, C R S = 400 (many K-steps), 70 filters", 2, 16, 12, 12, 70, 5, 5, (1, 1), (2, 2),
     (1, 1)),
    ("200 filters (two tile rows)", 1, 8, 9, 9, 200, 3, 3, (1, 1), (1, 1), (1, 1)),
    ("1x7 filter", 2, 4, 8, 20, 6, 1, 7, (1, 1), (0, 3), (1, 1)),
    ("7x7 stride 2 pad 3 (input-layer form)", 2, 3, 30, 30, 16, 7, 7, (2, 2), (3, 3), (1, 1)),
    ("stride larger than the filter", 2, 3, 20, 20, 5, 2, 2, (3, 3), (0, 0), (1, 1)),
    ("one output position per image", 5, 7, 3, 3, 6, 3, 3, (1, 1), (0, 0), (1, 1)),
    # tap masks of two words: 63 taps (the most they hold; bit 63 marks rows past K), and 64
    # taps, gathered without masks
    ("7x9 filter, 63 taps, padded", 1, 2, 12, 12, 5, 7, 9, (1, 1), (3, 4), (1, 1)),
    ("8x8 filter, 64 taps, padded", 1, 2, 11, 11, 3, 8, 8, (1, 1), (2, 2), (1, 1)),
    # C R S = 2160: more rows than the direct gather's LDS row table takes (2048), so the
    # tap masks run with their rows stepped in scalar registers
    ("3x3, C R S = 2160 (tap masks without the row table)", 1, 240, 6, 6, 12, 3, 3, (1, 1), (1, 1),
     (1, 1)),
]
GEO_IDS = [g[0] for g in GEOMETRIES]


def make_inputs(geo, dist, seed):
    _, N, C, H, W, K, R, S, st, pd, dl = geo
    cw = wl.ConvWorkload("case", N, C, H, W, K, R, S, st, pd, dl, seed, dist, dist)
    return cw, *wl.conv_inputs(cw)


def run_gpu(x, w, cw, dev, cfg=None):
    """The convolution on the GPU into a NaN-filled buffer one output image longer than y;
    returns (y, the tail after y)."""
    P, Q = cw.out_hw()
    n_out = cw.N * cw.K * P * Q
    buf = torch.full((n_out + cw.K * P * Q + 64,), float("nan"), dtype=torch.float32, device=dev)
    y = buf[:n_out].view(cw.N, cw.K, P, Q)
    mm.conv2d(to_device(x, dev), to_device(w, dev), cw.stride, cw.pad, cw.dilation, out=y,
              config=cfg)
    torch.cuda.synchronize()
    return y.cpu().numpy(), buf[n_out:].cpu().numpy()


def check(y, x, w, cw, exact):
    y64, s64 = oracle.conv2d(x, w, cw.stride, cw.pad, cw.dilation)
    r = verify.exact(y, y64) if exact else verify.within_tol(y, y64, s64, REL_TOL)
    assert r, f"{cw.describe()}: {r}"


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("geo", GEOMETRIES, ids=GEO_IDS)
def test_integer_inputs_bit_exact(dev, geo, cfg):
    cw, x, w = make_inputs(geo, "int4", 2101)
    y, tail = run_gpu(x, w, cw, dev, cfg)
    check(y, x, w, cw, exact=True)
    assert np.isnan(tail).all(), "wrote past the end of y"


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("geo", GEOMETRIES, ids=GEO_IDS)
def test_random_inputs_within_tolerance(dev, geo, cfg):
    cw, x, w = make_inputs(geo, "normal", 2102)
    y, _ = run_gpu(x, w, cw, dev, cfg)
    check(y, x, w, cw, exact=False)


@pytest.mark.parametrize("cfg", [None] + CONFIGS)
def test_pointwise_large_maps_take_the_batched_gemm(dev, cfg):
    # 1x1, unit stride, no padding, H W >= 1024: each image is a C x HW matrix
    geo = ("1x1, 40x33 maps", 3, 20, 40, 33, 9, 1, 1, (1, 1), (0, 0), (1, 1))
    for dist, exact in (("int4", True), ("u11", False)):
        cw, x, w = make_inputs(geo, dist, 2103)
        y, tail = run_gpu(x, w, cw, dev, cfg)
        check(y, x, w, cw, exact)
        assert np.isnan(tail).all()


def test_default_choice_small_workload(dev):
    cw = wl.CONV_WORKLOADS["conv_small"]
    x, w = wl.conv_inputs(cw)
    y, _ = run_gpu(x, w, cw, dev)
    check(y, x, w, cw, exact=False)
    cwi = cw.with_dist("int4")
    x, w = wl.conv_inputs(cwi)
    y, _ = run_gpu(x, w, cwi, dev)
    check(y, x, w, cwi, exact=True)


@pytest.mark.parametrize("name", [n for n in wl.CONV_WORKLOADS if n != "conv_small"])
def test_full_size_workloads_sampled_images(dev, name):
    """The layer shapes at full size, in the configuration mm_conv2d_f32 chooses; the
    oracle recomputes the sampled images (each image's outputs depend on it alone)."""
    _full_size_check(dev, wl.CONV_WORKLOADS[name], None)


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("name", ["conv3x3", "conv7x7_s2"])
def test_full_size_every_config(dev, name, cfg):
    _full_size_check(dev, wl.CONV_WORKLOADS[name], cfg)


def _full_size_check(dev, cw, cfg):
    x, w = wl.conv_inputs(cw)
    used = mm.mm_conv2d_f32_select(*cw.geometry()) if cfg is None else cfg
    print(f"\n{cw.describe()}: config {used}", flush=True)
    y = mm.conv2d(to_device(x, dev), to_device(w, dev), cw.stride, cw.pad, cw.dilation, config=cfg)
    torch.cuda.synchronize()
    imgs = wl.sample_images(cw)
    got = y[torch.from_numpy(imgs).to(dev)].cpu().numpy()
    assert np.isfinite(y.sum().item())
    y64, s64 = oracle.conv2d(np.ascontiguousarray(x[imgs]), w, cw.stride, cw.pad, cw.dilation)
    r = verify.within_tol(got, y64, s64, REL_TOL)
    assert r, f"{cw.describe()}, images {imgs}: {r}"


def test_zero_channels_gives_zeros(dev):
    N, K, H, W = 2, 3, 5, 4
    x = torch.empty((N, 0, H, W), dtype=torch.float32, device=dev)
    w = torch.empty((K, 0, 3, 3), dtype=torch.float32, device=dev)
    y = torch.full((N, K, H, W), float("nan"), dtype=torch.float32, device=dev)
    mm.conv2d(x, w, pad=(1, 1), out=y)
    torch.cuda.synchronize()
    assert (y == 0).all().item()


def test_no_outputs_is_a_no_op(dev):
    x = torch.empty((0, 3, 5, 5), dtype=torch.float32, device=dev)
    w = torch.ones((4, 3, 3, 3), dtype=torch.float32, device=dev)
    y = mm.conv2d(x, w)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 4, 3, 3)


def test_repeated_calls_identical(dev):
    # fixed summation order: the same inputs give the same bits every time
    cw = wl.CONV_WORKLOADS["conv_small"]
    x, w = wl.conv_inputs(cw)
    xd, wd = to_device(x, dev), to_device(w, dev)
    first = mm.conv2d(xd, wd, cw.stride, cw.pad, cw.dilation)
    for _ in range(3):
        again = mm.conv2d(xd, wd, cw.stride, cw.pad, cw.dilation)
        torch.cuda.synchronize()
        assert torch.equal(first, again)


@pytest.mark.parametrize("H,W", [(0, 0), (0, 4), (3, 0)])
def test_empty_input_plane_gives_zeros(dev, H, W):
    # an input plane with no pixels but padding that still gives outputs: every tap of
    # the sum lands in the zero padding, so y is all zeros, as the oracle computes
    N, C, K, R, S, pad = 2, 3, 4, 3, 3, (2, 2)
    x = np.zeros((N, C, H, W), np.float32)
    w = wl.random_matrix(2104, K, C * R * S, "int4").reshape(K, C, R, S)
    y64, _ = oracle.conv2d(x, w, (1, 1), pad, (1, 1))
    P, Q = y64.shape[2:]
    assert P >= 1 and Q >= 1
    y = torch.full((N, K, P, Q), float("nan"), dtype=torch.float32, device=dev)
    mm.conv2d(torch.empty((N, C, H, W), dtype=torch.float32, device=dev), to_device(w, dev),
              pad=pad, out=y)
    torch.cuda.synchronize()
    r = verify.exact(y.cpu().numpy(), y64)
    assert r, r
    assert (y == 0).all().item()
