"""GPU parity of the 16-bit-input GEMM (bf16 and fp16 in, fp32 accumulate and out).

The inputs are drawn in fp32, rounded to the 16-bit format (round to nearest even),
and the oracle multiplies the rounded values exactly (they are exact in fp32).
Bars as for the fp32 GEMM: integer inputs bit-exact (every product and partial
sum is an integer below 2^24), random inputs within 1e-5 * sum_k |A_ik B_kj|.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import verify
import tiled_gemm_gemv_amd as mm
import workloads as wl
from gpu_helpers import nan_output, outside_untouched, require_gpu

pytestmark = pytest.mark.gpu

REL_TOL = 1e-5
FORMATS = {
    "bf16": (wl.to_bf16_bits, wl.bf16_bits_to_f32, torch.bfloat16),
    "f16": (wl.to_f16_bits, wl.f16_bits_to_f32, torch.float16),
}


@pytest.fixture(scope="module")
def dev():
    d = require_gpu()
    mm.load()
    return d


def n16():
    try:
        return mm.mm_gemm_h16_num_configs()
    except OSError:
        return 3


CONFIGS = list(range(n16()))


def quantize(a, fmt):
    to_bits, to_f32, tdtype = FORMATS[fmt]
    bits = to_bits(a)
    return bits, to_f32(bits)


def on_device(bits, fmt, dev, ld=None, offset=0):
    """uint16 bit patterns -> a device tensor of the 16-bit dtype (optionally a view
    with row stride ld, `offset` elements into a NaN-filled buffer)."""
    tdtype = FORMATS[fmt][2]
    rows, cols = bits.shape
    t = torch.from_numpy(bits.view(np.int16)).to(dev).view(tdtype)
    if ld is None and offset == 0:
        return t
    ld = ld or cols
    buf = torch.full(((rows - 1) * ld + cols + offset + 8,), float("nan"), dtype=tdtype, device=dev)
    view = torch.as_strided(buf, (rows, cols), (ld, 1), offset)
    view.copy_(t)
    return view


def run(A, B, fmt, dev, cfg=None, lda=None, ldb=None, offs=(0, 0), ldc=None):
    """C = A B on the GPU after rounding A and B to the 16-bit format; with ldc, C is a view
    with that row stride into a NaN-filled buffer, whose gaps must stay NaN."""
    Ab, Af = quantize(A, fmt)
    Bb, Bf = quantize(B, fmt)
    M, N = A.shape[0], B.shape[1]
    out = buf = None
    if ldc is not None:
        buf, out = nan_output(M, N, ldc, dev)
    C = mm.gemm16(on_device(Ab, fmt, dev, lda, offs[0]), on_device(Bb, fmt, dev, ldb, offs[1]),
                  out=out, config=cfg)
    torch.cuda.synchronize()
    if buf is not None:
        assert outside_untouched(buf, M, N), "wrote outside C"
    return C.cpu().numpy(), Af, Bf


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cfg", CONFIGS + [None])
@pytest.mark.parametrize("name", ["gemm128", "gemm1024", "gemm_ragged"])
def test_workloads(dev, fmt, cfg, name):
    w = wl.WORKLOADS[name]
    A, B = wl.gemm_inputs(w)
    C, Af, Bf = run(A, B, fmt, dev, cfg)
    C64, S64 = oracle.gemm(Af, Bf)
    r = verify.within_tol(C, C64, S64, REL_TOL)
    assert r, str(r)
    A, B = wl.gemm_inputs(w.with_dist("int4"))
    C, Af, Bf = run(A, B, fmt, dev, cfg)
    C64, _ = oracle.gemm(Af, Bf)
    r = verify.exact(C, C64)
    assert r, str(r)


# Aligned shapes on the direct HBM -> LDS pipeline (K % 32 == 0, N % 8 == 0): K of one
# step of 32, of whole steps of 64 and of whole steps plus a tail step, M and N that are
# not tile multiples (clamped rows, shifted last tile column, masked stores), a single row.
DIRECT_SHAPES = [(1, 8, 32), (37, 8, 64), (300, 264, 96), (257, 520, 128), (300, 264, 192),
                 (129, 136, 4096), (1000, 1528, 800)]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cfg", [5, 6, 7, None])
@pytest.mark.parametrize("shape", DIRECT_SHAPES)
def test_direct_pipeline_shapes(dev, fmt, cfg, shape):
    M, N, K = shape
    A = wl.random_matrix(700 + M, M, K, "int4")
    B = wl.random_matrix(800 + N, K, N, "int4")
    C, Af, Bf = run(A, B, fmt, dev, cfg)
    C64, _ = oracle.gemm(Af, Bf)
    r = verify.exact(C, C64)
    assert r, f"{shape}: {r}"
    A = wl.random_matrix(900 + M, M, K, "normal")
    B = wl.random_matrix(1000 + N, K, N, "normal")
    C, Af, Bf = run(A, B, fmt, dev, cfg)
    C64, S64 = oracle.gemm(Af, Bf)
    r = verify.within_tol(C, C64, S64, REL_TOL)
    assert r, f"{shape}: {r}"


# Shapes for the direct pipeline's general edges: K tails of 1 to 63 after whole K-steps
# (the tail step overlaps the one before), K of exactly one step of 32 or 64, N just past a
# tile width (the last tile column's B panel moves left), N below the tile width (a
# multiple of 8), odd widths and leading dimensions (2-byte-aligned rows), a single row.
GENERAL_SHAPES = [(1000, 1531, 777), (1, 65, 65), (37, 64, 64), (70, 129, 127), (130, 257, 33),
                  (300, 200, 1000), (64, 40, 100), (129, 67, 191), (257, 520, 96), (65, 300, 4097)]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cfg", [c for c in CONFIGS if c >= 5] + [None])
@pytest.mark.parametrize("shape", GENERAL_SHAPES, ids=[f"{m}x{n}x{k}" for m, n, k in GENERAL_SHAPES])
def test_direct_general_edges(dev, fmt, cfg, shape):
    M, N, K = shape
    A = wl.random_matrix(1100 + M, M, K, "int4")
    B = wl.random_matrix(1200 + N, K, N, "int4")
    # packed, then offset starts with odd leading dimensions and NaN around the views
    for lda, ldb, offs in ((None, None, (0, 0)), (K + 1, N + 3, (1, 3))):
        C, Af, Bf = run(A, B, fmt, dev, cfg, lda=lda, ldb=ldb, offs=offs, ldc=N + 5)
        C64, _ = oracle.gemm(Af, Bf)
        r = verify.exact(C, C64)
        assert r, f"{shape} lda={lda} ldb={ldb} offs={offs}: {r}"
    A = wl.random_matrix(1300 + M, M, K, "normal")
    B = wl.random_matrix(1400 + N, K, N, "normal")
    C, Af, Bf = run(A, B, fmt, dev, cfg, lda=K + 3, ldb=N + 1, offs=(3, 1))
    C64, S64 = oracle.gemm(Af, Bf)
    r = verify.within_tol(C, C64, S64, REL_TOL)
    assert r, f"{shape}: {r}"


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cfg", CONFIGS)
def test_permutation_and_edges(dev, fmt, cfg):
    M = K = 96
    perm = np.random.default_rng(6).permutation(K)
    P = np.zeros((M, K), np.float32)
    P[np.arange(M), perm] = 1
    B = (np.arange(K * 80, dtype=np.float32).reshape(K, 80) % 251) - 125   # exact in 16 bits
    C, _, Bf = run(P, B, fmt, dev, cfg)
    assert np.array_equal(C, Bf[perm])
    rng = np.random.default_rng(200 + cfg)
    edge = [1, 2, 3, 7, 8, 9, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    for t in range(16):
        M, N, K = (int(v) for v in rng.choice(edge, 3))
        A = wl.random_matrix(3000 + t, M, K, "int4")
        B = wl.random_matrix(4000 + t, K, N, "int4")
        C, Af, Bf = run(A, B, fmt, dev, cfg)
        C64, _ = oracle.gemm(Af, Bf)
        r = verify.exact(C, C64)
        assert r, f"{(M, N, K)}: {r}"


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("lds,offs", [((None, None), (0, 0)), ((203, 190), (1, 3)),
                                      ((208, 188), (0, 4))])
def test_strided_unaligned(dev, fmt, cfg, lds, offs):
    """Odd leading dimensions and starts off 16-byte alignment (2-byte loads), and
    aligned ones (16- and 8-byte loads); NaN around the views must not leak in."""
    M, N, K = 150, 181, 200
    A = wl.random_matrix(51, M, K, "int4")
    B = wl.random_matrix(52, K, N, "int4")
    C, Af, Bf = run(A, B, fmt, dev, cfg, lda=lds[0], ldb=lds[1], offs=offs)
    C64, _ = oracle.gemm(Af, Bf)
    r = verify.exact(C, C64)
    assert r, str(r)


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cfg", [5, 6, 7])
@pytest.mark.parametrize("K", [96, 192])
def test_direct_strided_views(dev, fmt, cfg, K):
    """The direct pipeline addresses its loads from the tile's corner plus a fixed offset
    per lane: leading dimensions beyond the width (here multiples of 8, so every lane is
    16-byte aligned) with NaN around the views; K = 96 (a whole K-step of 64 and a tail
    step over [32, 96)) and K = 192 (three whole steps)."""
    M, N = 300, 264
    A = wl.random_matrix(53, M, K, "int4")
    B = wl.random_matrix(54, K, N, "int4")
    C, Af, Bf = run(A, B, fmt, dev, cfg, lda=K + 24, ldb=N + 40, offs=(8, 16))
    C64, _ = oracle.gemm(Af, Bf)
    r = verify.exact(C, C64)
    assert r, str(r)


@pytest.mark.parametrize("cfg", [5, 6, 7])
def test_direct_huge_leading_dimension(dev, cfg):
    """lda of 9M elements: 255 rows of it exceed the 32-bit lane offsets of the direct
    pipeline, so the register-staged tile of the same size runs; still exact."""
    A = wl.random_matrix(55, 3, 64, "int4")
    B = wl.random_matrix(56, 64, 64, "int4")
    C, Af, Bf = run(A, B, "bf16", dev, cfg, lda=9_000_000)
    C64, _ = oracle.gemm(Af, Bf)
    r = verify.exact(C, C64)
    assert r, str(r)


def test_k_zero(dev):
    for fmt in FORMATS:
        tdtype = FORMATS[fmt][2]
        out = torch.full((5, 7), float("nan"), device=dev)
        mm.gemm16(torch.empty((5, 0), dtype=tdtype, device=dev),
                  torch.empty((0, 7), dtype=tdtype, device=dev), out=out)
        torch.cuda.synchronize()
        assert (out == 0).all().item()


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_projection_spot_rows(dev, fmt):
    """The 8192 x 4096 x 14336 projection with 16-bit inputs: 64 sampled rows."""
    w = wl.WORKLOADS["gemm_proj"]
    A, B = wl.gemm_inputs(w)
    Ab, Af = quantize(A, fmt)
    Bb, Bf = quantize(B, fmt)
    del A, B
    C = mm.gemm16(on_device(Ab, fmt, dev), on_device(Bb, fmt, dev))
    torch.cuda.synchronize()
    rows = wl.sample_rows(w, 64)
    got = C[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del C
    C64, S64 = oracle.gemm(Af, Bf, rows=rows)
    r = verify.within_tol(got, C64, S64, REL_TOL)
    assert r, str(r)
