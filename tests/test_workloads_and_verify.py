"""Seeded input generators and the result checker (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import verify
import workloads as wl


def test_generators_are_reproducible_and_distinct():
    w = wl.WORKLOADS["gemm_ragged"]
    A1, B1 = wl.gemm_inputs(w)
    A2, B2 = wl.gemm_inputs(w)
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2)
    assert A1.shape == (1000, 777) and B1.shape == (777, 1531)
    assert A1.dtype == np.float32 and A1.flags.c_contiguous
    assert not np.array_equal(A1[:100, :100], B1[:100, :100])


def test_uniform_is_half_open_and_exact():
    u = wl.draw(wl.rng_for(7, 0), (1 << 20,), "u11")
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(float(u.mean())) < 5e-3
    # 2u - 1 with u a float32 multiple of 2**-24 stays on the 2**-23 grid
    assert np.all(np.ldexp(u.astype(np.float64), 23) == np.round(np.ldexp(u.astype(np.float64), 23)))


def test_integer_variant_range():
    v = wl.draw(wl.rng_for(3, 1), (100000,), "int4")
    assert set(np.unique(v).tolist()) == set(range(-4, 5))


def test_projection_scales():
    w = wl.WORKLOADS["gemm_proj"]
    B = wl.draw(wl.rng_for(w.seed, wl.OPERAND_B), (512, 1024), "normal", w.b_std)
    assert abs(float(B.std()) - 1 / 64) < 2e-4
    assert w.b_std == 1 / 64 and w.K == 4096


def test_workload_table_matches_shapes():
    W = wl.WORKLOADS
    assert (W["gemm128"].M, W["gemm128"].N, W["gemm128"].K) == (128, 128, 128)
    assert (W["gemv4096"].M, W["gemv4096"].N) == (4096, 4096)
    assert (W["gemm1024"].M, W["gemm1024"].N, W["gemm1024"].K) == (1024, 1024, 1024)
    assert (W["gemm_ragged"].M, W["gemm_ragged"].N, W["gemm_ragged"].K) == (1000, 1531, 777)
    assert (W["gemm_proj"].M, W["gemm_proj"].N, W["gemm_proj"].K) == (8192, 14336, 4096)


def test_sample_rows_distinct_sorted():
    w = wl.WORKLOADS["gemm_proj"]
    r = wl.sample_rows(w)
    assert len(r) == 64 and len(set(r.tolist())) == 64 and np.all(np.diff(r) > 0)
    assert r.min() >= 0 and r.max() < w.M
    assert np.array_equal(r, wl.sample_rows(w))


def test_embed_poisons_gaps():
    a = np.arange(6, dtype=np.float32).reshape(2, 3)
    buf, view = wl.embed(a, 5, extra_rows=1)
    assert buf.shape == (3, 5) and np.array_equal(view, a)
    assert np.isnan(buf[:, 3:]).all() and np.isnan(buf[2]).all()
    assert view.strides == (20, 4)


def test_exact_checker():
    A = wl.draw(wl.rng_for(5, 0), (20, 30), "int4")
    B = wl.draw(wl.rng_for(5, 1), (30, 10), "int4")
    C64, _ = oracle.gemm(A, B)
    good = C64.astype(np.float32)
    assert verify.exact(good, C64)
    bad = good.copy()
    bad.view(np.uint32)[3, 4] ^= 1                     # one flipped bit
    r = verify.exact(bad, C64)
    assert not r and r.first_bad == (3, 4) and r.bad == 1
    nan = good.copy()
    nan[0, 0] = np.nan
    assert not verify.exact(nan, C64)
    negz = good.copy()
    negz[C64 == 0] = -0.0                                 # -0 == +0 by value
    assert verify.exact(negz, C64)


def test_tolerance_checker_boundary():
    A = wl.draw(wl.rng_for(9, 0), (16, 64), "u11")
    B = wl.draw(wl.rng_for(9, 1), (64, 12), "u11")
    C64, S64 = oracle.gemm(A, B)
    assert verify.within_tol(C64.astype(np.float32), C64, S64)
    # fp32 sequential sums pass with a wide margin
    C32 = np.zeros((16, 12), np.float32)
    for k in range(64):
        C32 += A[:, k:k + 1] * B[k:k + 1, :]
    r = verify.within_tol(C32, C64, S64)
    assert r and r.worst < 0.1
    # a 2e-5 * S perturbation of one element is flagged
    pert = (C64 + 0).astype(np.float64)
    pert[5, 7] += 2e-5 * S64[5, 7]
    r = verify.within_tol(pert.astype(np.float32), C64, S64)
    assert not r and r.first_bad == (5, 7)
    inf = C64.astype(np.float32)
    inf[1, 1] = np.inf
    assert not verify.within_tol(inf, C64, S64)


def test_tolerance_zero_magnitude_demands_zero():
    ref = np.zeros((2, 2))
    assert verify.within_tol(np.zeros((2, 2), np.float32), ref, ref)
    out = np.zeros((2, 2), np.float32)
    out[1, 0] = 1e-30
    assert not verify.within_tol(out, ref, ref)


def test_checkers_reject_shape_mismatch():
    with pytest.raises(ValueError):
        verify.exact(np.zeros((2, 3), np.float32), np.zeros((3, 2)))


def test_sixteen_bit_rounding_matches_torch():
    """to_bf16_bits / to_f16_bits round to nearest even, as torch's CPU casts do, and
    the bit patterns convert back to the same values exactly."""
    import torch
    a = np.concatenate([wl.draw(wl.rng_for(11, 0), (20000,), "normal"),
                        np.array([1.00390625, 1.01171875, -2.5, 0.0, 65504.0, 1e-3], np.float32)])
    t = torch.from_numpy(a)
    bf = wl.to_bf16_bits(a)
    assert np.array_equal(bf, t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(wl.bf16_bits_to_f32(bf), t.to(torch.bfloat16).float().numpy())
    h = wl.to_f16_bits(a)
    assert np.array_equal(h, t.to(torch.float16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(wl.f16_bits_to_f32(h), t.to(torch.float16).float().numpy())
