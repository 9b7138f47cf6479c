"""The CPU oracle against its pins (closed forms, page counts, exact arithmetic).

Runs on the CPU only. See tests/oracle_pins.py for what each pin fixes.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


@settings(max_examples=60, deadline=None)
@given(M=st.integers(0, 12), N=st.integers(0, 12), K=st.integers(0, 12),
       seed=st.integers(0, 2**31 - 1))
def test_bruteforce_sweep_int(M, N, K, seed):
    """Every shape with extents 0..12 and integer entries in [-4, 4]: exact match with a
    Python-int triple loop."""
    rng = np.random.default_rng(seed)
    A = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    B = rng.integers(-4, 5, size=(K, N)).astype(np.float32)
    C, S = oracle.gemm(A, B, threads=3)
    Cw, Sw = oracle_pins._brute_int_gemm(A, B)
    assert np.array_equal(C, Cw) and np.array_equal(S, Sw)


def test_rejects_bad_arguments(orc):
    with pytest.raises(ValueError):
        orc.gemm(np.ones((2, 3), np.float32), np.ones((4, 2), np.float32))
    with pytest.raises(TypeError):
        orc.gemm(np.ones((2, 3), np.float64), np.ones((3, 2), np.float32))
    with pytest.raises(RuntimeError):
        orc.gemm(np.ones((2, 3), np.float32), np.ones((3, 2), np.float32), rows=[2])
    with pytest.raises(ValueError):
        orc.gemv(np.ones((2, 3), np.float32), np.ones(4, np.float32))
