"""Pins for the CPU oracle: checks that tie it to something other than itself.

Each pin is a function pin_*(orc) that raises AssertionError when the oracle
`orc` (an oracle.Oracle) disagrees with what the pages or plain mathematics fix:
hand-worked products, the pages' operation counts, closed forms (all-ones,
identity, permutation, one-hot), exact rational arithmetic within the fp64
error bound, brute force on tiny integer inputs, and algebraic invariants that
are exact on small integers. tests/test_oracle.py runs them on the real oracle;
tests/test_oracle_mutants.py runs them on copies of oracle.c with a planted
mistake and requires every mistake to be caught.
"""
import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _ints(seed, shape, lo=-4, hi=4):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def _floats(seed, shape):
    return (np.random.default_rng(seed).random(shape, dtype=np.float32) * np.float32(2)
            - np.float32(1))


def _brute_int_gemm(A, B):
    """Exact integer triple loop in Python ints (independent of the C code)."""
    M, K = A.shape
    N = B.shape[1]
    a = [[int(v) for v in row] for row in A]
    b = [[int(v) for v in row] for row in B]
    C = [[0] * N for _ in range(M)]
    S = [[0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            acc = mag = 0
            for k in range(K):
                p = a[i][k] * b[k][j]
                acc += p
                mag += abs(p)
            C[i][j] = acc
            S[i][j] = mag
    return np.array(C, dtype=np.float64).reshape(M, N), np.array(S, dtype=np.float64).reshape(M, N)


def _gamma(n):
    u = 2.0 ** -53
    return n * u / (1 - n * u)


# --------------------------------------------------------------------------- GEMM

def pin_golden_small_products(orc):
    """Hand-worked products (tests/golden/small_products.json) are reproduced exactly."""
    g = _golden("small_products.json")
    for case in g["gemm"]:
        A = np.array(case["A"], dtype=np.float32)
        B = np.array(case["B"], dtype=np.float32)
        C, _ = orc.gemm(A, B, threads=1)
        assert np.array_equal(C, np.array(case["C"], dtype=np.float64)), case["name"]
    for case in g["gemv"]:
        A = np.array(case["A"], dtype=np.float32)
        x = np.array(case["x"], dtype=np.float32)
        y, _ = orc.gemv(A, x, threads=1)
        assert np.array_equal(y, np.array(case["y"], dtype=np.float64)), case["name"]


def pin_bruteforce_int(orc):
    """Tiny integer shapes (including 0 and 1 extents) equal an exact Python-int triple loop."""
    shapes = [(1, 1, 1), (2, 3, 4), (3, 1, 5), (5, 4, 1), (4, 7, 3), (7, 2, 9), (6, 6, 6),
              (1, 9, 2), (9, 1, 8), (3, 5, 0), (0, 4, 3), (4, 0, 3)]
    for t, (M, N, K) in enumerate(shapes):
        A = _ints(100 + t, (M, K), -9, 9)
        B = _ints(200 + t, (K, N), -9, 9)
        C, S = orc.gemm(A, B, threads=2)
        Cw, Sw = _brute_int_gemm(A, B)
        assert np.array_equal(C, Cw), (M, N, K)
        assert np.array_equal(S, Sw), (M, N, K)


def pin_exact_rational_within_bound(orc):
    """Random fp32 inputs: the fp64 sums lie within the recursive-summation bound of the
    exact rational sums, gamma_K * sum|a b| with unit roundoff 2**-53."""
    M, N, K = 4, 5, 37
    A = _floats(11, (M, K))
    B = _floats(12, (K, N))
    C, S = orc.gemm(A, B, threads=1)
    fa = [[Fraction(float(v)) for v in row] for row in A]
    fb = [[Fraction(float(v)) for v in row] for row in B]
    bound = _gamma(K)
    for i in range(M):
        for j in range(N):
            prods = [fa[i][k] * fb[k][j] for k in range(K)]
            exact = sum(prods, Fraction(0))
            mag = sum((abs(p) for p in prods), Fraction(0))
            assert abs(Fraction(C[i, j]) - exact) <= bound * mag, (i, j)
            assert abs(Fraction(S[i, j]) - mag) <= bound * mag, (i, j)


def pin_all_ones(orc):
    """All-ones A and B give C[i][j] = K and sum|a b| = K everywhere (ragged shape)."""
    M, N, K = 7, 13, 129
    C, S = orc.gemm(np.ones((M, K), np.float32), np.ones((K, N), np.float32), threads=3)
    assert np.all(C == K) and np.all(S == K)


def pin_identity(orc):
    """A = I gives C = B; B = I gives C = A, bit for bit (each sum has one non-zero term)."""
    n, m = 9, 14
    B = _floats(21, (n, m))
    C, _ = orc.gemm(np.eye(n, dtype=np.float32), B)
    assert np.array_equal(C, B.astype(np.float64))
    A = _floats(22, (m, n))
    C, _ = orc.gemm(A, np.eye(n, dtype=np.float32))
    assert np.array_equal(C, A.astype(np.float64))


def pin_rectangular_identity(orc):
    """A[i][k] = delta(i, k) (M x K, M != K) gives C[i] = B[i] for i < K and 0 beyond."""
    for M, K, N in [(9, 5, 6), (4, 7, 3)]:
        B = _floats(31 + M, (K, N))
        C, _ = orc.gemm(np.eye(M, K, dtype=np.float32), B)
        want = np.zeros((M, N))
        r = min(M, K)
        want[:r] = B[:r]
        assert np.array_equal(C, want), (M, K, N)


def pin_permutation(orc):
    """A permutation matrix P with unique-integer B gives C = P B exactly."""
    K, N = 11, 6
    perm = np.random.default_rng(41).permutation(K)
    P = np.zeros((K, K), np.float32)
    P[np.arange(K), perm] = 1
    B = np.arange(K * N, dtype=np.float32).reshape(K, N) - 20
    C, _ = orc.gemm(P, B)
    assert np.array_equal(C, B[perm].astype(np.float64))


def pin_one_hot(orc):
    """A with a single 1 at (i, k) gives C whose row i is B's row k and is zero elsewhere;
    with B one-hot at (k, j), C's column j is A's column k. Localises index mix-ups."""
    M, K, N = 5, 7, 4
    Bf = _floats(51, (K, N))
    Af = _floats(52, (M, K))
    for (i, k) in [(0, 0), (4, 6), (2, 3), (1, 5)]:
        A = np.zeros((M, K), np.float32)
        A[i, k] = 1
        C, _ = orc.gemm(A, Bf)
        want = np.zeros((M, N))
        want[i] = Bf[k]
        assert np.array_equal(C, want), (i, k)
    for (k, j) in [(0, 0), (6, 3), (3, 1)]:
        B = np.zeros((K, N), np.float32)
        B[k, j] = 1
        C, _ = orc.gemm(Af, B)
        want = np.zeros((M, N))
        want[:, j] = Af[:, k]
        assert np.array_equal(C, want), (k, j)


def pin_transpose_identity(orc):
    """(A B)^T = B^T A^T, exact on small integers, non-square."""
    A = _ints(61, (6, 11))
    B = _ints(62, (11, 8))
    C, _ = orc.gemm(A, B)
    Ct, _ = orc.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(C.T, Ct)


def pin_linearity(orc):
    """A (B1 + B2) = A B1 + A B2, exact on small integers."""
    A = _ints(71, (5, 9))
    B1 = _ints(72, (9, 7))
    B2 = _ints(73, (9, 7))
    C12, _ = orc.gemm(A, B1 + B2)
    C1, _ = orc.gemm(A, B1)
    C2, _ = orc.gemm(A, B2)
    assert np.array_equal(C12, C1 + C2)


def pin_threads_invariant(orc):
    """Results are identical bit for bit for any thread count (rows are independent)."""
    A = _floats(81, (23, 40))
    B = _floats(82, (40, 17))
    ref = orc.gemm(A, B, threads=1)
    for t in (2, 3, 7, 64):
        got = orc.gemm(A, B, threads=t)
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), t
    x = _floats(83, (40,))
    refv = orc.gemv(A, x, threads=1)
    for t in (2, 5, 64):
        got = orc.gemv(A, x, threads=t)
        assert np.array_equal(refv[0], got[0]) and np.array_equal(refv[1], got[1]), t


def pin_row_subset(orc):
    """Asking for a subset of rows returns exactly those rows of the full product."""
    A = _floats(91, (12, 10))
    B = _floats(92, (10, 9))
    full, fullS = orc.gemm(A, B)
    rows = [5, 0, 11, 7]
    sub, subS = orc.gemm(A, B, rows=rows, threads=2)
    assert np.array_equal(sub, full[rows]) and np.array_equal(subS, fullS[rows])


def pin_strided_nan_gaps(orc):
    """Row strides beyond the matrix width: NaN in every gap and in a row past the end
    must not reach the result, which equals the packed product."""
    from workloads import embed
    M, K, N = 6, 10, 7
    A = _floats(101, (M, K))
    B = _floats(102, (K, N))
    _, Av = embed(A, K + 3, extra_rows=1)
    _, Bv = embed(B, N + 5, extra_rows=1)
    C, S = orc.gemm(Av, Bv)
    Cp, Sp = orc.gemm(A, B)
    assert np.array_equal(C, Cp) and np.array_equal(S, Sp)
    assert not np.isnan(C).any()
    x = _floats(103, (K,))
    y, s = orc.gemv(Av, x)
    yp, sp = orc.gemv(A, x)
    assert np.array_equal(y, yp) and np.array_equal(s, sp)
    assert not np.isnan(y).any()


def pin_empty_sums(orc):
    """K = 0 gives C = 0 (an empty sum, as the pages' kernels write 0); N = 0 gives y = 0."""
    C, S = orc.gemm(np.zeros((3, 0), np.float32), np.zeros((0, 4), np.float32))
    assert C.shape == (3, 4) and np.all(C == 0) and np.all(S == 0)
    y, s = orc.gemv(np.zeros((5, 0), np.float32), np.zeros(0, np.float32))
    assert y.shape == (5,) and np.all(y == 0) and np.all(s == 0)


def pin_ieee_specials(orc):
    """A NaN in A[i][k] makes all of row i NaN; an Inf in B[k][j] times a zero gives NaN."""
    A = _floats(111, (4, 5))
    B = _floats(112, (5, 6))
    A2 = A.copy()
    A2[2, 3] = np.nan
    C, _ = orc.gemm(A2, B)
    assert np.isnan(C[2]).all() and not np.isnan(np.delete(C, 2, axis=0)).any()
    A3 = A.copy()
    A3[:, 1] = [0, 1, 0, 1]
    B3 = B.copy()
    B3[1, 4] = np.inf
    C, _ = orc.gemm(A3, B3)
    assert np.isnan(C[0, 4]) and np.isnan(C[2, 4]) and np.isinf(C[1, 4]) and np.isinf(C[3, 4])


# --------------------------------------------------------------------------- GEMV

def pin_gemv_bruteforce_int(orc):
    """Integer GEMV equals the exact Python-int loop, for several ragged shapes."""
    for t, (M, N) in enumerate([(1, 1), (3, 7), (8, 1), (5, 33), (17, 4)]):
        A = _ints(121 + t, (M, N), -9, 9)
        x = _ints(131 + t, (N,), -9, 9)
        y, s = orc.gemv(A, x, threads=3)
        C, S = _brute_int_gemm(A, x.reshape(N, 1))
        assert np.array_equal(y, C[:, 0]) and np.array_equal(s, S[:, 0]), (M, N)


def pin_gemv_exact_rational_within_bound(orc):
    """Random fp32 GEMV lies within gamma_N * sum|a x| of the exact rational sum."""
    M, N = 6, 53
    A = _floats(141, (M, N))
    x = _floats(142, (N,))
    y, s = orc.gemv(A, x, threads=1)
    bound = _gamma(N)
    for i in range(M):
        prods = [Fraction(float(A[i, j])) * Fraction(float(x[j])) for j in range(N)]
        exact = sum(prods, Fraction(0))
        mag = sum((abs(p) for p in prods), Fraction(0))
        assert abs(Fraction(y[i]) - exact) <= bound * mag, i
        assert abs(Fraction(s[i]) - mag) <= bound * mag, i


def pin_gemv_all_ones_and_onehot(orc):
    """All-ones GEMV gives y = N; x one-hot at j gives y = column j of A."""
    M, N = 9, 77
    y, s = orc.gemv(np.ones((M, N), np.float32), np.ones(N, np.float32))
    assert np.all(y == N) and np.all(s == N)
    A = _floats(151, (M, N))
    for j in (0, 40, N - 1):
        x = np.zeros(N, np.float32)
        x[j] = 1
        y, _ = orc.gemv(A, x)
        assert np.array_equal(y, A[:, j].astype(np.float64)), j


def pin_gemv_is_gemm_column(orc):
    """GEMV(A, x) equals GEMM(A, x as an N x 1 matrix): same sums, same order, same bits."""
    A = _floats(161, (13, 29))
    x = _floats(162, (29,))
    y, s = orc.gemv(A, x)
    C, S = orc.gemm(A, x.reshape(-1, 1))
    assert np.array_equal(y, C[:, 0]) and np.array_equal(s, S[:, 0])


# --------------------------------------------------------------------- page counts

def pin_page_operation_counts(orc):
    """With all-ones inputs every product is 1, so the outputs add up to the number of
    multiply-adds, which the pages give for their two example workloads."""
    g = _golden("page_counts.json")
    fc = g["fc_layer_macs"]
    y, _ = orc.gemv(np.ones((fc["M"], fc["N"]), np.float32), np.ones(fc["N"], np.float32))
    assert int(y.sum()) == fc["value"]
    sq = g["square_gemm_macs"]
    n = sq["n"]
    C, _ = orc.gemm(np.ones((n, n), np.float32), np.ones((n, n), np.float32))
    assert int(C.sum()) == sq["value"]




# ---------------------------------------------------------------- convolution

def _brute_int_conv(x, w, stride, pad, dil):
    """Exact Python-int convolution from the definition (independent of the C code)."""
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    P = (H + 2 * ph - dh * (R - 1) - 1) // sh + 1
    Q = (W + 2 * pw - dw * (S - 1) - 1) // sw + 1
    xi = x.astype(np.int64).tolist()
    wi = w.astype(np.int64).tolist()
    y = np.zeros((N, K, P, Q))
    s = np.zeros((N, K, P, Q))
    for n in range(N):
        for k in range(K):
            for p in range(P):
                for q in range(Q):
                    acc = mag = 0
                    for c in range(C):
                        for r in range(R):
                            for t in range(S):
                                h, v = p * sh + r * dh - ph, q * sw + t * dw - pw
                                if 0 <= h < H and 0 <= v < W:
                                    prod = xi[n][c][h][v] * wi[k][c][r][t]
                                    acc += prod
                                    mag += abs(prod)
                    y[n, k, p, q] = acc
                    s[n, k, p, q] = mag
    return y, s


def pin_conv_golden(orc):
    """Hand-worked convolutions (tests/golden/conv_examples.json) are reproduced exactly."""
    for case in _golden("conv_examples.json")["cases"]:
        y, _ = orc.conv2d(np.array(case["x"], np.float32), np.array(case["w"], np.float32),
                          case["stride"], case["pad"], case["dilation"], threads=1)
        assert np.array_equal(y, np.array(case["y"], np.float64)), case["name"]


def pin_conv_bruteforce_int(orc):
    """Integer convolutions over strides, paddings and dilations equal an exact loop."""
    cases = [((2, 3, 7, 6), (4, 3, 3, 3), (1, 1), (1, 1), (1, 1)),
             ((1, 2, 9, 8), (3, 2, 3, 2), (2, 3), (1, 0), (1, 1)),
             ((2, 1, 8, 8), (2, 1, 3, 3), (1, 2), (2, 2), (2, 3)),
             ((1, 4, 5, 5), (2, 4, 1, 1), (1, 1), (0, 0), (1, 1)),
             ((1, 2, 4, 6), (1, 2, 4, 6), (1, 1), (0, 0), (1, 1))]
    for t, (xs, ws, st, pd, dl) in enumerate(cases):
        x = _ints(300 + t, xs)
        w = _ints(400 + t, ws)
        y, s = orc.conv2d(x, w, st, pd, dl, threads=3)
        yw, sw = _brute_int_conv(x, w, st, pd, dl)
        assert np.array_equal(y, yw) and np.array_equal(s, sw), (xs, ws, st, pd, dl)


def pin_conv_1x1_is_gemm(orc):
    """A 1x1 convolution with stride 1 and no padding is, per image, the GEMM
    W (K x C) times the image as a C x (H W) matrix."""
    x = _floats(501, (2, 5, 6, 7))
    w = _floats(502, (4, 5, 1, 1))
    y, _ = orc.conv2d(x, w)
    for n in range(2):
        C64, _ = orc.gemm(w.reshape(4, 5), x[n].reshape(5, 42))
        assert np.array_equal(y[n].reshape(4, 42), C64)


def pin_conv_identity_and_delta(orc):
    """A centred delta filter (w[k][c] = delta_kc at the centre, padding 1) returns the
    input; a one-hot input returns the filter, mirrored into place."""
    x = _floats(503, (1, 3, 6, 5))
    w = np.zeros((3, 3, 3, 3), np.float32)
    for c in range(3):
        w[c, c, 1, 1] = 1
    y, _ = orc.conv2d(x, w, pad=(1, 1))
    assert np.array_equal(y, x.astype(np.float64))
    xs = np.zeros((1, 1, 7, 7), np.float32)
    xs[0, 0, 3, 3] = 1
    wf = _floats(504, (1, 1, 3, 3))
    y, _ = orc.conv2d(xs, wf)   # P = Q = 5; output (p,q) sees tap (3-p, 3-q)
    want = np.zeros((5, 5))
    for p in range(5):
        for q in range(5):
            r, t = 3 - p, 3 - q
            if 0 <= r < 3 and 0 <= t < 3:
                want[p, q] = wf[0, 0, r, t]
    assert np.array_equal(y[0, 0], want)


def pin_conv_all_ones_counts_taps(orc):
    """All-ones input and filter: each output counts the filter taps that land inside
    the padded image, C * (rows inside) * (columns inside)."""
    C, H, W, R, S = 3, 6, 5, 3, 4
    y, s = orc.conv2d(np.ones((1, C, H, W), np.float32), np.ones((2, C, R, S), np.float32),
                      stride=(2, 1), pad=(1, 2))
    P, Q = y.shape[2:]
    for p in range(P):
        rows = sum(1 for r in range(R) if 0 <= p * 2 + r - 1 < H)
        for q in range(Q):
            cols = sum(1 for t in range(S) if 0 <= q + t - 2 < W)
            assert y[0, 0, p, q] == C * rows * cols == s[0, 1, p, q]


def pin_conv_ieee_specials_and_padding(orc):
    """IEEE values through the convolution, read as the product of the filters with the
    input's im2col matrix, whose padded entries are zeros: an infinite filter tap that
    lands in the padding multiplies a zero (NaN), one that lands inside multiplies the
    pixel (infinite); a NaN pixel makes every output whose window holds it NaN."""
    x = np.full((1, 1, 1, 1), 5.0, np.float32)
    w = np.ones((2, 1, 3, 3), np.float32)
    w[0, 0, 0, 0] = np.inf   # the corner tap: in the padding for the only output
    w[1, 0, 1, 1] = -np.inf  # the centre tap: on the pixel
    y, _ = orc.conv2d(x, w, pad=(1, 1))
    assert y.shape == (1, 2, 1, 1)
    assert np.isnan(y[0, 0, 0, 0]) and y[0, 1, 0, 0] == -np.inf
    x = np.arange(1 * 2 * 5 * 6, dtype=np.float32).reshape(1, 2, 5, 6) % 7 - 3
    x[0, 1, 2, 3] = np.nan
    y, _ = orc.conv2d(x, np.ones((1, 2, 3, 3), np.float32), pad=(1, 1))
    for p in range(5):
        for q in range(6):
            assert np.isnan(y[0, 0, p, q]) == (abs(p - 2) <= 1 and abs(q - 3) <= 1), (p, q)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
CHEAP_PINS = [p for p in ALL_PINS if p is not pin_page_operation_counts]
