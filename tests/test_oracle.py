"""Pins of the CPU GEMM oracle against facts fixed by the pages and by
mathematics, never against the oracle itself:

* exact brute force with rational arithmetic on tiny shapes (every entry of
  A.B by its definition, MikPoly page part 1 item 2, untiled loop);
* closed forms: identity, permutation, all-ones, outer product (K = 1), K = 0;
* linearity in each operand (Korch page, section 3, linear-transformation
  primitive: additivity and homogeneity in every input);
* the product as K ascending rank-1 updates equals the row-by-row loop bit
  for bit, since both add each element's terms in ascending k (the order in
  which elements are visited does not change any element's rounding);
* numpy's float64 matmul (an independent library) within rounding.

Shapes use M != N != K so a transposed operand or swapped index fails.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits, bf16_bits_to_f32


def bits(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def exact_gemm(a_bits, b_bits):
    """Rational-arithmetic product: no rounding at all."""
    A = bf16_bits_to_f32(a_bits).astype(np.float64)
    B = bf16_bits_to_f32(b_bits).astype(np.float64)
    M, K = A.shape
    N = B.shape[1]
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
            out[i][j] = s
    return out


def test_bf16_rounding_rne():
    # ties to even at the bf16 boundary, exact values pass through
    one = 0x3F800000
    vals = np.array([one, one + 0x8000, one + 0x18000, one + 0x7FFF, one + 0x8001], dtype=np.uint32)
    got = f32_to_bf16_bits(vals.view(np.float32))
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F80, 0x3F81]
    assert np.array_equal(bf16_bits_to_f32(got[:1]), np.array([1.0], dtype=np.float32))


def test_bruteforce_exact_small_integers():
    rng = np.random.default_rng(7)
    for M, N, K in itertools.product(range(0, 7), range(0, 7), range(0, 7)):
        a = bits(rng.integers(-8, 9, size=(M, K)))
        b = bits(rng.integers(-8, 9, size=(K, N)) / 8.0)
        c = oracle.gemm(a, b)
        assert c.shape == (M, N)
        ex = exact_gemm(a, b)
        for i in range(M):
            for j in range(N):
                assert Fraction(float(c[i, j])) == ex[i][j], (M, N, K, i, j)


def test_bruteforce_random_within_bound():
    """Random bf16 values: the binary64 sum is within Higham's bound of the
    exact rational sum (u = 2^-53)."""
    rng = np.random.default_rng(8)
    for M, N, K in [(3, 5, 7), (6, 2, 33), (1, 9, 64)]:
        a = bits(rng.uniform(-1, 1, size=(M, K)))
        b = bits(rng.uniform(-1, 1, size=(K, N)))
        c, cabs = oracle.gemm(a, b, with_abs=True)
        ex = exact_gemm(a, b)
        u = 2.0 ** -53
        g = K * u / (1 - K * u)
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(float(c[i, j])) - ex[i][j])
                assert err <= Fraction(g * cabs[i, j]) + Fraction(1, 2 ** 1074)


def test_identity_and_permutation():
    rng = np.random.default_rng(9)
    M, K, N = 37, 29, 41
    a = bits(rng.uniform(-1, 1, size=(M, K)))
    b = bits(rng.uniform(-1, 1, size=(K, N)))
    af = bf16_bits_to_f32(a).astype(np.float64)
    bfl = bf16_bits_to_f32(b).astype(np.float64)
    assert np.array_equal(oracle.gemm(a, bits(np.eye(K))), af)
    assert np.array_equal(oracle.gemm(bits(np.eye(K)), b), bfl)
    p = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), p] = 1.0  # (P.B)[i] = B[p[i]]
    assert np.array_equal(oracle.gemm(bits(P), b), bfl[p])
    q = rng.permutation(K)
    Q = np.zeros((K, K))
    Q[q, np.arange(K)] = 1.0  # (A.Q)[:, j] = A[:, q[j]]
    assert np.array_equal(oracle.gemm(a, bits(Q)), af[:, q])


def test_ones_outer_and_empty():
    M, N, K = 5, 7, 300
    c = oracle.gemm(bits(np.ones((M, K))), bits(np.ones((K, N))))
    assert np.all(c == K)
    rng = np.random.default_rng(10)
    a = bits(rng.uniform(-1, 1, size=(6, 1)))
    b = bits(rng.uniform(-1, 1, size=(1, 8)))
    af = bf16_bits_to_f32(a).astype(np.float64)
    bfl = bf16_bits_to_f32(b).astype(np.float64)
    assert np.array_equal(oracle.gemm(a, b), af[:, 0:1] * bfl[0:1, :])
    z = oracle.gemm(np.zeros((4, 0), np.uint16), np.zeros((0, 3), np.uint16))
    assert z.shape == (4, 3) and np.all(z == 0)


def test_linearity_additive_and_homogeneous():
    rng = np.random.default_rng(11)
    M, K, N = 19, 23, 17
    a1 = rng.integers(-16, 17, size=(M, K)) / 16.0
    a2 = rng.integers(-16, 17, size=(M, K)) / 16.0
    b = rng.integers(-16, 17, size=(K, N)) / 16.0
    # every value and every partial sum below is a small dyadic: all exact
    lhs = oracle.gemm(bits(a1 + a2), bits(b))
    rhs = oracle.gemm(bits(a1), bits(b)) + oracle.gemm(bits(a2), bits(b))
    assert np.array_equal(lhs, rhs)
    b1 = rng.integers(-16, 17, size=(K, N)) / 16.0
    lhs = oracle.gemm(bits(a1), bits(b + b1))
    rhs = oracle.gemm(bits(a1), bits(b)) + oracle.gemm(bits(a1), bits(b1))
    assert np.array_equal(lhs, rhs)
    for p in (-3, 4):
        assert np.array_equal(oracle.gemm(bits(a1 * 2.0 ** p), bits(b)), 2.0 ** p * oracle.gemm(bits(a1), bits(b)))


def test_outer_product_form_equals_row_form_bitwise():
    """The product as K ascending rank-1 updates equals the row-by-row loop
    bit for bit; summing one element's terms in descending k instead (a
    plausible slip, planted here on the CPU) changes the rounding, so the
    pin would see a wrong summation order."""
    rng = np.random.default_rng(12)
    for M, N, K in [(70, 45, 99), (33, 65, 31), (1, 1, 257)]:
        a = bits(rng.uniform(-1, 1, size=(M, K)))
        b = bits(rng.uniform(-1, 1, size=(K, N)))
        assert np.array_equal(oracle.gemm_outer(a, b), oracle.gemm(a, b))
    # terms 1, 2^-53, 2^-53: in ascending k each small term is a tie that
    # rounds back to 1 (the sum is 1); in descending k the two small terms
    # first add exactly to 2^-52, which then survives (1 + 2^-52)
    a = bits(np.array([[1.0, 2.0 ** -53, 2.0 ** -53]]))
    b = bits(np.ones((3, 1)))
    assert oracle.gemm(a, b)[0, 0] == 1.0 and oracle.gemm_outer(a, b)[0, 0] == 1.0
    A = bf16_bits_to_f32(a).astype(np.float64)
    desc = 0.0
    for k in (2, 1, 0):
        desc += A[0, k]
    assert desc == 1.0 + 2.0 ** -52


def test_numpy_crosscheck():
    rng = np.random.default_rng(13)
    M, K, N = 123, 301, 77
    a = bits(rng.uniform(-1, 1, size=(M, K)))
    b = bits(rng.normal(0, 1, size=(K, N)))
    c, cabs = oracle.gemm(a, b, with_abs=True)
    ref = bf16_bits_to_f32(a).astype(np.float64) @ bf16_bits_to_f32(b).astype(np.float64)
    assert np.all(np.abs(c - ref) <= 1e-13 * cabs + 1e-300)


def test_batched_and_entries_agree():
    rng = np.random.default_rng(14)
    batch, M, N, K = 3, 21, 13, 40
    a = bits(rng.uniform(-1, 1, size=(batch, M, K)))
    b = bits(rng.uniform(-1, 1, size=(batch, K, N)))
    cb = oracle.gemm(a, b)
    for z in range(batch):
        assert np.array_equal(cb[z], oracle.gemm(a[z], b[z]))
    rows = rng.integers(0, M, size=50)
    cols = rng.integers(0, N, size=50)
    bidx = rng.integers(0, batch, size=50)
    vals, _ = oracle.gemm_entries(a, b, rows, cols, bidx)
    assert np.array_equal(vals, cb[bidx, rows, cols])


def test_planted_mistake_is_caught():
    """A transposed operand (a plausible bug) breaks the permutation pin."""
    rng = np.random.default_rng(15)
    K = 9
    b = bits(rng.uniform(-1, 1, size=(K, K)))
    p = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), p] = 1.0
    good = oracle.gemm(bits(P), b)
    wrong = oracle.gemm(bits(P.T), b)  # the planted mistake, on the CPU
    assert np.array_equal(good, bf16_bits_to_f32(b).astype(np.float64)[p])
    assert not np.array_equal(wrong, good)


def _f32_recursive_sum(terms):
    """Left-to-right binary32 summation, every partial sum rounded to
    binary32 by numpy (an independent model of the GPU's fp32 accumulator)."""
    acc = np.float32(0.0)
    for t in terms:
        acc = np.float32(acc + np.float32(t))
    return float(acc)


def test_error_bound_is_attained_by_rounding_every_add_down():
    """Tightness: 1 followed by K-1 copies of d = 2^-24 (1 - 2^-8) (a bf16
    product: 2^-24 times the bf16 value 1 - 2^-8).  Each d is below half a
    binary32 ulp of 1, so every add rounds back to 1: the binary32 sum is 1
    and its error is (K-1) d, within a few per cent of gamma_K * sum|x|.
    A bound that used u = 2^-23, dropped the factor K or its 1/(1 - Ku)
    would be off by far more than that."""
    d = 2.0 ** -24 * (1.0 - 2.0 ** -8)
    for K in (512, 2048, 4096):
        terms = [1.0] + [d] * (K - 1)
        exact = 1.0 + (K - 1) * d               # exact in binary64 (few significant bits)
        err = abs(_f32_recursive_sum(terms) - exact)
        assert err == pytest.approx((K - 1) * d, rel=1e-12)
        bound = oracle.error_bound(K, np.array([exact]), slack=1.0)[0]
        assert err <= bound
        assert err >= 0.98 * bound, (K, err, bound)


def test_error_bound_holds_for_random_bf16_products():
    """Validity: binary32 recursive sums of random bf16 x bf16 products stay
    within gamma_K * sum|a b| of the correctly rounded exact sum (math.fsum)."""
    import math
    rng = np.random.default_rng(21)
    for K in (1, 7, 100, 1000, 3000):
        for _ in range(5):
            a = bf16_bits_to_f32(bits(rng.uniform(-1, 1, size=K))).astype(np.float64)
            b = bf16_bits_to_f32(bits(rng.normal(0, 1, size=K))).astype(np.float64)
            prods = a * b                       # exact: at most 16 significant bits
            exact = math.fsum(prods)
            err = abs(_f32_recursive_sum(prods) - exact)
            bound = oracle.error_bound(K, np.array([float(np.sum(np.abs(prods)))]), slack=1.0)[0]
            assert err <= bound, (K, err, bound)
    assert oracle.error_bound(0, np.array([1.0]))[0] == 0.0
