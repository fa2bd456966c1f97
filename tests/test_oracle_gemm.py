"""Pins of the oracle's scaled GEMM and grouped GEMM: integer-exact products,
identity operands, exact rational arithmetic on tiny shapes, an independent
numpy matmul, and the grouped product as per-group dense products. CPU only."""
from fractions import Fraction

import numpy as np
import pytest


def codes_for_small_ints(orc, fmt, ints):
    """FP8 codes whose values are the given small integers (exactly representable)."""
    table = orc.decode_table(fmt)
    lut = {}
    for c in range(256):
        v = table[c]
        if np.isfinite(v) and v == int(v) and int(v) not in lut:
            lut[int(v)] = c
    return np.vectorize(lambda v: lut[int(v)])(ints).astype(np.uint8)


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_integer_codes_equal_int_matmul(orc, fa, fb):
    """Small integer values with unit scales: the result is an integer matmul."""
    rng = np.random.default_rng(0)
    m, n, k = 19, 23, 96
    ia = rng.integers(-6, 7, (m, k))
    ib = rng.integers(-6, 7, (n, k))
    a = codes_for_small_ints(orc, fa, ia)
    b = codes_for_small_ints(orc, fb, ib)
    y, bound = orc.gemm(a, fa, b, fb, np.float32(1.0), np.float32(1.0))
    assert np.array_equal(y, (ia @ ib.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(ia) @ np.abs(ib).T).astype(np.float64))


def test_identity_operand_returns_dequantized_a(orc):
    rng = np.random.default_rng(1)
    m, k = 17, 64
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x11      # no NaN codes
    one = codes_for_small_ints(orc, 0, np.array([1]))[0]
    b = np.zeros((k, k), np.uint8)
    b[np.arange(k), np.arange(k)] = one
    sa = np.exp2(rng.integers(-3, 4, m)).astype(np.float32)     # powers of two: exact
    y, _ = orc.gemm(a, 0, b, 0, sa, np.float32(0.25))
    assert np.array_equal(y, orc.decode(0, a) * sa[:, None].astype(np.float64) * 0.25)


def test_tiny_shapes_exact_rational(orc):
    """K <= 64 of e4m3/e5m2 values: every product and partial sum is exact in fp64,
    so the fp64 sum equals exact rational arithmetic (before the scales)."""
    rng = np.random.default_rng(2)
    for fa, fb in [(0, 0), (1, 0)]:
        m, n, k = 3, 4, 64
        a = rng.integers(0, 256, (m, k)).astype(np.uint8)
        b = rng.integers(0, 256, (n, k)).astype(np.uint8)
        for arr, f in ((a, fa), (b, fb)):
            t = orc.decode(f, arr)
            arr[~np.isfinite(t)] = 0x22
        y, bound = orc.gemm(a, fa, b, fb, np.float32(1.0), np.float32(1.0))
        ta, tb = orc.decode_table(fa), orc.decode_table(fb)
        for i in range(m):
            for j in range(n):
                exact = sum(Fraction(ta[a[i, kk]]) * Fraction(tb[b[j, kk]]) for kk in range(k))
                absum = sum(abs(Fraction(ta[a[i, kk]]) * Fraction(tb[b[j, kk]])) for kk in range(k))
                assert Fraction(y[i, j]) == exact
                assert Fraction(bound[i, j]) == absum


def test_matches_numpy_matmul_nonsquare(orc):
    """Against numpy's matmul of the decoded operands (A B^T, non-square so a
    transposed operand or swapped scale cannot pass), with row and column scales."""
    rng = np.random.default_rng(3)
    m, n, k = 29, 41, 160
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    b = rng.integers(0, 256, (n, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    b[(b & 0x7C) == 0x7C] = 0x31
    sa = rng.uniform(0.5, 2, m).astype(np.float32)
    sb = rng.uniform(0.5, 2, n).astype(np.float32)
    y, bound = orc.gemm(a, 0, b, 1, sa, sb)
    da, db = orc.decode(0, a), orc.decode(1, b)
    ref = (da @ db.T) * sa[:, None].astype(np.float64) * sb[None, :].astype(np.float64)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-300)
    assert np.allclose(bound, (np.abs(da) @ np.abs(db).T) * np.abs(sa[:, None] * sb[None, :].astype(np.float64)),
                       rtol=1e-12)
    ii = rng.integers(0, m, 50)
    jj = rng.integers(0, n, 50)
    ye, be = orc.gemm_entries(a, 0, b, 1, sa, sb, ii, jj)
    assert np.allclose(ye, y[ii, jj], rtol=1e-13) and np.allclose(be, bound[ii, jj], rtol=1e-13)


def test_acceptance_rule(orc):
    y = np.array([1.0, 100.0, -3.0, np.nan])
    bound = np.array([1.0, 100.0, 3.0, np.nan])
    gpu = np.array([1.0 + 2.0 ** -8 + 0.9e-3, 100.5, -3.0 - 1e-2, np.nan])
    ok = orc.gemm_within_bound(gpu, y, bound)
    assert ok.tolist() == [True, False, True, True]
    assert not orc.gemm_within_bound(np.array([1.01]), np.array([1.0]), np.array([1.0]))[0]


@pytest.mark.parametrize("sizes", [[0, 1, 17, 255, 257], [64], [0, 0, 40, 0]])
def test_grouped_equals_per_group_dense(orc, sizes):
    rng = np.random.default_rng(4)
    g, n, k = len(sizes), 24, 48
    offsets = np.zeros(g + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    a = rng.integers(0, 0x70, (total, k)).astype(np.uint8)
    b = rng.integers(0, 0x70, (g, n, k)).astype(np.uint8)
    sa = rng.uniform(0.5, 2, total).astype(np.float32)
    sb = rng.uniform(0.5, 2, (g, n)).astype(np.float32)
    y, bound = orc.grouped_gemm(a, 0, b, 0, offsets, sa, sb)
    for gg in range(g):
        lo, hi = offsets[gg], offsets[gg + 1]
        if hi > lo:
            da, db = orc.decode(0, a[lo:hi]), orc.decode(0, b[gg])
            ref = (da @ db.T) * sa[lo:hi, None].astype(np.float64) * sb[gg][None, :].astype(np.float64)
            assert np.allclose(y[lo:hi], ref, rtol=1e-12)
    assert not np.isnan(y).any()
    ii = rng.integers(0, total, 64)
    jj = rng.integers(0, n, 64)
    ye, _ = orc.grouped_gemm_entries(a, 0, b, 0, offsets, sa, sb, ii, jj)
    assert np.allclose(ye, y[ii, jj], rtol=1e-13)
    if g == 1:
        yd, _ = orc.gemm(a, 0, b[0], 0, sa, sb[0])
        assert np.array_equal(yd, y)
