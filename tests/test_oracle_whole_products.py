"""Pins of the oracle's whole-product functions (gemm_by_rows,
mx_gemm_by_rows, blockwise_gemm_by_rows), which evaluate every output of a
full-size workload with numpy's fp64 matrix product over decoded, block-scaled
operands, in row blocks. Each is checked against an independent form of the
same definition: the C loops of fp8_oracle.c (dense and MX), the per-K-block
sums of blockwise_gemm, and exact integer arithmetic. Shapes give several row
blocks with a ragged last one, so a dropped or shifted block fails. CPU only."""
import numpy as np
import pytest


def collect(gen, m, n):
    y = np.full((m, n), np.nan)
    bound = np.full((m, n), np.nan)
    seen = np.zeros(m, np.int64)
    for r0, r1, yb, bb in gen:
        assert yb.shape == (r1 - r0, n)
        y[r0:r1], bound[r0:r1] = yb, bb
        seen[r0:r1] += 1
    assert (seen == 1).all(), "every row exactly once"
    return y, bound


def rand_codes(rng, shape, fmt, orc):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[~np.isfinite(orc.decode(fmt, c))] = 0x21
    return c


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (2, 3)])
@pytest.mark.parametrize("vec", [(True, True), (False, True), (True, False)])
def test_gemm_by_rows_equals_c_loops(orc, fa, fb, vec):
    """Random codes of all four encodings (NaN codes excluded), row/tensor
    scales: equal to the C oracle's loops up to fp64 summation order."""
    rng = np.random.default_rng(fa * 10 + fb + 100 * vec[0] + 200 * vec[1])
    m, n, k = 45, 37, 320
    a = rand_codes(rng, (m, k), fa, orc)
    b = rand_codes(rng, (n, k), fb, orc)
    sa = rng.uniform(0.25, 4, m if vec[0] else 1).astype(np.float32)
    sb = rng.uniform(0.25, 4, n if vec[1] else 1).astype(np.float32)
    want_y, want_b = orc.gemm(a, fa, b, fb, sa, sb)
    got_y, got_b = collect(orc.gemm_by_rows(a, fa, b, fb, sa, sb, chunk=16), m, n)
    tol = 1e-13 * want_b + 1e-300
    assert np.all(np.abs(got_y - want_y) <= tol)
    assert np.all(np.abs(got_b - want_b) <= tol)


def test_gemm_by_rows_integer_exact_and_nan(orc):
    """Small integers with unit scales: exactly the int64 matmul; a NaN code
    makes exactly its row's outputs NaN."""
    from test_oracle_gemm import codes_for_small_ints
    rng = np.random.default_rng(7)
    m, n, k = 33, 19, 128
    ia = rng.integers(-7, 8, (m, k))
    ib = rng.integers(-7, 8, (n, k))
    a = codes_for_small_ints(orc, 0, ia)
    b = codes_for_small_ints(orc, 1, ib)
    y, bound = collect(orc.gemm_by_rows(a, 0, b, 1, np.float32(1), np.float32(1), chunk=8), m, n)
    assert np.array_equal(y, (ia @ ib.T).astype(np.float64))
    assert np.array_equal(bound, (np.abs(ia) @ np.abs(ib).T).astype(np.float64))
    a[5, 17] = 0x7F
    y, _ = collect(orc.gemm_by_rows(a, 0, b, 1, np.float32(1), np.float32(1), chunk=8), m, n)
    assert np.isnan(y[5]).all() and not np.isnan(np.delete(y, 5, axis=0)).any()


@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0)])
def test_mx_gemm_by_rows_equals_c_loops(orc, fa, fb):
    """Random codes and random E8M0 block scales over a wide range, incl. a NaN
    scale byte: equal to the C oracle's MX loops."""
    rng = np.random.default_rng(11 + fa)
    m, n, k = 40, 24, 256
    a = rand_codes(rng, (m, k), fa, orc)
    b = rand_codes(rng, (n, k), fb, orc)
    sa = rng.integers(90, 160, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(90, 160, (n, k // 32)).astype(np.uint8)
    sa[3, 2] = 255
    want_y, want_b = orc.mx_gemm(a, fa, sa, b, fb, sb)
    got_y, got_b = collect(orc.mx_gemm_by_rows(a, fa, sa, b, fb, sb, chunk=16), m, n)
    both_nan = np.isnan(want_y) & np.isnan(got_y)
    assert np.array_equal(np.isnan(want_y), np.isnan(got_y)) and np.isnan(got_y[3]).all()
    fin = ~both_nan
    assert np.all(np.abs(got_y - want_y)[fin] <= 1e-13 * want_b[fin])
    assert np.all(np.abs(got_b - want_b)[fin] <= 1e-13 * want_b[fin])


def test_blockwise_gemm_by_rows_equals_block_sums(orc):
    """Against blockwise_gemm (explicit per-128-block sums times both block
    factors), with a ragged last weight tile (n = 200) and several row blocks."""
    rng = np.random.default_rng(21)
    m, n, k = 70, 200, 384
    a = rand_codes(rng, (m, k), 0, orc)
    b = rand_codes(rng, (n, k), 0, orc)
    ea = rng.integers(100, 150, (m, k // 128)).astype(np.uint8)
    eb = rng.integers(100, 150, ((n + 127) // 128, k // 128)).astype(np.uint8)
    want_y, want_b = orc.blockwise_gemm(a, 0, ea, b, 0, eb)
    got_y, got_b = collect(orc.blockwise_gemm_by_rows(a, 0, ea, b, 0, eb, chunk=32), m, n)
    assert np.all(np.abs(got_y - want_y) <= 1e-13 * want_b)
    assert np.all(np.abs(got_b - want_b) <= 1e-13 * want_b)
