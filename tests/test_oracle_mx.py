"""Pins of the oracle's MX (block-32, E8M0-scaled) quantizer and product: blocks
worked by hand in both element formats, the saturating top binade, special
blocks (zeros, NaN, Inf, tiny), invariants of random blocks, and the product
against exact integer arithmetic with power-of-two block scales. CPU only."""
import numpy as np
import pytest

import workloads
from test_oracle_gemm import codes_for_small_ints


def block(vals):
    row = np.zeros(32, np.float32)
    row[:len(vals)] = vals
    return workloads.bf16_bits(row[None, :])


def test_hand_blocks(orc):
    """amax 3 -> floor(log2 3) = 1: e4m3 e = 1 - 8 = -7 (E8M0 120), elements
    x * 128: 384 -> 0x7C, 128 -> 0x70, -64 -> 0xE8; e5m2 e = 1 - 15 = -14
    (E8M0 113), elements x * 2^14: 49152 -> 0x7A, 16384 -> 0x74, -8192 -> 0xF0."""
    x = block([3.0, 1.0, -0.5, 0.0])
    q, s = orc.mx_quantize_row(x, 0)
    assert s[0, 0] == 120 and list(q[0, :4]) == [0x7C, 0x70, 0xE8, 0x00]
    q, s = orc.mx_quantize_row(x, 1)
    assert s[0, 0] == 113 and list(q[0, :4]) == [0x7A, 0x74, 0xF0, 0x00]


def test_top_binade_saturates(orc):
    """amax 3.75 keeps e = -7, so 3.75 * 128 = 480 > 448 saturates to 0x7E;
    2.5 * 128 = 320 is exact (0x7A)."""
    q, s = orc.mx_quantize_row(block([3.75, 2.5]), 0)
    assert s[0, 0] == 120 and q[0, 0] == 0x7E and q[0, 1] == 0x7A


def test_special_blocks(orc):
    zeros = block([])
    q, s = orc.mx_quantize_row(zeros, 0)
    assert s[0, 0] == 0 and not q.any()                   # e = -127
    x = block([1.0, np.inf, -2.0])
    q, s = orc.mx_quantize_row(x, 0)
    assert s[0, 0] == 0xFF                                # non-finite block: NaN scale
    assert q[0, 0] == 0x38 and q[0, 1] == 0x7E and q[0, 2] == 0xC0   # cast with scale 1, Inf saturates
    xb = block([1.0])
    xb[0, 1] = 0xFFC0                                     # -NaN
    q, s = orc.mx_quantize_row(xb, 1)
    assert s[0, 0] == 0xFF and q[0, 1] == 0xFF
    tiny = block([2.0 ** -130])                           # bf16 subnormal: e clamps to -127
    q, s = orc.mx_quantize_row(tiny, 0)
    assert s[0, 0] == 0 and orc.decode(0, q[0, :1])[0] == 2.0 ** -3


def test_scale_value(orc):
    assert orc.mx_scale_value(127) == 1.0 and orc.mx_scale_value(0) == 2.0 ** -127
    assert np.isnan(orc.mx_scale_value(255))
    assert orc.mx_scale(0, 448.0) == 127 and orc.mx_scale(0, 256.0) == 127 and orc.mx_scale(0, 255.0) == 126
    assert orc.mx_scale(1, 1.0) == 112 and orc.mx_scale(1, 65536.0) == 128


@pytest.mark.parametrize("fmt", [0, 1])
def test_random_block_invariants(orc, fmt):
    """Every block: E8M0 = floor(log2 amax) - emax + 127; the largest magnitude
    code decodes into [2^emax, fmax] (the top binade, saturated); every element
    is within half a quantum of x / X unless it saturated at fmax."""
    fmax, _, mbits, bias = orc.fmt_info(fmt)
    emax = 8 if fmt == 0 else 15
    rng = np.random.default_rng(1)
    xf = rng.standard_normal((40, 256)).astype(np.float32)
    xf *= np.exp2(rng.integers(-20, 20, (40, 8))).repeat(32, axis=1).astype(np.float32)
    x = workloads.bf16_bits(xf)
    xv = workloads.bf16_to_f32(x).astype(np.float64)
    q, s = orc.mx_quantize_row(x, fmt)
    dec = orc.decode(fmt, q)
    for r in range(40):
        for b in range(8):
            blk = xv[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            e = int(np.floor(np.log2(amax))) - emax
            assert s[r, b] == e + 127
            X = 2.0 ** e
            d = dec[r, 32 * b:32 * b + 32]
            assert 2.0 ** emax <= np.abs(d).max() <= fmax
            t = blk / X
            ex = np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 1e-300))), 1 - bias)
            ok = (np.abs(d - t) <= 0.5 * np.exp2(ex - mbits)) | ((np.abs(d) == fmax) & (np.abs(t) > fmax))
            assert ok.all()


def test_mx_gemm_exact_integers(orc):
    """Small-integer elements with random power-of-two block scales: every
    block's dot product is an integer and every fp64 sum is exact."""
    rng = np.random.default_rng(2)
    m, n, k = 7, 9, 128
    ia = rng.integers(-6, 7, (m, k))
    ib = rng.integers(-6, 7, (n, k))
    a = codes_for_small_ints(orc, 0, ia)
    b = codes_for_small_ints(orc, 1, ib)
    sa = rng.integers(120, 135, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(120, 135, (n, k // 32)).astype(np.uint8)
    y, bound = orc.mx_gemm(a, 0, sa, b, 1, sb)
    for i in range(m):
        for j in range(n):
            want = 0.0
            mag = 0.0
            for blk in range(k // 32):
                sl = slice(32 * blk, 32 * blk + 32)
                x = 2.0 ** (int(sa[i, blk]) - 127 + int(sb[j, blk]) - 127)
                want += x * float(np.dot(ia[i, sl], ib[j, sl]))
                mag += x * float(np.abs(ia[i, sl] * ib[j, sl]).sum())
            assert y[i, j] == want and bound[i, j] == mag


def test_mx_entries_match_the_whole_product(orc):
    """The sampled-entry form (used on full-size outputs) against the whole
    product on random codes and scales, dense and grouped (a NaN scale byte
    included); the two sum in different orders, so to fp64 rounding."""
    rng = np.random.default_rng(7)
    m, n, k = 20, 12, 256
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8)
    b = rng.integers(0x80, 0xFB, (n, k)).astype(np.uint8)
    sa = rng.integers(110, 140, (m, k // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (n, k // 32)).astype(np.uint8)
    sa[3, 2] = 0xFF
    y, bound = orc.mx_gemm(a, 0, sa, b, 1, sb)
    ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    ye, be = orc.mx_gemm_entries(a, 0, sa, b, 1, sb, ii.ravel(), jj.ravel())
    assert np.allclose(ye.reshape(m, n), y, rtol=1e-12, atol=0, equal_nan=True)
    assert np.allclose(be.reshape(m, n), bound, rtol=1e-12, atol=0, equal_nan=True)
    assert np.isnan(ye.reshape(m, n)[3]).all()
    offsets = np.array([0, 5, 5, 20], np.int64)
    bg = rng.integers(0, 0x7E, (3, n, k)).astype(np.uint8)
    sbg = rng.integers(110, 140, (3, n, k // 32)).astype(np.uint8)
    yg, bg_bound = orc.mx_grouped_gemm(a, 0, sa, bg, 0, sbg, offsets)
    ye, be = orc.mx_grouped_gemm_entries(a, 0, sa, bg, 0, sbg, offsets, ii.ravel(), jj.ravel())
    assert np.allclose(ye.reshape(m, n), yg, rtol=1e-12, atol=0, equal_nan=True)
    assert np.allclose(be.reshape(m, n), bg_bound, rtol=1e-12, atol=0, equal_nan=True)
