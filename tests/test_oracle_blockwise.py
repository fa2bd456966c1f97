"""Pins of the oracle's blockwise recipe (1 x 128 activation blocks, 128 x 128
weight tiles, power-of-two scales below fmax / amax): blocks worked by hand,
including one where the power-of-two rule and MX's rule part ways, special
blocks, a tile shared by its rows, invariants of random blocks, and the
product against exact integer sums. CPU only."""
import numpy as np
import pytest

import workloads
from test_oracle_gemm import codes_for_small_ints


def row_block(vals, n=128):
    r = np.zeros(n, np.float32)
    r[:len(vals)] = vals
    return workloads.bf16_bits(r[None, :])


def test_hand_blocks(orc):
    """amax 3: 448 / 3 = 149.3 -> s = 128 (E8M0 of 1/128 = 120); 3, 1, -0.5
    -> 384, 128, -64 -> 0x7C, 0x70, 0xE8 (here the same as MX). amax 460:
    448 / 460 < 1 -> s = 1/2 (byte 128), 460 -> 230 -> 224 = 0x76, where MX
    keeps scale 1 and saturates to 448."""
    q, e = orc.blockwise_quantize_act(row_block([3.0, 1.0, -0.5]), 0)
    assert e[0, 0] == 120 and list(q[0, :4]) == [0x7C, 0x70, 0xE8, 0x00]
    q, e = orc.blockwise_quantize_act(row_block([460.0]), 0)
    assert e[0, 0] == 128 and q[0, 0] == 0x76
    qm, sm = orc.mx_quantize_row(row_block([460.0], 32), 0)
    assert sm[0, 0] == 127 and qm[0, 0] == 0x7E


def test_special_blocks(orc):
    """Zero block: s = 1 (byte 127), zero codes; NaN: s = 1, NaN code; Inf:
    s = 1, saturated; a tiny amax: s capped at FLT_MAX -> 2^127 (byte 0)."""
    q, e = orc.blockwise_quantize_act(row_block([]), 0)
    assert e[0, 0] == 127 and not q.any()
    x = row_block([1.0, 2.0])
    x[0, 1] = 0x7FC0
    q, e = orc.blockwise_quantize_act(x, 1)
    assert e[0, 0] == 127 and q[0, 1] == 0x7F and q[0, 0] == 0x3C
    q, e = orc.blockwise_quantize_act(row_block([np.inf, 1.0]), 0)
    assert e[0, 0] == 127 and q[0, 0] == 0x7E
    q, e = orc.blockwise_quantize_act(row_block([2.0 ** -133]), 0)
    assert e[0, 0] == 0


def test_weight_tile_shared_by_its_rows(orc):
    """130 rows: tile 0 (rows 0-127) holds one element of 96 (s = 4: 448/96 =
    4.67), so all its rows take byte 125; tile 1 (rows 128-129) has amax 1
    (s = 256, byte 119)."""
    w = np.full((130, 256), 0.5, np.float32)
    w[40, 7] = 96.0
    w[128:, :] = 1.0
    q, e = orc.blockwise_quantize_weight(workloads.bf16_bits(w), 0)
    assert e.shape == (2, 2)
    assert e[0, 0] == 125 and e[1, 0] == 119
    dec = orc.decode(0, q)
    assert dec[40, 7] == 384.0 and dec[3, 3] == 2.0 and dec[129, 200] == 256.0


@pytest.mark.parametrize("fmt", [0, 1])
def test_random_block_invariants(orc, fmt):
    """Every block: s is a power of two with fmax / 2 < amax s <= fmax; every
    code is within half a quantum of x s (no saturation)."""
    fmax, _, mbits, bias = orc.fmt_info(fmt)
    rng = np.random.default_rng(11)
    xf = rng.standard_normal((12, 512)).astype(np.float32)
    xf *= np.exp2(rng.integers(-20, 20, (12, 4))).repeat(128, axis=1).astype(np.float32)
    x = workloads.bf16_bits(xf)
    xv = workloads.bf16_to_f32(x).astype(np.float64)
    q, e = orc.blockwise_quantize_act(x, fmt)
    dec = orc.decode(fmt, q)
    for r in range(12):
        for b in range(4):
            blk = xv[r, 128 * b:128 * b + 128]
            s = 2.0 ** (127 - int(e[r, b]))
            am = np.abs(blk).max()
            assert fmax / 2 < am * s <= fmax
            t = blk * s
            ex = np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 1e-300))), 1 - bias)
            assert np.all(np.abs(dec[r, 128 * b:128 * b + 128] - t) <= 0.5 * np.exp2(ex - mbits))


def test_blockwise_gemm_exact_integers(orc):
    """Small-integer codes with random block bytes: every 128-block's dot
    product is an integer, the power-of-two factors exact, the fp64 sums exact."""
    rng = np.random.default_rng(12)
    m, n, K = 5, 260, 256
    ia = rng.integers(-6, 7, (m, K))
    ib = rng.integers(-6, 7, (n, K))
    a = codes_for_small_ints(orc, 0, ia)
    b = codes_for_small_ints(orc, 1, ib)
    ea = rng.integers(115, 140, (m, K // 128)).astype(np.uint8)
    eb = rng.integers(115, 140, (3, K // 128)).astype(np.uint8)
    y, bound = orc.blockwise_gemm(a, 0, ea, b, 1, eb)
    for i in range(m):
        for j in range(0, n, 37):
            want = mag = 0.0
            for kb in range(K // 128):
                sl = slice(128 * kb, 128 * kb + 128)
                x = 2.0 ** (int(ea[i, kb]) - 127 + int(eb[j // 128, kb]) - 127)
                want += x * float(np.dot(ia[i, sl], ib[j, sl]))
                mag += x * float(np.abs(ia[i, sl] * ib[j, sl]).sum())
            assert y[i, j] == want and bound[i, j] == mag


def test_blockwise_entries_match_the_whole_product(orc):
    """The sampled-entry form against the whole product (to fp64 rounding)."""
    rng = np.random.default_rng(13)
    m, n, K = 9, 300, 384
    a = rng.integers(0, 0x7E, (m, K)).astype(np.uint8)
    b = rng.integers(0x80, 0xFB, (n, K)).astype(np.uint8)
    ea = rng.integers(110, 140, (m, 3)).astype(np.uint8)
    eb = rng.integers(110, 140, (3, 3)).astype(np.uint8)
    y, bound = orc.blockwise_gemm(a, 0, ea, b, 1, eb)
    ii, jj = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    ye, be = orc.blockwise_gemm_entries(a, 0, ea, b, 1, eb, ii.ravel(), jj.ravel())
    assert np.allclose(ye.reshape(m, n), y, rtol=1e-12, atol=0)
    assert np.allclose(be.reshape(m, n), bound, rtol=1e-12, atol=0)
