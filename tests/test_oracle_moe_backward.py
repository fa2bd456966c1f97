"""Pins of the oracle's MoE-backward pieces (grouped colwise quantization into
the padded transposed layout, and the ragged-K grouped product of the weight
gradient): a layout and scale example worked by hand, invariants of the
per-group scales, and a brute-force token loop over the untransposed codes.
CPU only."""
import numpy as np

import workloads
from test_oracle_gemm import codes_for_small_ints


def bits(vals):
    return workloads.bf16_bits(np.asarray(vals, np.float32))


def test_grouped_quantize_col_hand_example(orc):
    """Groups of 2, 0 and 3 rows, two columns, alignment 4: every scale is
    fmax / amax with an exact quotient (448 / 1, 448 / 4, 448 / 7, 448 / 2) and
    every scaled value is an e4m3 number, so the codes follow by hand:
    448 -> 0x7E, 224 -> 0x76, 112 -> 0x6E, 0 -> 0x00 (sign bit 0x80)."""
    x = bits([[1.0, -2.0],
              [0.5, 4.0],
              [7.0, 0.0],
              [-3.5, 1.0],
              [1.75, -2.0]])
    offsets = np.array([0, 2, 2, 5], np.int64)
    qt, si, am = orc.grouped_quantize_col(x, 0, offsets, align=4)
    # P = [0, 4, 4, 8]: group 0 at columns 0-1 (2-3 zero), group 2 at 4-6 (7 zero)
    want = np.array([[0x7E, 0x76, 0, 0, 0x7E, 0xF6, 0x6E, 0],
                     [0xF6, 0x7E, 0, 0, 0x00, 0x76, 0xFE, 0]], np.uint8)
    assert np.array_equal(qt, want)
    assert np.array_equal(am, np.float32([[1, 4], [0, 0], [7, 2]]))
    assert np.array_equal(si, np.float32([[1 / 448, 1 / 112], [1, 1], [1 / 64, 1 / 224]]))


def test_grouped_quantize_col_invariants(orc):
    """Random groups (some empty): in each group and column with a nonzero amax
    the largest code magnitude decodes to fmax (the scale maps amax to fmax),
    every decoded code times scale_inv is within half a quantum of the input,
    and the padding columns hold zero codes."""
    rng = np.random.default_rng(5)
    sizes = [3, 0, 17, 1, 0, 40]
    offsets = np.zeros(len(sizes) + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    cols = 24
    xf = rng.standard_normal((int(offsets[-1]), cols)).astype(np.float32)
    xf *= np.exp2(rng.integers(-6, 7, (1, cols))).astype(np.float32)
    x = workloads.bf16_bits(xf)
    xv = workloads.bf16_to_f32(x).astype(np.float64)
    for fmt in (0, 1):
        fmax, _, mbits, bias = orc.fmt_info(fmt)
        qt, si, am = orc.grouped_quantize_col(x, fmt, offsets, align=16)
        P = orc.padded_offsets(offsets, 16)
        assert qt.shape == (cols, int(P[-1]))
        dec = orc.decode(fmt, qt)
        for g in range(len(sizes)):
            lo, hi = int(offsets[g]), int(offsets[g + 1])
            seg = dec[:, P[g]:P[g] + (hi - lo)]
            pad = qt[:, P[g] + (hi - lo):P[g + 1]]
            assert not pad.any()
            if hi == lo:
                assert np.all(si[g] == 1) and np.all(am[g] == 0)
                continue
            assert np.array_equal(am[g], np.abs(xv[lo:hi]).max(axis=0).astype(np.float32))
            assert np.all(np.abs(seg).max(axis=1) == fmax)
            # cast error: half a quantum of the scaled value at most (x / scale_inv
            # stands for x * s, which it matches to a few fp32 ulps: hence 1e-5)
            scaled = xv[lo:hi].T / si[g][:, None].astype(np.float64)
            err = np.abs(seg - scaled)
            # quantum of the binade (subnormal binade below the smallest normal exponent)
            e = np.maximum(np.floor(np.log2(np.maximum(np.abs(scaled), 1e-300))), 1 - bias)
            assert np.all(err <= 0.5 * np.exp2(e - mbits) * (1 + 1e-5))


def test_grouped_gemm_ragged_k_brute_force(orc):
    """The weight-gradient product against a loop over tokens on the
    untransposed codes: D_g[i, j] = sum over the group's tokens t of
    dy[t, i] * x[t, j], times the group's scales. Small integer values and
    power-of-two scales keep every fp64 sum exact; empty groups give zeros."""
    rng = np.random.default_rng(6)
    sizes = [3, 0, 5, 1]
    offsets = np.zeros(len(sizes) + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    T, m, n, align = int(offsets[-1]), 4, 6, 8
    idy = rng.integers(-6, 7, (T, m))
    ix = rng.integers(-6, 7, (T, n))
    dyq = codes_for_small_ints(orc, 1, idy)       # e5m2 gradient codes
    xq = codes_for_small_ints(orc, 0, ix)         # e4m3 activation codes
    P = orc.padded_offsets(offsets, align)
    a_t = np.zeros((m, int(P[-1])), np.uint8)
    b_t = np.zeros((n, int(P[-1])), np.uint8)
    for g in range(len(sizes)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        a_t[:, P[g]:P[g] + hi - lo] = dyq[lo:hi].T
        b_t[:, P[g]:P[g] + hi - lo] = xq[lo:hi].T
    sa = np.exp2(rng.integers(-3, 4, (len(sizes), m))).astype(np.float32)
    sb = np.exp2(rng.integers(-3, 4, (len(sizes), n))).astype(np.float32)
    d, bound = orc.grouped_gemm_ragged_k(a_t, 1, b_t, 0, offsets, align, sa, sb)
    for g in range(len(sizes)):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        for i in range(m):
            for j in range(n):
                acc = 0
                mag = 0
                for t in range(lo, hi):
                    acc += int(idy[t, i]) * int(ix[t, j])
                    mag += abs(int(idy[t, i]) * int(ix[t, j]))
                assert d[g, i, j] == acc * float(sa[g, i]) * float(sb[g, j])
                assert bound[g, i, j] == mag * float(sa[g, i]) * float(sb[g, j])
    assert not d[1].any()
