"""Pins of the oracle's MoE-layer forward pieces: routing worked by hand and
against a stable sort, the permuted quantization worked by hand, SwiGLU's
closed forms and the quantization of its fp32 rows (hand values and
invariants), and the weighted combine against one-hot weights and a
brute-force loop. CPU only."""
import numpy as np

import workloads


def test_route_hand_example(orc):
    """Entries (token, slot) -> expert: (0,0)->1 (0,1)->3 (1,0)->1 (1,1)->0
    (2,0)->3 (2,1)->1. Counts 1, 3, 0, 2; expert 1's rows keep token order."""
    offsets, dest = orc.moe_route(np.array([[1, 3], [1, 0], [3, 1]]), 4)
    assert list(offsets) == [0, 1, 4, 4, 6]
    assert dest.tolist() == [[1, 4], [2, 0], [5, 3]]


def test_route_drops_out_of_range_indices(orc):
    """Indices -1 and E drop their entries: dest -1, the rest as if absent."""
    offsets, dest = orc.moe_route(np.array([[1, -1], [4, 0], [1, 1]]), 4)
    assert list(offsets) == [0, 1, 4, 4, 4]
    assert dest.tolist() == [[1, -1], [-1, 0], [2, 3]]


def test_route_matches_a_stable_sort(orc):
    rng = np.random.default_rng(3)
    T, k, E = 300, 6, 20
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    idx[:40] = idx[0]                                   # repeated rows
    offsets, dest = orc.moe_route(idx, E)
    order = np.argsort(idx.reshape(-1), kind="stable")  # entry of each sorted row
    want = np.empty(T * k, np.int64)
    want[order] = np.arange(T * k)
    assert np.array_equal(dest.reshape(-1), want)
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(idx.reshape(-1), minlength=E))]))


def test_permute_quantize_hand_example(orc):
    """Token 0 = [1, -2] (amax 2, e4m3 scale 224: 224 -> 0x76, -448 -> 0xFE),
    token 1 = [0.5, 0.25] (amax 0.5, scale 896: 448 -> 0x7E, 224 -> 0x76), each
    written to both of its rows."""
    x = workloads.bf16_bits(np.float32([[1.0, -2.0], [0.5, 0.25]]))
    dest = np.array([[2, 0], [1, 3]])
    q, si = orc.moe_permute_quantize_row(x, dest, 0)
    assert q.tolist() == [[0x76, 0xFE], [0x7E, 0x76], [0x76, 0xFE], [0x7E, 0x76]]
    assert np.array_equal(si, np.float32([1 / 224, 1 / 896, 1 / 224, 1 / 896]))


def test_silu_closed_forms(orc):
    x = np.random.default_rng(4).standard_normal(1000) * 8
    assert np.allclose(orc.silu(x) - orc.silu(-x), x, rtol=1e-14, atol=1e-14)   # sigmoid(x) + sigmoid(-x) = 1
    assert orc.silu(0.0) == 0.0
    assert orc.silu(60.0) == 60.0                       # sigmoid(60) = 1 - 9e-27 rounds to 1
    assert abs(orc.silu(-60.0)) < 1e-24


def test_swiglu_quantize_hand_rows(orc):
    """gate 60 makes silu exact to fp64 (60), so a = 60 * up: [90, -15] with
    up = [1.5, -0.25]: amax 90, e4m3 s = fl32(448/90); 90 s -> 448 (0x7E) and
    -15 s = -74.67 -> -72 (0xE9). A zero gate row gives a = [0, -0] (0 * -7):
    scale 1, codes 0x00 and 0x80 (OCP keeps the sign of zero)."""
    h = workloads.bf16_bits(np.float32([[60.0, 60.0, 1.5, -0.25], [0.0, 0.0, 3.0, -7.0]]))
    q, si, a = orc.swiglu_quantize_row(h, 0)
    assert a.tolist() == [[90.0, -15.0], [0.0, 0.0]]
    assert q.tolist() == [[0x7E, 0xE9], [0x00, 0x80]]
    assert si[0] == orc.reciprocal(np.float32(448) / np.float32(90)) and si[1] == 1.0


def test_swiglu_quantize_invariants(orc):
    """Random rows: a is fl32(silu(g) u); the largest code decodes to fmax; every
    code times scale_inv is within half a quantum of a (x 1 + 1e-5 for the
    x / scale_inv stand-in of x * s)."""
    rng = np.random.default_rng(5)
    rows, inter = 30, 96
    hf = (rng.standard_normal((rows, 2 * inter)) * np.exp2(rng.integers(-4, 5, (rows, 1)))).astype(np.float32)
    h = workloads.bf16_bits(hf)
    hv = workloads.bf16_to_f32(h).astype(np.float64)
    for fmt in (0, 1):
        fmax, _, mbits, bias = orc.fmt_info(fmt)
        q, si, a = orc.swiglu_quantize_row(h, fmt)
        g, u = hv[:, :inter], hv[:, inter:]
        assert np.array_equal(a, (g / (1 + np.exp(-g)) * u).astype(np.float32))
        dec = orc.decode(fmt, q)
        assert np.all(np.abs(dec).max(axis=1) == fmax)
        scaled = a.astype(np.float64) / si[:, None].astype(np.float64)
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(scaled), 1e-300))), 1 - bias)
        assert np.all(np.abs(dec - scaled) <= 0.5 * np.exp2(e - mbits) * (1 + 1e-5))


def test_unpermute_combine(orc):
    rng = np.random.default_rng(6)
    T, k, H = 7, 3, 40
    idx = np.stack([rng.choice(5, k, replace=False) for _ in range(T)])
    _, dest = orc.moe_route(idx, 5)
    y = workloads.bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    yv = workloads.bf16_to_f32(y).astype(np.float64)
    for j in range(k):                                  # one-hot weights pick one slot's row back
        w = np.zeros((T, k))
        w[:, j] = 1.0
        out, _ = orc.moe_unpermute_combine(y, dest, w)
        assert np.array_equal(out, yv[dest[:, j]])
    w = rng.uniform(0, 1, (T, k))
    out, mag = orc.moe_unpermute_combine(y, dest, w)
    for t in range(T):                                  # brute force
        for c in range(H):
            terms = [w[t, j] * yv[dest[t, j], c] for j in range(k)]
            assert abs(out[t, c] - sum(terms)) <= 1e-15 * sum(abs(v) for v in terms)
            assert abs(mag[t, c] - sum(abs(v) for v in terms)) <= 1e-15 * mag[t, c]


def test_bf16_round_ties_and_exactness(orc):
    """Nearest even at ties (1 + 2^-8 -> 1, 1 + 3 * 2^-8 -> 1 + 2^-6); just past
    a tie rounds away even where fp32 would land on the tie; exact values stay."""
    one = 1.0 + 2.0 ** -8
    x = np.array([1.0, one, 1.0 + 3 * 2.0 ** -8, one + 2.0 ** -40, -one - 2.0 ** -40, 3.0, np.nan])
    r = orc.bf16_round(x)
    assert r.tolist()[:6] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBF81, 0x4040]
    assert r[6] == 0x7FC0
