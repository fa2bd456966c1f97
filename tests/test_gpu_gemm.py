"""GPU parity of the scaled FP8 GEMM and grouped GEMM against the CPU oracle,
through the C ABI. Acceptance per output element:
    |gpu - oracle| <= 1e-3 * sa*sb*sum_k |a_ik b_jk|  +  2^-8 |oracle|   (bf16 out)
(the second term is dropped for fp32 output): the first covers fp32
accumulation over k <= 16384, the second bf16 rounding of the result."""
import numpy as np
import pytest
import torch

import workloads
from helpers import check_full, check_guard, dev_f32, dev_u8, guarded, say

pytestmark = pytest.mark.gpu

PAIRS = [(0, 0), (1, 0), (0, 1), (1, 1)]


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def operands(orc, rows, k, fmt, seed, spread=4):
    """FP8 codes and per-row scale_inv of a random bf16 matrix (quantized by the oracle)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)).astype(np.float32)
    x *= np.exp2(rng.integers(-spread, spread + 1, size=(rows, 1))).astype(np.float32)
    q, si, _ = orc.quantize_row(workloads.bf16_bits(x), fmt)
    return q, si


def gpu_gemm(fp8, a, fa, b, fb, sa, sb, a_mode, b_mode, out_f32=False, ldd=None):
    m, n = a.shape[0], b.shape[0]
    dt = torch.float32 if out_f32 else torch.bfloat16
    d, dbuf, org = guarded(m, n, dt, ld=ldd)
    fp8.fp8_gemm_scaled(dev_u8(a), fa, dev_u8(b), fb, dev_f32(sa), a_mode, dev_f32(sb), b_mode, d)
    torch.cuda.synchronize()
    check_guard(dbuf, org, m, n)
    return d.float().cpu().numpy().astype(np.float64)


def assert_within(orc, got, y, bound, out_bf16, what):
    ok = orc.gemm_within_bound(got, y, bound, out_bf16=out_bf16)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outside the bound; first {i}: gpu {got[i]!r} "
                             f"oracle {y[i]!r} bound {bound[i]!r}")


def test_layout_identity(fp8, orc):
    """B = identity: d must be dequant(A) times the scales, element for element
    (pins the operand and accumulator lane layouts)."""
    rng = np.random.default_rng(0)
    m, k = 96, 64
    a = rng.integers(0, 0x7E, (m, k)).astype(np.uint8)
    a |= (rng.integers(0, 2, (m, k)) << 7).astype(np.uint8)
    one = 0x38                                          # e4m3 1.0
    b = np.zeros((k, k), np.uint8)
    b[np.arange(k), np.arange(k)] = one
    sa = np.exp2(rng.integers(-2, 3, m)).astype(np.float32)
    say("layout identity")
    got = gpu_gemm(fp8, a, 0, b, 0, sa, np.float32([1.0]), 1, 0, out_f32=True)
    want = orc.decode(0, a) * sa[:, None].astype(np.float64)
    assert np.array_equal(got, want)


def test_layout_single_entries(fp8, orc):
    """One nonzero per operand row at distinct k: each output is a single product."""
    m, n, k = 64, 64, 128
    a = np.zeros((m, k), np.uint8)
    b = np.zeros((n, k), np.uint8)
    for i in range(m):
        a[i, (3 * i) % k] = 0x38 + (i % 8)              # 1.0 .. 1.875
    for j in range(n):
        b[j, (3 * j) % k] = 0x40                        # 2.0
    say("layout single entries")
    got = gpu_gemm(fp8, a, 0, b, 0, np.float32([1.0]), np.float32([1.0]), 0, 0, out_f32=True)
    y, bound = orc.gemm(a, 0, b, 0, np.float32(1.0), np.float32(1.0))
    assert np.array_equal(got, y)


SHAPES = [(32, 32, 64), (128, 128, 128), (256, 512, 512), (300, 520, 1040), (1, 1, 16), (17, 33, 48),
          (129, 257, 272), (255, 130, 4096), (0, 5, 16), (5, 0, 16), (4, 4, 0)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("fa,fb", PAIRS)
def test_gemm_parity(fp8, orc, shape, fa, fb):
    m, n, k = shape
    a, sa = operands(orc, m, k, fa, seed=m + 3 * k)
    b, sb = operands(orc, n, k, fb, seed=n + 5 * k + 1)
    y, bound = orc.gemm(a, fa, b, fb, sa, sb)
    say("gemm", shape, fa, fb, "bf16")
    got = gpu_gemm(fp8, a, fa, b, fb, sa, sb, 1, 1, ldd=n + 8)
    assert_within(orc, got, y, bound, True, f"{shape} {fa}x{fb} bf16")
    say("gemm", shape, fa, fb, "f32 tensor scales")
    sa0, sb0 = np.float32([0.37]), np.float32([2.5])
    y0, bound0 = orc.gemm(a, fa, b, fb, sa0, sb0)
    got = gpu_gemm(fp8, a, fa, b, fb, sa0, sb0, 0, 0, out_f32=True)
    assert_within(orc, got, y0, bound0, False, f"{shape} {fa}x{fb} f32")


def test_gemm_mixed_scale_modes(fp8, orc):
    m, n, k = 200, 136, 320
    a, sa = operands(orc, m, k, 0, seed=1)
    b, sb = operands(orc, n, k, 1, seed=2)
    for sa_x, am, sb_x, bm in ((sa, 1, np.float32([3.0]), 0), (np.float32([0.5]), 0, sb, 1)):
        say("gemm mixed modes", am, bm)
        y, bound = orc.gemm(a, 0, b, 1, sa_x, sb_x)
        got = gpu_gemm(fp8, a, 0, b, 1, sa_x, sb_x, am, bm)
        assert_within(orc, got, y, bound, True, f"modes {am}{bm}")


def test_gemm_nan_inf_codes(fp8, orc):
    """NaN codes propagate to their output row/column; e5m2 Inf codes give Inf or NaN as in fp64."""
    m, n, k = 64, 64, 64
    a, sa = operands(orc, m, k, 1, seed=3)
    b, sb = operands(orc, n, k, 1, seed=4)
    a[3, 5] = 0x7F          # e5m2 NaN
    b[7, 9] = 0x7C          # e5m2 +Inf
    say("gemm nan/inf")
    y, bound = orc.gemm(a, 1, b, 1, sa, sb)
    got = gpu_gemm(fp8, a, 1, b, 1, sa, sb, 1, 1, out_f32=True)
    assert np.array_equal(np.isnan(got), np.isnan(y))
    fin = np.isfinite(y)
    assert_within(orc, np.where(fin, got, 0), np.where(fin, y, 0), np.where(fin, bound, 0), False, "finite part")


def test_gemm_deterministic(fp8, orc):
    a, sa = operands(orc, 300, 1040, 0, seed=5)
    b, sb = operands(orc, 520, 1040, 0, seed=6)
    say("gemm determinism")
    g1 = gpu_gemm(fp8, a, 0, b, 0, sa, sb, 1, 1)
    g2 = gpu_gemm(fp8, a, 0, b, 0, sa, sb, 1, 1)
    assert np.array_equal(g1, g2)


# ------------------------------------------------------------------- grouped --

def gpu_grouped(fp8, a, fa, b, fb, offsets, sa, sb, out_f32=False):
    total, n = a.shape[0], b.shape[1]
    dt = torch.float32 if out_f32 else torch.bfloat16
    d, dbuf, org = guarded(total, n, dt)
    fp8.fp8_grouped_gemm_scaled(dev_u8(a), fa, dev_u8(b), fb, torch.from_numpy(offsets).to("cuda:0"),
                                dev_f32(sa), dev_f32(sb), d)
    torch.cuda.synchronize()
    check_guard(dbuf, org, total, n)
    return d.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("sizes", [[0, 1, 17, 255, 257], [300], [0, 0, 129, 0], [128, 128, 1, 0, 127],
                                   [5] * 40])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0)])
def test_grouped_gemm_parity(fp8, orc, sizes, fa, fb):
    g, n, k = len(sizes), 136, 272
    offsets = np.zeros(g + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    a, sa = operands(orc, total, k, fa, seed=7)
    bq = [operands(orc, n, k, fb, seed=100 + e) for e in range(g)]
    b = np.stack([q for q, _ in bq])
    sb = np.stack([s for _, s in bq])
    say("grouped", sizes, fa, fb)
    y, bound = orc.grouped_gemm(a, fa, b, fb, offsets, sa, sb)
    got = gpu_grouped(fp8, a, fa, b, fb, offsets, sa, sb)
    assert_within(orc, got, y, bound, True, f"grouped {sizes}")
    if g == 1:
        dense = gpu_gemm(fp8, a, fa, b[0], fb, sa, sb[0], 1, 1)
        assert np.array_equal(dense, got), "one group equals the dense GEMM"


LARGE = [((2100, 4100, 256), 0, 0, False, 4104), ((4096, 2048, 512), 1, 0, False, 2048),
         ((1024, 8192, 768), 0, 1, True, 8200), ((2304, 3100, 256), 1, 1, False, 3107),
         ((2304, 3100, 256), 0, 0, False, 3104), ((4096, 2048, 384), 1, 0, False, 2048),
         # more tiles than CUs with bf16 output (the persistent kernel: a workgroup
         # per CU walks several tiles, loading the next tile's first K steps during
         # the current tile's last ones): edge tiles shifted back to end at m / n
         # (n - 256 off the 8-column grid), m below one tile (clamped rows), an
         # output stride off the 8-element grid
         ((4100, 4500, 256), 0, 0, False, 4504), ((200, 65800, 256), 1, 0, False, 65800),
         ((2600, 7000, 512), 0, 0, False, 7003)]


@pytest.mark.parametrize("shape,fa,fb,out_f32,ldd", LARGE)
def test_gemm_parity_large_tiles(fp8, orc, shape, fa, fb, out_f32, ldd):
    """Shapes with >= 128 output tiles of 256 x 256 and k % 256 == 0 take the
    large-tile kernel (direct-to-LDS loads, LDS-staged epilogue); ragged m / n,
    fp32 output and an output stride off the 8-element grid cover its other
    store paths; k = 384 falls back to the 128 x 128 kernel."""
    m, n, k = shape
    a, sa = operands(orc, m, k, fa, seed=m + k)
    b, sb = operands(orc, n, k, fb, seed=n + k + 9)
    say("gemm large", shape, fa, fb, out_f32, ldd)
    y, bound = orc.gemm(a, fa, b, fb, sa, sb)
    got = gpu_gemm(fp8, a, fa, b, fb, sa, sb, 1, 1, out_f32=out_f32, ldd=ldd)
    assert_within(orc, got, y, bound, not out_f32, f"large {shape}")


@pytest.mark.parametrize("shape,fa,fb", [((2304, 8192, 256), 0, 0), ((2350, 8100, 512), 1, 0)])
def test_gemm_parity_persistent_scalar_scales(fp8, orc, shape, fa, fb):
    """One scale per operand (tensorwise recipes): the persistent kernel and its
    half-tile tail apply sa * sb as one factor. 288 / 320 tiles of 256 x 256:
    one round of 256 plus a tail of 32 / 64 tiles run as 256 x 128 halves;
    the second shape has ragged edges."""
    m, n, k = shape
    a, _ = operands(orc, m, k, fa, seed=m + 5)
    b, _ = operands(orc, n, k, fb, seed=n + 6)
    sa, sb = np.array([0.37], np.float32), np.array([2.5], np.float32)
    say("gemm persistent scalar scales", shape, fa, fb)
    y, bound = orc.gemm(a, fa, b, fb, sa, sb)
    got = gpu_gemm(fp8, a, fa, b, fb, sa, sb, 0, 0)
    assert_within(orc, got, y, bound, True, f"scalar scales {shape}")


def test_gemm_persistent_whole_last_round(fp8, orc):
    """450 tiles of 256 x 256: one round of 256 and a last round of 194 tiles,
    more than half the workgroups, so it runs as whole tiles (no half-tile
    tail); every output against the oracle."""
    m, n, k = 4608, 6400, 256
    a, sa = operands(orc, m, k, 0, seed=41)
    b, sb = operands(orc, n, k, 0, seed=42)
    say("gemm persistent whole last round", (m, n, k))
    d = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    fp8.fp8_gemm_scaled(dev_u8(a), 0, dev_u8(b), 0, dev_f32(sa), 1, dev_f32(sb), 1, d)
    torch.cuda.synchronize()
    check_full(orc, d, orc.gemm_by_rows(a, 0, b, 0, sa, sb), f"whole last round {(m, n, k)}")


@pytest.mark.parametrize("fa,fb", [(1, 0), (0, 0)])
def test_gemm_full_output_long_k(fp8, orc, fa, fb):
    """K = 14336 (the Llama3-8B backward's dgrad contraction) on 17 x 16 tiles of
    256 x 256 (the persistent kernel, ragged last row of tiles): every output
    against the oracle's whole product, with per-row scales spread over 2^-4 .. 2^4."""
    m, n, k = 4300, 4096, 14336
    a, sa = operands(orc, m, k, fa, seed=31)
    b, sb = operands(orc, n, k, fb, seed=32)
    say("gemm long k", (m, n, k), fa, fb)
    d = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
    fp8.fp8_gemm_scaled(dev_u8(a), fa, dev_u8(b), fb, dev_f32(sa), 1, dev_f32(sb), 1, d)
    torch.cuda.synchronize()
    check_full(orc, d, orc.gemm_by_rows(a, fa, b, fb, sa, sb), f"long k {(m, n, k)}")


def random_codes(rng, shape, fmt):
    """Uniformly random finite FP8 codes of format fmt (no NaN or Inf codes)."""
    top = 0x7E if fmt == 0 else 0x7B          # e4m3: 0x7F is NaN; e5m2: 0x7C.. are Inf / NaN
    c = rng.integers(0, top + 1, size=shape, dtype=np.uint8)
    c |= rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    return c


def many_groups(g=300, seed=11):
    rng = np.random.default_rng(seed)
    sizes = rng.integers(1, 30, g)
    sizes[::3] = 0                              # every third expert gets no rows
    sizes[7] = 1300                             # one large expert spanning several tiles
    return [int(x) for x in sizes]


GROUPED_LARGE = [([0, 1000, 1, 255, 257, 0, 2583], 2048, 512, 0, 0, False),
                 (many_groups(), 2048, 256, 1, 0, False),
                 ([4096], 2048, 256, 0, 1, True),
                 ([3000, 0, 1100], 2200, 768, 1, 1, False),
                 ([600, 0, 3500, 100], 2048, 4096, 0, 0, False)]


GROUPED_TAIL = [([0, 300, 1, 255, 257, 0, 700], 2300, 4352, 0, 0),
                ([4000, 0, 1, 255, 257, 3500], 2100, 4352, 1, 0)]


@pytest.mark.parametrize("sizes,n,k,fa,fb", GROUPED_TAIL, ids=["fewer_tiles_than_cus", "more_tiles_than_cus"])
def test_grouped_gemm_parity_long_k_bf16(fp8, orc, sizes, n, k, fa, fb):
    """Grouped products longer than the persistent form takes (k > 4096, bf16
    output: one 256 x 256 tile per workgroup), with fewer (81) and more (306)
    tiles than CUs, n off the 256 grid, empty and one-row groups. Every output
    against the oracle."""
    g = len(sizes)
    offsets = np.zeros(g + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    rng = np.random.default_rng(total + n + k + 2)
    a = random_codes(rng, (total, k), fa)
    b = random_codes(rng, (g, n, k), fb)
    sa = np.exp2(rng.integers(-8, 2, total)).astype(np.float32) * np.float32(1.375)
    sb = np.exp2(rng.integers(-8, 2, (g, n))).astype(np.float32)
    say("grouped long k bf16", g, total, n, k, fa, fb)
    got = gpu_grouped(fp8, a, fa, b, fb, offsets, sa, sb)
    rows = 0
    for e in range(g):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows += check_full(orc, got, orc.gemm_by_rows(a[lo:hi], fa, b[e], fb, sa[lo:hi], sb[e]),
                               f"grouped long k group {e}", row_offset=lo)
    assert rows == total


GROUPED_PERSIST = [([0, 1000, 1, 255, 257, 0, 2583, 60, 700], 3000, 512, 0, 0),
                   ([100, 0, 156], 16400, 256, 1, 0),
                   ([30000, 0, 25000, 15000], 200, 256, 0, 1),
                   ([600, 0, 3500, 100, 2000], 2304, 4096, 1, 0),
                   ([5000], 3100, 512, 0, 0)]


@pytest.mark.parametrize("sizes,n,k,fa,fb", GROUPED_PERSIST,
                         ids=["ragged_shifted", "one_tile_of_rows", "n_below_tile", "k4096", "one_group"])
def test_grouped_gemm_parity_persistent(fp8, orc, sizes, n, k, fa, fb):
    """Shapes that take the persistent grouped kernel (bf16 output, k <= 4096,
    more tile slots than CUs): a group's partial last m-tile shifted back inside
    the token matrix (its extra rows belong to other groups and are never
    stored), 256 rows in all (every tile loads the whole matrix), n off the 256
    grid (column tiles shifted back) and below one tile (clamped), the longest
    contraction it takes, empty and one-row groups; every output against the
    oracle. One group must equal the dense product (the same K loop)."""
    g = len(sizes)
    offsets = np.zeros(g + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    assert total >= 256 and ((total + 255) // 256 + g) * ((n + 255) // 256) > 256 and k % 256 == 0
    rng = np.random.default_rng(total + n + k + 1)
    a = random_codes(rng, (total, k), fa)
    b = random_codes(rng, (g, n, k), fb)
    sa = np.exp2(rng.integers(-8, 2, total)).astype(np.float32) * np.float32(1.375)
    sb = np.exp2(rng.integers(-8, 2, (g, n))).astype(np.float32)
    say("grouped persistent", g, total, n, k, fa, fb)
    got = gpu_grouped(fp8, a, fa, b, fb, offsets, sa, sb)
    rows = 0
    for e in range(g):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows += check_full(orc, got, orc.gemm_by_rows(a[lo:hi], fa, b[e], fb, sa[lo:hi], sb[e]),
                               f"grouped persistent group {e}", row_offset=lo)
    assert rows == total
    if g == 1:
        say("grouped persistent: one group vs dense")
        dense = gpu_gemm(fp8, a, fa, b[0], fb, sa, sb[0], 1, 1)
        assert np.array_equal(dense, got), "one group equals the dense GEMM"


@pytest.mark.parametrize("sizes,n,k,fa,fb,out_f32", GROUPED_LARGE,
                         ids=["ragged", "g300", "one", "ragged_n", "long_k"])
def test_grouped_gemm_parity_large_tiles(fp8, orc, sizes, n, k, fa, fb, out_f32):
    """Shapes that take the 256 x 256 grouped kernel (k % 256 == 0, at least 128
    tiles of 256 x 256 estimated from the total row count): empty groups, a
    one-row group, groups spanning several m-tiles, more groups than threads of
    a workgroup (the per-group tile counts are summed in parallel), ragged n,
    and a long contraction (k = 4096)."""
    g = len(sizes)
    offsets = np.zeros(g + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    assert -(-total // 256) * -(-n // 256) >= 128 and k % 256 == 0
    rng = np.random.default_rng(total + n + k)
    a = random_codes(rng, (total, k), fa)
    b = random_codes(rng, (g, n, k), fb)
    sa = np.exp2(rng.integers(-8, 2, total)).astype(np.float32) * np.float32(1.375)
    sb = np.exp2(rng.integers(-8, 2, (g, n))).astype(np.float32)
    say("grouped large", g, total, n, k, fa, fb, out_f32)
    y, bound = orc.grouped_gemm(a, fa, b, fb, offsets, sa, sb)
    got = gpu_grouped(fp8, a, fa, b, fb, offsets, sa, sb, out_f32=out_f32)
    assert_within(orc, got, y, bound, not out_f32, f"grouped large {g} groups")
    if g == 1:
        say("grouped large: one group vs dense")
        dense = gpu_gemm(fp8, a, fa, b[0], fb, sa, sb[0], 1, 1, out_f32=out_f32, ldd=n + 32)
        assert np.array_equal(dense, got), "one group equals the dense GEMM"
