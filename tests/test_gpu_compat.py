"""GPU parity of the fnuz compatibility products ("FP8 Training on MI300X": the
fnuz encodings MI300 parts consume) against the CPU oracle, which decodes each
encoding natively: dense and grouped scaled GEMMs with at least one fnuz
operand, every output within the GEMM bound; fnuz's special codes (the single
NaN 0x80, the top binade that is Inf / NaN as OCP bits, 2^-10); exact integer
products; and the wrong-encoding corruption the page warns about (the same
bytes read as OCP halve or double every value)."""
import numpy as np
import pytest
import torch

from helpers import check_full, check_guard, dev_f32, dev_u8, guarded, say

pytestmark = pytest.mark.gpu

NAMES = {0: "e4m3", 1: "e5m2", 2: "e4m3fnuz", 3: "e5m2fnuz"}
FNUZ_PAIRS = [(fa, fb) for fa in range(4) for fb in range(4) if fa >= 2 or fb >= 2]


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def finite_codes(orc, rng, shape, fmt):
    """Uniform random codes of fmt whose values are finite (NaN / Inf codes replaced)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    bad = ~np.isfinite(orc.decode(fmt, c))
    c[bad] = 0x3A
    return c


def gpu_gemm(fp8, a, fa, b, fb, sa, sb, a_mode=1, b_mode=1, out_f32=False, ldd=None):
    m, n = a.shape[0], b.shape[0]
    dt = torch.float32 if out_f32 else torch.bfloat16
    d, dbuf, org = guarded(m, n, dt, ld=ldd)
    fp8.fp8_gemm_scaled(dev_u8(a), fa, dev_u8(b), fb, dev_f32(sa), a_mode, dev_f32(sb), b_mode, d)
    torch.cuda.synchronize()
    check_guard(dbuf, org, m, n)
    return d


@pytest.mark.parametrize("fa,fb", FNUZ_PAIRS, ids=[f"{NAMES[a]}x{NAMES[b]}" for a, b in FNUZ_PAIRS])
def test_compat_gemm_every_pair(fp8, orc, fa, fb):
    """Random finite codes on ragged shapes (m, n off the 128 tile, k = 304 off
    the 32-deep step), row and column scales, bf16 and fp32 output, a padded
    output stride; every output against the oracle."""
    rng = np.random.default_rng(10 * fa + fb)
    m, n, k = 200, 130, 304
    a = finite_codes(orc, rng, (m, k), fa)
    b = finite_codes(orc, rng, (n, k), fb)
    sa = np.exp2(rng.integers(-6, 3, m)).astype(np.float32) * np.float32(1.1)
    sb = rng.uniform(0.5, 2.0, n).astype(np.float32)
    for out_f32 in (False, True):
        say("compat gemm", NAMES[fa], NAMES[fb], "f32" if out_f32 else "bf16")
        d = gpu_gemm(fp8, a, fa, b, fb, sa, sb, out_f32=out_f32, ldd=n + 8)
        check_full(orc, d, orc.gemm_by_rows(a, fa, b, fb, sa, sb, chunk=64), f"compat {fa} {fb}",
                   out_bf16=not out_f32)


def test_compat_gemm_tensor_scales_and_larger_shape(fp8, orc):
    """1040 x 1300 x 1024, e5m2fnuz x e4m3fnuz (the fnuz hybrid backward pair),
    tensor scales, every output."""
    rng = np.random.default_rng(3)
    m, n, k = 1040, 1300, 1024
    a = finite_codes(orc, rng, (m, k), 3)
    b = finite_codes(orc, rng, (n, k), 2)
    sa, sb = np.float32([0.37]), np.float32([2.5])
    say("compat gemm larger", (m, n, k))
    d = gpu_gemm(fp8, a, 3, b, 2, sa, sb, a_mode=0, b_mode=0)
    check_full(orc, d, orc.gemm_by_rows(a, 3, b, 2, sa, sb), "compat larger")


def test_compat_fnuz_special_codes(fp8, orc):
    """fnuz NaN (0x80) makes exactly its row's outputs NaN; the fnuz top
    binade (e4m3fnuz +-240 = 0x7F / 0xFF, e5m2fnuz 0x7C..0x7F), which OCP would
    read as Inf / NaN, and the e4m3fnuz subnormal 2^-10 (0x01) are finite and
    exact: unit scales, fp32 output, k = 64 (sums exact in fp32)."""
    rng = np.random.default_rng(4)
    m, n, k = 40, 48, 64
    a = finite_codes(orc, rng, (m, k), 2)
    b = finite_codes(orc, rng, (n, k), 3)
    a[0, :] = 0x7F
    a[1, :] = 0xFF
    a[2, :] = 0x01
    a[3, 5] = 0x80                                      # NaN
    b[0, :] = 0x7C
    b[1, :] = 0x7F
    b[2, :] = 0xFE
    one = np.float32([1.0])
    say("compat specials")
    d = gpu_gemm(fp8, a, 2, b, 3, one, one, a_mode=0, b_mode=0, out_f32=True).cpu().numpy().astype(np.float64)
    y, bound = orc.gemm(a, 2, b, 3, one, one)
    assert orc.decode(2, np.uint8([0x7F]))[0] == 240.0 and orc.decode(2, np.uint8([0x01]))[0] == 2.0 ** -10
    assert orc.decode(3, np.uint8([0x7F]))[0] == 57344.0
    assert np.isnan(d[3]).all() and not np.isnan(np.delete(d, 3, axis=0)).any()
    keep = np.ones(m, bool)
    keep[3] = False
    assert orc.gemm_within_bound(d[keep], y[keep], bound[keep], out_bf16=False).all()
    assert np.isfinite(d[:3]).all() and np.abs(d[:2, :2]).max() > 1e6      # the +-240 x top-binade rows


def test_compat_integer_products_exact(fp8, orc):
    """Small integer values in e4m3fnuz and e5m2fnuz with unit scales: the
    result is the int64 matmul exactly (fp32 output)."""
    from test_oracle_gemm import codes_for_small_ints
    rng = np.random.default_rng(5)
    m, n, k = 130, 70, 512
    ia = rng.integers(-7, 8, (m, k))
    ib = rng.integers(-7, 8, (n, k))
    a = codes_for_small_ints(orc, 2, ia)
    b = codes_for_small_ints(orc, 3, ib)
    one = np.float32([1.0])
    say("compat integers")
    d = gpu_gemm(fp8, a, 2, b, 3, one, one, a_mode=0, b_mode=0, out_f32=True).cpu().numpy()
    assert np.array_equal(d.astype(np.int64), ia @ ib.T)


def test_compat_wrong_encoding_corrupts_silently(fp8, orc):
    """The same bytes read as OCP instead of fnuz (the mismatch the MI300X page
    describes): normal e4m3 values come out doubled, with no error; the library
    computes with the encoding it is given."""
    rng = np.random.default_rng(6)
    m, n, k = 64, 64, 128
    a = rng.integers(0x08, 0x78, (m, k)).astype(np.uint8)          # normal, finite in both encodings
    b = rng.integers(0x08, 0x78, (n, k)).astype(np.uint8)
    one = np.float32([1.0])
    say("compat wrong encoding")
    d_fnuz = gpu_gemm(fp8, a, 2, b, 2, one, one, a_mode=0, b_mode=0, out_f32=True).cpu().numpy()
    d_ocp = gpu_gemm(fp8, a, 0, b, 0, one, one, a_mode=0, b_mode=0, out_f32=True).cpu().numpy()
    y, bound = orc.gemm(a, 2, b, 2, one, one)
    assert orc.gemm_within_bound(d_fnuz, y, bound, out_bf16=False).all()
    # read as OCP each operand doubles: 4x the product, no error (the two kernels
    # accumulate differently, so the match is to the bound, not bitwise)
    assert orc.gemm_within_bound(d_ocp, 4.0 * y, 4.0 * bound, out_bf16=False).all()
    assert np.all(np.abs(d_ocp / d_fnuz - 4.0) < 1e-3)


def test_compat_grouped_gemm(fp8, orc):
    """Grouped product with fnuz operands: group sizes {0, 1, 17, 255, 257},
    every row of every group against the per-group oracle."""
    sizes = [0, 1, 17, 255, 257]
    g, n, k = len(sizes), 144, 256
    offsets = np.zeros(g + 1, np.int64)
    offsets[1:] = np.cumsum(sizes)
    total = int(offsets[-1])
    rng = np.random.default_rng(7)
    a = finite_codes(orc, rng, (total, k), 3)
    b = finite_codes(orc, rng, (g, n, k), 2)
    sa = rng.uniform(0.5, 2, total).astype(np.float32)
    sb = rng.uniform(0.5, 2, (g, n)).astype(np.float32)
    d = torch.full((total, n), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    say("compat grouped", sizes)
    fp8.fp8_grouped_gemm_scaled(dev_u8(a), 3, dev_u8(b), 2, torch.from_numpy(offsets).to("cuda:0"), dev_f32(sa),
                                dev_f32(sb), d)
    torch.cuda.synchronize()
    host = d.float().cpu().numpy()
    rows = 0
    for e in range(g):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows += check_full(orc, host, orc.gemm_by_rows(a[lo:hi], 3, b[e], 2, sa[lo:hi], sb[e]),
                               f"compat group {e}", row_offset=lo)
    assert rows == total
