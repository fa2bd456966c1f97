"""GPU parity of the MXFP8 entry points against the CPU oracle, through the C
ABI: the block-32 E8M0 quantizer bit-exact (codes and scale bytes, every bf16
value, special blocks, row slices past 16384 columns, strided views with guard
bands) and the block-scaled products, dense and grouped, within the GEMM
bound (several tiles and ragged edges, a NaN scale byte, k = 0)."""
import numpy as np
import pytest
import torch

import workloads
from helpers import SENTINEL, assert_codes_equal, check_full, check_guard, dev_bf16, dev_u8, guarded, say

pytestmark = pytest.mark.gpu

BLOCK = 32


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def block_scaled_bf16(rows, cols, seed, spread=20):
    """N(0, 1) values times a power of two drawn per 32-element block from
    2^-spread .. 2^spread, as bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-spread, spread + 1, (rows, cols // BLOCK))).repeat(BLOCK, axis=1).astype(np.float32)
    return workloads.bf16_bits(x)


def to_records(s):
    """Scale bytes [rows x nb] (the oracle's row-major blocks) -> the library's
    K-step-major records [ceil(nb/4) x rows x 4], zero bytes past nb."""
    rows, nb = s.shape
    J = (nb + 3) // 4
    pad = np.zeros((rows, 4 * J), np.uint8)
    pad[:, :nb] = s
    return np.ascontiguousarray(pad.reshape(rows, J, 4).transpose(1, 0, 2))


def dev_records(s):
    return dev_u8(to_records(s))


def gpu_mx_quantize(fp8, xb, fmt, ldx=None, ldq=None, lds_extra=3):
    """Quantize on the GPU into guarded outputs (the scale records with
    lds_extra spare records per K step); returns (codes, scale records)."""
    rows, cols = xb.shape
    J = (cols + 127) // 128
    if ldx is not None:
        xbuf = torch.zeros((rows, ldx), dtype=torch.bfloat16, device="cuda:0")
        xbuf[:, :cols] = dev_bf16(xb)
        x = xbuf[:, :cols]
    else:
        x = dev_bf16(xb)
    q, qbuf, qo = guarded(rows, cols, torch.uint8, ld=ldq)
    ld = rows + lds_extra
    sbuf = torch.full((J + 2, ld * 4), SENTINEL, dtype=torch.uint8, device="cuda:0")
    s = sbuf[1:1 + J].view(J, ld, 4)[:, :rows, :]
    fp8.fp8_mx_quantize_row(x, fmt, q, s)
    torch.cuda.synchronize()
    check_guard(qbuf, qo, rows, cols)
    host = sbuf.cpu().numpy()
    outside = np.ones(host.shape, bool)
    outside[1:1 + J, :rows * 4] = False
    assert np.all(host[outside] == SENTINEL), "write outside the scale records"
    return q.cpu().numpy(), s.cpu().numpy()


SHAPES = [(1, 32), (7, 96), (64, 512), (33, 4096 + 32), (5, 16384), (3, 16384 + 512), (2, 40000)]


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_mx_quantize_row_parity(fp8, orc, fmt, rows, cols):
    """Random blocks over forty binades; one slice, several chunks per lane, a
    ragged chunk count, and rows longer than one 16384-column slice."""
    xb = block_scaled_bf16(rows, cols, seed=rows * 7 + cols + fmt)
    say("mx quantize", rows, cols, fmt)
    q, s = gpu_mx_quantize(fp8, xb, fmt)
    oq, osc = orc.mx_quantize_row(xb, fmt)
    assert_codes_equal(s, to_records(osc), "scale records")
    assert_codes_equal(q, oq, "codes")


@pytest.mark.parametrize("fmt", [0, 1])
def test_mx_quantize_every_bf16_value(fp8, orc, fmt):
    """All 65536 bf16 patterns, in order (each block a run of neighbouring
    patterns) and shuffled (blocks mixing NaN, Inf, zeros, subnormals and
    normals of every binade)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for name, bits in (("ordered", allb), ("shuffled", np.random.default_rng(3).permutation(allb))):
        xb = bits.reshape(64, 1024)
        say("mx every bf16", name, fmt)
        q, s = gpu_mx_quantize(fp8, xb, fmt)
        oq, osc = orc.mx_quantize_row(xb, fmt)
        assert_codes_equal(s, to_records(osc), f"scale records ({name})")
        assert_codes_equal(q, oq, f"codes ({name})")


def test_mx_quantize_special_blocks(fp8, orc):
    """Blocks of zeros (both signs), one NaN, +-Inf, a lone subnormal, the
    largest bf16 values, and a block whose amax sits exactly on a power of two."""
    rows = np.zeros((6, 8 * BLOCK), np.float32)
    rows[1, 3] = np.inf
    rows[2, 40] = -np.inf
    rows[3, 64] = 2.0 ** -133
    rows[4, 100:132] = 3.3895314e38
    rows[5, 160:192] = np.linspace(-1.0, 1.0, 32)
    rows[5, 200] = 256.0
    xb = workloads.bf16_bits(rows)
    xb[0, 0:32] = 0x8000                                   # negative zeros
    xb[1, 70] = 0x7FC1                                     # NaN
    xb[2, 255] = 0xFFC0                                    # -NaN
    for fmt in (0, 1):
        say("mx special", fmt)
        q, s = gpu_mx_quantize(fp8, xb, fmt)
        oq, osc = orc.mx_quantize_row(xb, fmt)
        assert_codes_equal(s, to_records(osc), "scale records")
        assert_codes_equal(q, oq, "codes")


def test_mx_quantize_strided(fp8, orc):
    """Leading dimensions past the row: x, q and the scales as strided views."""
    xb = block_scaled_bf16(37, 1024, seed=11)
    say("mx strided")
    q, s = gpu_mx_quantize(fp8, xb, 0, ldx=1024 + 72, ldq=1024 + 40, lds_extra=61)
    oq, osc = orc.mx_quantize_row(xb, 0)
    assert_codes_equal(s, to_records(osc), "scale records")
    assert_codes_equal(q, oq, "codes")


def assert_within(orc, got, y, bound, out_bf16, what):
    ok = orc.gemm_within_bound(got, y, bound, out_bf16=out_bf16)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound; first {i}: "
                             f"gpu {got[i]!r} oracle {y[i]!r} bound {bound[i]!r}")


def mx_operands(orc, rows, k, fmt, seed, spread=6):
    xb = block_scaled_bf16(rows, k, seed, spread=spread)
    return orc.mx_quantize_row(xb, fmt)


def gpu_gemm_mx(fp8, a, fa, sa, b, fb, sb, out_f32=False):
    m, n = a.shape[0], b.shape[0]
    d, dbuf, do = guarded(m, n, torch.float32 if out_f32 else torch.bfloat16, ld=n + 8)
    fp8.fp8_gemm_mx(dev_u8(a), fa, dev_records(sa), dev_u8(b), fb, dev_records(sb), d)
    torch.cuda.synchronize()
    check_guard(dbuf, do, m, n)
    return d.float().cpu().numpy().astype(np.float64)


GEMMS = [(300, 520, 512, 0, 0, False), (256, 256, 256, 0, 1, False), (1, 7, 256, 1, 0, True),
         (513, 1000, 768, 0, 0, True), (1030, 260, 1536, 1, 1, False), (512, 768, 1024, 1, 0, True),
         (768, 512, 512, 0, 0, False)]


@pytest.mark.parametrize("m,n,k,fa,fb,out_f32", GEMMS)
def test_gemm_mx_parity(fp8, orc, m, n, k, fa, fb, out_f32):
    """Operands from the oracle's MX quantizer; tiles of 256 with ragged edges
    and whole tiles only, one to six 256-deep passes of the K loop, every
    format pair."""
    a, sa = mx_operands(orc, m, k, fa, seed=m + k)
    b, sb = mx_operands(orc, n, k, fb, seed=n + 2 * k)
    say("gemm mx", m, n, k, fa, fb, out_f32)
    got = gpu_gemm_mx(fp8, a, fa, sa, b, fb, sb, out_f32)
    y, bound = orc.mx_gemm(a, fa, sa, b, fb, sb)
    assert_within(orc, got, y, bound, not out_f32, f"mx gemm {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k,fa,fb", [(2350, 8100, 512, 0, 0), (4352, 4200, 256, 1, 0)])
def test_gemm_mx_persistent_parity(fp8, orc, m, n, k, fa, fb):
    """More 256 x 256 tiles than CUs with bf16 output: the persistent MX kernel
    (each workgroup walks several tiles, loading the next tile's first two K
    steps and scale records during the current tile's last two); ragged edges
    (shifted-back edge tiles), k = 256 (one step pair, which is also the
    last), every output against the oracle."""
    a, sa = mx_operands(orc, m, k, fa, seed=m + 3 * k)
    b, sb = mx_operands(orc, n, k, fb, seed=n + 5 * k)
    say("gemm mx persistent", m, n, k, fa, fb)
    got = gpu_gemm_mx(fp8, a, fa, sa, b, fb, sb)
    check_full(orc, got, orc.mx_gemm_by_rows(a, fa, sa, b, fb, sb), f"mx persistent {m}x{n}x{k}")


def test_gemm_mx_random_codes_and_scales(fp8, orc):
    """Codes drawn uniformly over the finite codes and scale bytes drawn
    independently per block (117 .. 137): a scale applied to the wrong block,
    row or half of the instruction shows at once."""
    rng = np.random.default_rng(21)
    m, n, k = 300, 290, 1024
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    b = rng.integers(0, 256, (n, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x10                           # no NaN codes (e4m3)
    b[(b & 0x7F) == 0x7F] = 0x10
    sa = rng.integers(117, 138, (m, k // BLOCK)).astype(np.uint8)
    sb = rng.integers(117, 138, (n, k // BLOCK)).astype(np.uint8)
    say("gemm mx random codes and scales")
    got = gpu_gemm_mx(fp8, a, 0, sa, b, 0, sb, out_f32=True)
    y, bound = orc.mx_gemm(a, 0, sa, b, 0, sb)
    assert_within(orc, got, y, bound, False, "mx gemm random scales")


def test_gemm_mx_nan_scale_and_empty_k(fp8, orc):
    """A NaN scale byte in one block of a row of a (that row of d is NaN, the
    others are not), and k = 0 (d = 0)."""
    m, n, k = 40, 72, 512
    a, sa = mx_operands(orc, m, k, 0, seed=5)
    b, sb = mx_operands(orc, n, k, 0, seed=6)
    sa[17, 9] = 0xFF
    say("gemm mx nan scale")
    got = gpu_gemm_mx(fp8, a, 0, sa, b, 0, sb, out_f32=True)
    y, bound = orc.mx_gemm(a, 0, sa, b, 0, sb)
    assert np.isnan(y[17]).all()
    assert_within(orc, got, y, bound, False, "mx gemm nan scale")
    say("gemm mx k = 0")
    d = torch.full((m, n), float("nan"), device="cuda:0")
    e = torch.empty((m, 0), dtype=torch.uint8, device="cuda:0")
    fp8.fp8_gemm_mx(e, 0, torch.empty((0, m, 4), dtype=torch.uint8, device="cuda:0"),
                    torch.empty((n, 0), dtype=torch.uint8, device="cuda:0"), 0,
                    torch.empty((0, n, 4), dtype=torch.uint8, device="cuda:0"), d)
    torch.cuda.synchronize()
    assert (d == 0).all().item()


def offsets_of(sizes):
    off = np.zeros(len(sizes) + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    return off


GROUPED = [([0, 1, 255, 256, 257, 0, 600], 520, 512, 0, 0, False), ([300], 256, 256, 1, 0, True),
           ([17] * 30, 96, 768, 0, 1, False), ([1000, 20, 700, 3], 1024, 2048, 0, 0, False),
           ([0, 300, 1, 257, 0, 520], 300, 4096, 1, 0, True), ([513, 2, 256], 520, 4352, 0, 1, False)]


@pytest.mark.parametrize("sizes,n,k,fa,fb,out_f32", GROUPED,
                         ids=["ragged", "one", "many", "large", "long_k", "long_k_ragged"])
def test_grouped_gemm_mx_parity(fp8, orc, sizes, n, k, fa, fb, out_f32):
    """Groups with empty, one-row and tile-straddling row counts; weights and
    their scales as strided [g x n x k] and [g x n x k/32] stacks."""
    offsets = offsets_of(sizes)
    T, g = int(offsets[-1]), len(sizes)
    a, sa = mx_operands(orc, T, k, fa, seed=T + k)
    bq, bs = mx_operands(orc, g * n, k, fb, seed=n + k)
    b = bq.reshape(g, n, k)
    sb = bs.reshape(g, n, k // BLOCK)
    say("grouped gemm mx", sizes, n, k, fa, fb, out_f32)
    dt = torch.float32 if out_f32 else torch.bfloat16
    d, dbuf, do = guarded(T, n, dt, ld=n + 8)
    sb_rec = np.stack([to_records(sb[e]) for e in range(g)])
    fp8.fp8_grouped_gemm_mx(dev_u8(a), fa, dev_records(sa), dev_u8(b), fb, dev_u8(sb_rec),
                            torch.from_numpy(offsets).to("cuda:0"), d)
    torch.cuda.synchronize()
    check_guard(dbuf, do, T, n)
    got = d.float().cpu().numpy().astype(np.float64)
    y, bound = orc.mx_grouped_gemm(a, fa, sa, b, fb, sb, offsets)
    assert_within(orc, got, y, bound, not out_f32, f"grouped mx {sizes}")


def test_grouped_gemm_mx_long_k_random_scales(fp8, orc):
    """The long-K grouped product (32 K steps through the two LDS stages) with
    codes drawn uniformly and scale bytes drawn independently per block: a
    scale byte taken from the wrong step, block or stage shows at once."""
    rng = np.random.default_rng(23)
    sizes, n, k = [260, 0, 1, 300], 270, 4096
    offsets = offsets_of(sizes)
    T, g = int(offsets[-1]), len(sizes)
    a = rng.integers(0, 256, (T, k)).astype(np.uint8)
    b = rng.integers(0, 256, (g, n, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x10                           # no NaN codes (e4m3)
    b[(b & 0x7F) == 0x7F] = 0x10
    sa = rng.integers(117, 138, (T, k // BLOCK)).astype(np.uint8)
    sb = rng.integers(117, 138, (g, n, k // BLOCK)).astype(np.uint8)
    say("grouped gemm mx long k random scales")
    d, dbuf, do = guarded(T, n, torch.float32, ld=n + 4)
    sb_rec = np.stack([to_records(sb[e]) for e in range(g)])
    fp8.fp8_grouped_gemm_mx(dev_u8(a), 0, dev_records(sa), dev_u8(b), 0, dev_u8(sb_rec),
                            torch.from_numpy(offsets).to("cuda:0"), d)
    torch.cuda.synchronize()
    check_guard(dbuf, do, T, n)
    y, bound = orc.mx_grouped_gemm(a, 0, sa, b, 0, sb, offsets)
    assert_within(orc, d.cpu().numpy().astype(np.float64), y, bound, False, "grouped mx long k random scales")


def test_mx_layer_forward_composed(fp8, orc):
    """bf16 activations and weights through the library only (MX quantizer on
    both, MX product) against the oracle's composition of the same steps."""
    m, n, k = 260, 300, 1024
    xb = workloads.bf16_bits(np.random.default_rng(8).standard_normal((m, k)).astype(np.float32))
    wb = workloads.bf16_bits((0.02 * np.random.default_rng(9).standard_normal((n, k))).astype(np.float32))
    say("mx layer forward")
    dev = "cuda:0"
    xq = torch.empty((m, k), dtype=torch.uint8, device=dev)
    xs = fp8.mx_scale_records(m, k)
    wq = torch.empty((n, k), dtype=torch.uint8, device=dev)
    ws = fp8.mx_scale_records(n, k)
    fp8.fp8_mx_quantize_row(dev_bf16(xb), 0, xq, xs)
    fp8.fp8_mx_quantize_row(dev_bf16(wb), 0, wq, ws)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    fp8.fp8_gemm_mx(xq, 0, xs, wq, 0, ws, y)
    torch.cuda.synchronize()
    oxq, oxs = orc.mx_quantize_row(xb, 0)
    owq, ows = orc.mx_quantize_row(wb, 0)
    assert_codes_equal(xq.cpu().numpy(), oxq, "x codes")
    assert_codes_equal(ws.cpu().numpy(), to_records(ows), "w scales")
    oy, ob = orc.mx_gemm(oxq, 0, oxs, owq, 0, ows)
    assert_within(orc, y.float().cpu().numpy().astype(np.float64), oy, ob, True, "mx forward")
