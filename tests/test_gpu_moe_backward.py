"""GPU parity of the MoE-backward entry points against the CPU oracle, through
the C ABI: the grouped colwise quantizer (codes of the whole padded layout,
scales and per-group amax bit-exact; nothing written past the layout) and the
grouped product over ragged contraction ranges (within the GEMM bound), then
the two composed into an expert layer's dgrad and wgrad."""
import numpy as np
import pytest
import torch

import workloads
from helpers import SENTINEL, assert_codes_equal, assert_f32_bits_equal, dev_bf16, dev_f32, dev_u8, say

pytestmark = pytest.mark.gpu

ALIGN = 256


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def offsets_of(sizes):
    off = np.zeros(len(sizes) + 1, np.int64)
    off[1:] = np.cumsum(sizes)
    return off


def rand_bf16(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-6, 7, size=(1, cols))).astype(np.float32)
    return workloads.bf16_bits(x)


def gpu_grouped_col(fp8, xb, fmt, offsets, ready=None):
    """Returns (qt [cols x P_G], scale_inv, amax) and checks that nothing was
    written past column P_G of the (wider) qt buffer."""
    total, cols = xb.shape
    g = len(offsets) - 1
    width = fp8.grouped_layout_width(total, g)
    qt = torch.full((cols, width), SENTINEL, dtype=torch.uint8, device="cuda:0")
    si = torch.full((g, cols), -1.0, device="cuda:0")
    ca = dev_f32(ready) if ready is not None else torch.full((g, cols), -1.0, device="cuda:0")
    fp8.fp8_grouped_quantize_col(dev_bf16(xb), fmt, 0, torch.from_numpy(offsets).to("cuda:0"), qt, si, ca,
                                 col_amax_ready=ready is not None)
    torch.cuda.synchronize()
    P = int(padded(offsets)[-1])
    host = qt.cpu().numpy()
    assert np.all(host[:, P:] == SENTINEL), "write past the grouped layout"
    return host[:, :P], si.cpu().numpy(), ca.cpu().numpy()


def padded(offsets):
    sizes = np.diff(offsets)
    out = np.zeros(len(offsets), np.int64)
    out[1:] = np.cumsum((sizes + ALIGN - 1) // ALIGN * ALIGN)
    return out


GROUPS = [[0, 1, 255, 256, 257, 0, 600], [300], [0, 0, 5], [512] * 4, [17] * 30,
          [3000, 5, 2100, 0, 2048, 2049], [2048] * 3 + [1]]


@pytest.mark.parametrize("fmt", [0, 1, 2])
@pytest.mark.parametrize("sizes", GROUPS)
def test_grouped_quantize_col_parity(fp8, orc, fmt, sizes):
    offsets = offsets_of(sizes)
    cols = 72                                              # 64-column tiles (two-pass) and 32-column strips
                                                           # (one pass, groups of <= 2048 rows), both ragged
    xb = rand_bf16(int(offsets[-1]), cols, seed=len(sizes) + fmt)
    say("grouped col", sizes, fmt)
    qt, si, am = gpu_grouped_col(fp8, xb, fmt, offsets)
    oq, osi, oam = orc.grouped_quantize_col(xb, fmt, offsets, ALIGN)
    assert_codes_equal(qt, oq, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(am, oam, "amax")


def test_grouped_quantize_col_one_pass(fp8, orc):
    """A tensor past 256 MB (70,000 rows x 2048 columns) takes the one-pass
    kernel for its groups of at most 2048 rows (32-column strips) and the two
    passes for the rest: 30 groups of 2048 rows, then 3000, 1, 0, 2500, 1003
    and 2049 rows, a NaN in a one-pass group; all codes, scales and amax
    bit-exact."""
    sizes = [2048] * 30 + [3000, 1, 0, 2500, 1003, 2049]
    offsets = offsets_of(sizes)
    xb = rand_bf16(int(offsets[-1]), 2048, seed=77)
    xb[5000, 100] = 0x7FC0                                 # group 2
    say("grouped col one pass", int(offsets[-1]))
    qt, si, am = gpu_grouped_col(fp8, xb, 0, offsets)
    oq, osi, oam = orc.grouped_quantize_col(xb, 0, offsets, ALIGN)
    assert_codes_equal(qt, oq, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(am, oam, "amax")


def test_grouped_quantize_col_nan_and_ready_amax(fp8, orc):
    """A NaN in one group's column (its codes take the bit-level encoder, the
    other groups' codes of that column are unaffected), in a small group and
    in one past 2048 rows, and col_amax_ready = 1 with the per-group amax
    supplied."""
    sizes = [40, 0, 300, 3, 2500]
    offsets = offsets_of(sizes)
    xb = rand_bf16(int(offsets[-1]), 64, seed=9)
    xb[50, 7] = 0xFFC0                                     # -NaN in group 2, column 7
    xb[5, 9] = 0x7F80                                      # +Inf in group 0
    xb[400, 11] = 0x7FC0                                   # NaN in group 4 (2500 rows)
    say("grouped col nan")
    qt, si, am = gpu_grouped_col(fp8, xb, 1, offsets)
    oq, osi, oam = orc.grouped_quantize_col(xb, 1, offsets, ALIGN)
    assert_codes_equal(qt, oq, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(am, oam, "amax")
    say("grouped col ready amax")
    qt2, si2, _ = gpu_grouped_col(fp8, xb, 1, offsets, ready=oam)
    assert_codes_equal(qt2, oq, "codes (ready amax)")
    assert_f32_bits_equal(si2, osi, "scale_inv (ready amax)")


def gpu_ragged(fp8, a_t, fa, b_t, fb, offsets, sa, sb, out_f32=False):
    g = len(offsets) - 1
    m, n = a_t.shape[0], b_t.shape[0]
    dt = torch.float32 if out_f32 else torch.bfloat16
    # a guard group of rows after the last output group
    dbuf = torch.full((g + 1, m, n), float("nan"), dtype=dt, device="cuda:0")
    d = dbuf[:g]
    fp8.fp8_grouped_gemm_ragged_k(dev_u8(a_t), fa, dev_u8(b_t), fb, torch.from_numpy(offsets).to("cuda:0"),
                                  int(offsets[-1]), dev_f32(sa), dev_f32(sb), d)
    torch.cuda.synchronize()
    assert torch.isnan(dbuf[g]).all().item(), "write past the last group"
    return d.float().cpu().numpy().astype(np.float64)


def assert_within(orc, got, y, bound, out_bf16, what):
    ok = orc.gemm_within_bound(got, y, bound, out_bf16=out_bf16)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside the bound; first {i}: "
                             f"gpu {got[i]!r} oracle {y[i]!r} bound {bound[i]!r}")


RAGGED = [([0, 1, 255, 256, 257, 0, 600], 300, 520, 1, 0, False),
          ([300], 256, 256, 0, 0, True),
          ([0, 0, 0], 64, 96, 1, 0, False),
          ([1000, 20, 700, 3], 2048, 1024, 1, 0, False)]


@pytest.mark.parametrize("sizes,m,n,fa,fb,out_f32", RAGGED, ids=["ragged", "one", "all_empty", "large"])
def test_grouped_gemm_ragged_k_parity(fp8, orc, sizes, m, n, fa, fb, out_f32):
    """Operands are the oracle's grouped colwise codes of random dY [T x m] and
    X [T x n]; every group's weight gradient within the GEMM bound, empty
    groups exactly zero, nothing written past the last group."""
    offsets = offsets_of(sizes)
    T = int(offsets[-1])
    rng = np.random.default_rng(m + n)
    if T > 0:
        a_t, sa, _ = orc.grouped_quantize_col(rand_bf16(T, m, 1), fa, offsets, ALIGN)
        b_t, sb, _ = orc.grouped_quantize_col(rand_bf16(T, n, 2), fb, offsets, ALIGN)
    else:
        a_t, b_t = np.zeros((m, 16), np.uint8), np.zeros((n, 16), np.uint8)
        sa = np.ones((len(sizes), m), np.float32)
        sb = np.ones((len(sizes), n), np.float32)
    sa = sa * np.float32(rng.uniform(0.5, 2))
    say("ragged k", sizes, m, n, fa, fb, out_f32)
    y, bound = orc.grouped_gemm_ragged_k(a_t, fa, b_t, fb, offsets, ALIGN, sa, sb)
    got = gpu_ragged(fp8, a_t, fa, b_t, fb, offsets, sa, sb, out_f32)
    assert_within(orc, got, y, bound, not out_f32, f"ragged {sizes}")
    for g, sz in enumerate(sizes):
        if sz == 0:
            assert not got[g].any(), f"empty group {g} is not zero"


PERSIST = [(40, 300, 520, 1, 0, 0, 11), (20, 100, 2100, 0, 0, 0, 12), (48, 512, 520, 1, 0, 1, 13)]


@pytest.mark.parametrize("g,m,n,fa,fb,cut,seed", PERSIST, ids=["shifted_edges", "m_below_tile", "cut_groups"])
def test_grouped_gemm_ragged_k_many_tiles_parity(fp8, orc, g, m, n, fa, fb, cut, seed):
    """More tile slots than CUs (the persistent kernel, tiles dealt longest
    contraction first): skewed group sizes with empty groups and sizes on and
    off the 256 boundary; m, n off the 256 tile (edge tiles shifted back) or
    m < 256 (loads clamped). With cut, the operands end 512 columns short of
    the padded layout: the groups whose range fits are within the bound, the
    ones that would lose columns are NaN. Every output of every group checked."""
    rng = np.random.default_rng(seed)
    sizes = rng.integers(0, 700, g)
    sizes[::7] = 0
    sizes[1], sizes[2], sizes[3], sizes[4] = 3000, 256, 257, 1
    offsets = offsets_of(sizes)
    T = int(offsets[-1])
    a_t, sa, _ = orc.grouped_quantize_col(rand_bf16(T, m, seed), fa, offsets, ALIGN)
    b_t, sb, _ = orc.grouped_quantize_col(rand_bf16(T, n, seed + 1), fb, offsets, ALIGN)
    kp = (sizes + ALIGN - 1) // ALIGN * ALIGN
    starts = np.concatenate([[0], np.cumsum(kp)[:-1]])
    cut_groups = np.zeros(g, bool)
    if cut:
        width = max((T + 15) // 16 * 16, int(a_t.shape[1]) - 512)
        a_t, b_t = np.ascontiguousarray(a_t[:, :width]), np.ascontiguousarray(b_t[:, :width])
        cut_groups = (kp > 0) & (starts + kp > width)
        assert cut_groups.any() and not cut_groups.all()
    say("ragged k many tiles", g, m, n, fa, fb, "cut" if cut else "")
    got = gpu_ragged(fp8, a_t, fa, b_t, fb, offsets, sa, sb)
    full_a, _, _ = orc.grouped_quantize_col(rand_bf16(T, m, seed), fa, offsets, ALIGN)
    full_b, _, _ = orc.grouped_quantize_col(rand_bf16(T, n, seed + 1), fb, offsets, ALIGN)
    y, bound = orc.grouped_gemm_ragged_k(full_a, fa, full_b, fb, offsets, ALIGN, sa, sb)
    keep = ~cut_groups
    assert_within(orc, got[keep], y[keep], bound[keep], True, f"ragged many tiles {g} {m} {n}")
    assert np.isnan(got[cut_groups]).all(), "a cut group is not NaN"
    for e in np.flatnonzero(sizes == 0):
        assert not got[e].any(), f"empty group {e} is not zero"


def test_grouped_gemm_ragged_k_short_operands_give_nan(fp8, orc):
    """Operands narrower than the grouped layout (lda = ldb below P_G, still >=
    total_m): the groups whose padded range fits are exact within the bound,
    the group that would lose contraction columns writes NaN everywhere
    instead of a short sum."""
    sizes = [300, 10, 300]
    offsets = offsets_of(sizes)                            # P = 0, 512, 768; P_G = 1280
    m, n = 256, 264
    a_t, sa, _ = orc.grouped_quantize_col(rand_bf16(610, m, 5), 1, offsets, ALIGN)
    b_t, sb, _ = orc.grouped_quantize_col(rand_bf16(610, n, 6), 0, offsets, ALIGN)
    assert a_t.shape[1] == 1280
    y, bound = orc.grouped_gemm_ragged_k(a_t, 1, b_t, 0, offsets, ALIGN, sa, sb)
    say("ragged k short operands")
    got = gpu_ragged(fp8, np.ascontiguousarray(a_t[:, :1024]), 1, np.ascontiguousarray(b_t[:, :1024]), 0, offsets,
                     sa, sb)
    assert_within(orc, got[:2], y[:2], bound[:2], True, "groups that fit")
    assert np.isnan(got[2]).all(), "the cut group is not NaN"


def test_moe_layer_backward_composed(fp8, orc):
    """An expert layer's backward from bf16 tensors through the library only:
    dgrad dX_g = dY_g W_g (dY rowwise e5m2, W_g colwise over its rows by the
    grouped quantizer with equal groups, grouped GEMM) and wgrad dW_g = dY_g^T X_g
    (both colwise over each group's tokens, ragged-K grouped GEMM), against the
    oracle's composition of the same steps."""
    E, N, K = 5, 256, 512                                  # experts, expert rows (fwd out), hidden (fwd in)
    sizes = [130, 0, 257, 40, 300]
    offsets = offsets_of(sizes)
    T = int(offsets[-1])
    rng = np.random.default_rng(12)
    x = workloads.bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    w = workloads.bf16_bits((0.02 * rng.standard_normal((E * N, K))).astype(np.float32))
    dy = workloads.bf16_bits((1e-3 * rng.standard_normal((T, N))).astype(np.float32))
    dev = "cuda:0"
    off_t = torch.from_numpy(offsets).to(dev)
    woff = offsets_of([N] * E)
    say("moe backward composed")
    # dgrad
    dyq = torch.empty((T, N), dtype=torch.uint8, device=dev)
    dys = torch.empty(T, device=dev)
    fp8.fp8_quantize_row(dev_bf16(dy), 1, 0, dyq, dys)
    wt = torch.empty((K, E * N), dtype=torch.uint8, device=dev)
    wts, wta = torch.empty((E, K), device=dev), torch.empty((E, K), device=dev)
    fp8.fp8_grouped_quantize_col(dev_bf16(w), 0, 0, torch.from_numpy(woff).to(dev), wt, wts, wta)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    b_view = torch.as_strided(wt, (E, K, N), (N, E * N, 1))     # expert g: columns g*N .. of W^T
    fp8.fp8_grouped_gemm_scaled(dyq, 1, b_view, 0, off_t, dys, wts, dx)
    # wgrad
    L = fp8.grouped_layout_width(T, E)
    dyt = torch.zeros((N, L), dtype=torch.uint8, device=dev)
    xt = torch.zeros((K, L), dtype=torch.uint8, device=dev)
    dyts, dyta = torch.empty((E, N), device=dev), torch.empty((E, N), device=dev)
    xts, xta = torch.empty((E, K), device=dev), torch.empty((E, K), device=dev)
    fp8.fp8_grouped_quantize_col(dev_bf16(dy), 1, 0, off_t, dyt, dyts, dyta)
    fp8.fp8_grouped_quantize_col(dev_bf16(x), 0, 0, off_t, xt, xts, xta)
    dw = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    fp8.fp8_grouped_gemm_ragged_k(dyt, 1, xt, 0, off_t, T, dyts, xts, dw)
    torch.cuda.synchronize()
    # oracle composition
    odyq, odys, _ = orc.quantize_row(dy, 1)
    owt, owts, _ = orc.grouped_quantize_col(w, 0, woff, ALIGN)
    ob = np.stack([owt[:, g * N:(g + 1) * N] for g in range(E)])
    ydx, bdx = orc.grouped_gemm(odyq, 1, ob, 0, offsets, odys, owts)
    assert_codes_equal(dyq.cpu().numpy(), odyq, "dY rowwise codes")
    assert_codes_equal(wt.cpu().numpy(), owt, "W grouped colwise codes")
    assert_within(orc, dx.float().cpu().numpy().astype(np.float64), ydx, bdx, True, "dgrad")
    odyt, odyts, _ = orc.grouped_quantize_col(dy, 1, offsets, ALIGN)
    oxt, oxts, _ = orc.grouped_quantize_col(x, 0, offsets, ALIGN)
    P = odyt.shape[1]
    assert_codes_equal(dyt.cpu().numpy()[:, :P], odyt, "dY^T grouped codes")
    assert_codes_equal(xt.cpu().numpy()[:, :P], oxt, "X^T grouped codes")
    ydw, bdw = orc.grouped_gemm_ragged_k(odyt, 1, oxt, 0, offsets, ALIGN, odyts, oxts)
    assert_within(orc, dw.float().cpu().numpy().astype(np.float64), ydw, bdw, True, "wgrad")
