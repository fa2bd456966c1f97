"""Full-size parity on the workloads, in the launch configuration the
benchmark times: every quantizer output compared bit for bit with the oracle on
the whole tensor, and every GEMM output compared with the oracle's whole
product (evaluated in row blocks) within the bound
|gpu - oracle| <= 1e-3 * sa*sb*sum_k |a_ik b_jk| + 2^-8 |oracle|."""
import numpy as np
import pytest
import torch

import workloads
from helpers import assert_codes_equal, assert_f32_bits_equal, check_full, dev_bf16, dev_f32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def row_quant(fp8, x, fmt, col_amax=False):
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda:0")
    si = torch.empty(rows, device="cuda:0")
    am = torch.empty(rows, device="cuda:0")
    ca = torch.empty(cols, device="cuda:0") if col_amax else None
    fp8.fp8_quantize_row(x, fmt, 0, q, si, am, ca)
    return q, si, am, ca


def col_quant(fp8, x, fmt, ready=None):
    rows, cols = x.shape
    qt = torch.empty((cols, rows), dtype=torch.uint8, device="cuda:0")
    si = torch.empty(cols, device="cuda:0")
    ca = ready if ready is not None else torch.empty(cols, device="cuda:0")
    fp8.fp8_quantize_col(x, fmt, 0, qt, si, ca, col_amax_ready=ready is not None)
    return qt, si, ca


def sample_entries(m, n, seed, extra=4096, tile=128):
    rng = np.random.default_rng(seed)
    tm, tn = (m + tile - 1) // tile, (n + tile - 1) // tile
    ti, tj = np.meshgrid(np.arange(tm), np.arange(tn), indexing="ij")
    ii = np.minimum(ti.ravel() * tile + rng.integers(0, tile, ti.size), m - 1)
    jj = np.minimum(tj.ravel() * tile + rng.integers(0, tile, tj.size), n - 1)
    ii = np.concatenate([ii, rng.integers(0, m, extra), np.full(16, m - 1), rng.integers(0, m, 16)])
    jj = np.concatenate([jj, rng.integers(0, n, extra), rng.integers(0, n, 16), np.full(16, n - 1)])
    return ii.astype(np.int64), jj.astype(np.int64)


def check_sampled(orc, d, a, fa, b, fb, sa, sb, seed, what, a_vec=True, b_vec=True):
    m, n = d.shape
    ii, jj = sample_entries(m, n, seed)
    y, bound = orc.gemm_entries(a, fa, b, fb, sa, sb, ii, jj)
    got = d[torch.from_numpy(ii).to(d.device), torch.from_numpy(jj).to(d.device)].float().cpu().numpy()
    ok = orc.gemm_within_bound(got.astype(np.float64), y, bound, out_bf16=d.dtype == torch.bfloat16)
    if not ok.all():
        e = int(np.argmin(ok))
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} sampled outputs outside the bound; "
                             f"first ({ii[e]}, {jj[e]}): gpu {got[e]!r} oracle {y[e]!r} bound {bound[e]!r}")


def gemm(fp8, a, fa, b, fb, sa, a_mode, sb, b_mode):
    d = torch.empty((a.shape[0], b.shape[0]), dtype=torch.bfloat16, device="cuda:0")
    fp8.fp8_gemm_scaled(a, fa, b, fb, sa, a_mode, sb, b_mode, d)
    return d


def test_c1_rowwise_linear_full(fp8, orc):
    """256 x 512 x 512 with outlier rows: whole output compared."""
    w = workloads.c1()
    say("c1 quantize")
    qx, sx, ax, _ = row_quant(fp8, dev_bf16(w["x"]), 0)
    qw, sw, aw, _ = row_quant(fp8, dev_bf16(w["w"]), 0)
    oqx, osx, oax = orc.quantize_row(w["x"], 0)
    oqw, osw, oaw = orc.quantize_row(w["w"], 0)
    assert_codes_equal(qx.cpu().numpy(), oqx, "X codes")
    assert_codes_equal(qw.cpu().numpy(), oqw, "W codes")
    assert_f32_bits_equal(sx.cpu().numpy(), osx, "X scale_inv")
    assert_f32_bits_equal(sw.cpu().numpy(), osw, "W scale_inv")
    # the outlier rows get their own scale: 50x larger amax, ~50x smaller scale
    rows = w["outlier_rows"]
    assert np.all(oax[rows] > 20 * np.median(oax))
    say("c1 gemm")
    d = gemm(fp8, qx, 0, qw, 0, sx, 1, sw, 1)
    y, bound = orc.gemm(oqx, 0, oqw, 0, osx, osw)
    ok = orc.gemm_within_bound(d.float().cpu().numpy().astype(np.float64), y, bound)
    assert ok.all(), f"{int((~ok).sum())} outputs outside the bound"


def test_c2_llama_up_proj(fp8, orc):
    """8192 x 14336 x 4096: full quantizer parity, every GEMM output."""
    say("c2 generate")
    w = workloads.c2()
    say("c2 quantize")
    qx, sx, ax, _ = row_quant(fp8, dev_bf16(w["x"]), 0)
    qw, sw, aw, _ = row_quant(fp8, dev_bf16(w["w"]), 0)
    d = gemm(fp8, qx, 0, qw, 0, sx, 1, sw, 1)
    torch.cuda.synchronize()
    oqx, osx, oax = orc.quantize_row(w["x"], 0)
    assert_codes_equal(qx.cpu().numpy(), oqx, "X codes")
    assert_f32_bits_equal(sx.cpu().numpy(), osx, "X scale_inv")
    assert_f32_bits_equal(ax.cpu().numpy(), oax, "X amax")
    oqw, osw, oaw = orc.quantize_row(w["w"], 0)
    assert_codes_equal(qw.cpu().numpy(), oqw, "W codes")
    assert_f32_bits_equal(sw.cpu().numpy(), osw, "W scale_inv")
    say("c2 gemm check")
    check_full(orc, d, orc.gemm_by_rows(oqx, 0, oqw, 0, osx, osw), "c2 GEMM")


def test_c3_flux_delayed_16_steps(fp8, orc):
    """4608 x 12288 x 3072 tensorwise delayed scaling, L = 1024, algo max,
    margin 0, 16 steps of drifting activations: codes and the whole delayed
    state bit-exact at every step; every GEMM output at the first and last
    steps and at the first saturating step, sampled outputs at the others."""
    w = workloads.c3()
    L, algo, margin, fmt = 1024, 1, 0, 0
    hist = torch.zeros((2, L), device="cuda:0")
    head = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    scale = torch.ones(2, device="cuda:0")
    scale_inv = torch.ones(2, device="cuda:0")
    cur = torch.zeros(2, device="cuda:0")
    st = orc.DelayedState(2, L)
    wd = dev_bf16(w["w"])
    n, k = w["w"].shape
    qw = torch.empty((n, k), dtype=torch.uint8, device="cuda:0")
    siw = torch.empty(1, device="cuda:0")
    saturated_steps = 0
    for t, (c, xb) in enumerate(w["x_steps"]()):
        say("c3 step", t, "c_t", c)
        m = xb.shape[0]
        xd = dev_bf16(xb)
        qx = torch.empty((m, k), dtype=torch.uint8, device="cuda:0")
        six = torch.empty(1, device="cuda:0")
        fp8.fp8_quantize_tensor_batch([xd, wd], fmt, [scale[0:1], scale[1:2]], [qx, qw], [six, siw],
                                      [cur[0:1], cur[1:2]])
        d = torch.empty((m, n), dtype=torch.bfloat16, device="cuda:0")
        fp8.fp8_gemm_scaled(qx, fmt, qw, fmt, six, 0, siw, 0, d)
        cur_before = cur.clone()
        fp8.fp8_delayed_scale_update(cur, hist, head, algo, margin, fmt, scale, scale_inv)
        torch.cuda.synchronize()
        # oracle step: cast with the scales in force, record amax, update
        oqx, osix, oamx = orc.quantize_tensor_scaled(xb, fmt, st.scale[0])
        oqw, osiw, oamw = orc.quantize_tensor_scaled(w["w"], fmt, st.scale[1])
        assert_codes_equal(qx.cpu().numpy(), oqx, f"X codes step {t}")
        assert_codes_equal(qw.cpu().numpy(), oqw, f"W codes step {t}")
        assert_f32_bits_equal(six.cpu().numpy(), [osix], "X scale_inv used")
        assert_f32_bits_equal(cur_before.cpu().numpy(), [oamx, oamw], f"amax step {t}")
        saturates = (np.abs(orc.decode(fmt, oqx[:64])) == 448.0).mean() > 1e-3
        if t in (0, 15) or (saturates and saturated_steps == 0):
            check_full(orc, d, orc.gemm_by_rows(oqx, fmt, oqw, fmt, np.float32([osix]), np.float32([osiw])),
                       f"c3 GEMM step {t}")
        else:
            check_sampled(orc, d, oqx, fmt, oqw, fmt, np.float32([osix]), np.float32([osiw]), seed=t,
                          what=f"c3 GEMM step {t}")
        saturated_steps += int(saturates)
        st.cur_amax[:] = [oamx, oamw]
        st.update(algo, margin, fmt)
        assert_f32_bits_equal(scale.cpu().numpy(), st.scale, f"scale step {t}")
        assert_f32_bits_equal(scale_inv.cpu().numpy(), st.scale_inv, f"scale_inv step {t}")
        assert_f32_bits_equal(hist.cpu().numpy(), st.history, f"history step {t}")
        assert head.item() == st.head[0]
    assert saturated_steps >= 1, "growth steps saturate by design"


def test_c4_moe_grouped(fp8, orc):
    """32 experts, 16384 tokens (Zipf counts, three experts empty), N = 2048,
    K = 7168: tokens and expert weights cast in one batched launch (587 MB of
    codes, stored nontemporally), full quantizer parity, every output of the
    grouped GEMM against each expert's product."""
    say("c4 generate")
    w = workloads.c4()
    offsets = w["offsets"]
    g, n, k = w["w"].shape
    assert (w["counts"] == 0).sum() >= 3
    say("c4 quantize (one batched launch)")
    T = int(offsets[-1])
    wflat = w["w"].reshape(g * n, k)
    qx = torch.empty((T, k), dtype=torch.uint8, device="cuda:0")
    qw = torch.empty((g * n, k), dtype=torch.uint8, device="cuda:0")
    sx = torch.empty(T, device="cuda:0")
    sw = torch.empty(g * n, device="cuda:0")
    fp8.fp8_quantize_row_batch([dev_bf16(w["x"]), dev_bf16(wflat)], 0, 0, [qx, qw], [sx, sw])
    d = torch.empty((offsets[-1], n), dtype=torch.bfloat16, device="cuda:0")
    fp8.fp8_grouped_gemm_scaled(qx, 0, qw.view(g, n, k), 0, torch.from_numpy(offsets).to("cuda:0"), sx,
                                sw.view(g, n), d)
    torch.cuda.synchronize()
    oqx, osx, _ = orc.quantize_row(w["x"], 0)
    assert_codes_equal(qx.cpu().numpy(), oqx, "token codes")
    assert_f32_bits_equal(sx.cpu().numpy(), osx, "token scale_inv")
    oqw, osw, _ = orc.quantize_row(wflat, 0)
    assert_codes_equal(qw.cpu().numpy(), oqw, "expert weight codes")
    assert_f32_bits_equal(sw.cpu().numpy(), osw, "expert weight scale_inv")
    say("c4 grouped gemm check")
    d = d.float().cpu().numpy()
    rows = 0
    for e in range(g):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows += check_full(orc, d, orc.gemm_by_rows(oqx[lo:hi], 0, oqw[e * n:(e + 1) * n], 0, osx[lo:hi],
                                                        osw[e * n:(e + 1) * n]), f"c4 expert {e}", row_offset=lo)
    assert rows == T


def test_c4b_moe_backward(fp8, orc):
    """The c4 expert layer's backward in the benchmark's launch configuration:
    the forward's rowwise cast of X and W leaves their per-group column amax
    (token groups; each expert's weight rows) as side outputs, dY [16384 x
    2048] is cast rowwise e5m2 with its per-expert column amax likewise; W^T,
    dY^T and X^T through the grouped colwise cast with those amax ready
    (per-expert column scales, transposed into the 256-padded grouped layout);
    dgrad dX_g = dY_g W_g as a grouped e5m2 x e4m3 product
    over a strided view of W^T, wgrad dW_g = dY_g^T X_g as the ragged-K
    product (the persistent kernel at this size). Every code and scale, every
    output of both products."""
    say("c4b generate")
    w = workloads.c4b()
    offsets = w["offsets"]
    g, n, k = w["w"].shape
    T = int(offsets[-1])
    L = fp8.grouped_layout_width(T, g)
    wflat = w["w"].reshape(g * n, k)
    woff = np.arange(g + 1, dtype=np.int64) * n
    off_d = torch.from_numpy(offsets).to("cuda:0")
    woff_d = torch.from_numpy(woff).to("cuda:0")
    xd, wd, dyd = dev_bf16(w["x"]), dev_bf16(wflat), dev_bf16(w["dy"])
    say("c4b forward cast (per-group column amax side outputs)")
    qx, qw = torch.empty((T, k), dtype=torch.uint8, device="cuda:0"), torch.empty((g * n, k), dtype=torch.uint8,
                                                                                  device="cuda:0")
    sx, sw = torch.empty(T, device="cuda:0"), torch.empty(g * n, device="cuda:0")
    xta, wta = torch.empty((g, k), device="cuda:0"), torch.empty((g, k), device="cuda:0")
    fp8.fp8_quantize_row_batch([xd, wd], 0, 0, [qx, qw], [sx, sw], None, [xta, wta], [off_d, woff_d])
    say("c4b quantize")
    dyq, dys = torch.empty((T, n), dtype=torch.uint8, device="cuda:0"), torch.empty(T, device="cuda:0")
    dyta = torch.empty((g, n), device="cuda:0")
    fp8.fp8_quantize_row_batch([dyd], 1, 0, [dyq], [dys], None, [dyta], [off_d])
    wt = torch.empty((k, g * n), dtype=torch.uint8, device="cuda:0")
    wts = torch.empty((g, k), device="cuda:0")
    fp8.fp8_grouped_quantize_col(wd, 0, 0, woff_d, wt, wts, wta, col_amax_ready=True)
    dyt = torch.zeros((n, L), dtype=torch.uint8, device="cuda:0")
    dyts = torch.empty((g, n), device="cuda:0")
    fp8.fp8_grouped_quantize_col(dyd, 1, 0, off_d, dyt, dyts, dyta, col_amax_ready=True)
    xt = torch.zeros((k, L), dtype=torch.uint8, device="cuda:0")
    xts = torch.empty((g, k), device="cuda:0")
    fp8.fp8_grouped_quantize_col(xd, 0, 0, off_d, xt, xts, xta, col_amax_ready=True)
    dx = torch.empty((T, k), dtype=torch.bfloat16, device="cuda:0")
    fp8.fp8_grouped_gemm_scaled(dyq, 1, torch.as_strided(wt, (g, k, n), (n, g * n, 1)), 0, off_d, dys, wts, dx)
    dw = torch.empty((g, n, k), dtype=torch.bfloat16, device="cuda:0")
    fp8.fp8_grouped_gemm_ragged_k(dyt, 1, xt, 0, off_d, T, dyts, xts, dw)
    torch.cuda.synchronize()
    say("c4b oracle quantize")
    oqx, osx, _ = orc.quantize_row(w["x"], 0)
    assert_codes_equal(qx.cpu().numpy(), oqx, "forward X codes")
    assert_f32_bits_equal(sx.cpu().numpy(), osx, "forward X scale_inv")
    del oqx, qx
    oqw, osw, _ = orc.quantize_row(wflat, 0)
    assert_codes_equal(qw.cpu().numpy(), oqw, "forward W codes")
    assert_f32_bits_equal(sw.cpu().numpy(), osw, "forward W scale_inv")
    del oqw, qw
    oqdy, osdy, _ = orc.quantize_row(w["dy"], 1)
    assert_codes_equal(dyq.cpu().numpy(), oqdy, "dY codes")
    assert_f32_bits_equal(dys.cpu().numpy(), osdy, "dY scale_inv")
    oqwt, oswt, oawt = orc.grouped_quantize_col(wflat, 0, woff, 256)
    assert_codes_equal(wt.cpu().numpy(), oqwt, "W^T codes")
    assert_f32_bits_equal(wts.cpu().numpy(), oswt, "W^T scale_inv")
    assert_f32_bits_equal(wta.cpu().numpy(), oawt, "W per-expert column amax (forward side output)")
    oqdyt, osdyt, oadyt = orc.grouped_quantize_col(w["dy"], 1, offsets, 256)
    assert oqdyt.shape[1] <= L
    assert_codes_equal(dyt.cpu().numpy()[:, :oqdyt.shape[1]], oqdyt, "dY^T codes")
    assert_f32_bits_equal(dyts.cpu().numpy(), osdyt, "dY^T scale_inv")
    assert_f32_bits_equal(dyta.cpu().numpy(), oadyt, "dY per-expert column amax (row cast side output)")
    oqxt, osxt, oaxt = orc.grouped_quantize_col(w["x"], 0, offsets, 256)
    assert_codes_equal(xt.cpu().numpy()[:, :oqxt.shape[1]], oqxt, "X^T codes")
    assert_f32_bits_equal(xts.cpu().numpy(), osxt, "X^T scale_inv")
    assert_f32_bits_equal(xta.cpu().numpy(), oaxt, "X per-expert column amax (forward side output)")
    say("c4b dgrad check")
    dxh = dx.float().cpu().numpy()
    rows = 0
    for e in range(g):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            bt = np.ascontiguousarray(oqwt[:, e * n:(e + 1) * n])          # W_e^T rows: [k x n]
            rows += check_full(orc, dxh, orc.gemm_by_rows(oqdy[lo:hi], 1, bt, 0, osdy[lo:hi], oswt[e]),
                               f"c4b dgrad expert {e}", row_offset=lo)
    assert rows == T
    say("c4b wgrad check")
    P = np.concatenate([[0], np.cumsum((np.diff(offsets) + 255) // 256 * 256)])
    for e in range(g):
        if P[e + 1] > P[e]:
            at = np.ascontiguousarray(oqdyt[:, P[e]:P[e + 1]])
            bt = np.ascontiguousarray(oqxt[:, P[e]:P[e + 1]])
            check_full(orc, dw[e], orc.gemm_by_rows(at, 1, bt, 0, osdyt[e], osxt[e]), f"c4b wgrad expert {e}")
        else:
            assert not dw[e].any().item(), f"empty expert {e}: dW is not zero"


def test_c5_hybrid_backward(fp8, orc):
    """In the benchmark's launch configuration: dY [8192 x 14336] through the
    dual cast (e5m2 rowwise codes and colwise-transposed codes in two passes),
    X and W cast rowwise with their column-amax side outputs (the forward), then
    W^T / X^T colwise-transposed with those amax (e4m3); dgrad dX = dY W and
    wgrad dW = dY^T X as e5m2 x e4m3 GEMMs. Every code, scale and amax and every
    GEMM output compared."""
    say("c5 generate")
    w = workloads.c5()
    xd, wd, dyd = dev_bf16(w["x"]), dev_bf16(w["w"]), dev_bf16(w["dy"])
    m, k = w["x"].shape
    n = w["w"].shape[0]
    say("c5 quantize")
    qdy, sdy, ady = torch.empty((m, n), dtype=torch.uint8, device="cuda:0"), torch.empty(m, device="cuda:0"), \
        torch.empty(m, device="cuda:0")
    qdyt, sdyt, ca_dy = torch.empty((n, m), dtype=torch.uint8, device="cuda:0"), torch.empty(n, device="cuda:0"), \
        torch.empty(n, device="cuda:0")
    fp8.fp8_quantize_rowcol(dyd, 1, 0, qdy, sdy, ady, qdyt, sdyt, ca_dy)
    cax, caw = torch.empty(k, device="cuda:0"), torch.empty(k, device="cuda:0")
    fwd = [torch.empty((m, k), dtype=torch.uint8, device="cuda:0"), torch.empty((n, k), dtype=torch.uint8, device="cuda:0")]
    fp8.fp8_quantize_row_batch([xd, wd], 0, 0, fwd, [torch.empty(m, device="cuda:0"), torch.empty(n, device="cuda:0")],
                               None, [cax, caw])
    qwt, swt, _ = col_quant(fp8, wd, 0, ready=caw)
    qxt, sxt, _ = col_quant(fp8, xd, 0, ready=cax)
    dx = gemm(fp8, qdy, 1, qwt, 0, sdy, 1, swt, 1)       # [8192 x 4096]
    dw = gemm(fp8, qdyt, 1, qxt, 0, sdyt, 1, sxt, 1)     # [14336 x 4096]
    torch.cuda.synchronize()
    say("c5 oracle quantize")
    oqdy, osdy, _ = orc.quantize_row(w["dy"], 1)
    assert_codes_equal(qdy.cpu().numpy(), oqdy, "dY row codes")
    assert_f32_bits_equal(sdy.cpu().numpy(), osdy, "dY row scale_inv")
    oqdyt, osdyt, oady = orc.quantize_col(w["dy"], 1)
    assert_f32_bits_equal(ca_dy.cpu().numpy(), oady, "dY col amax")
    assert_f32_bits_equal(ady.cpu().numpy(), orc.amax(w["dy"], orc.AXIS_ROW), "dY row amax")
    assert_codes_equal(qdyt.cpu().numpy(), oqdyt, "dY^T codes")
    assert_f32_bits_equal(sdyt.cpu().numpy(), osdyt, "dY^T scale_inv")
    oqwt, oswt, oaw = orc.quantize_col(w["w"], 0)
    assert_f32_bits_equal(caw.cpu().numpy(), oaw, "W col amax (forward side output)")
    assert_codes_equal(qwt.cpu().numpy(), oqwt, "W^T codes")
    assert_f32_bits_equal(swt.cpu().numpy(), oswt, "W^T scale_inv")
    oqxt, osxt, oax = orc.quantize_col(w["x"], 0)
    assert_f32_bits_equal(cax.cpu().numpy(), oax, "X col amax (forward side output)")
    assert_codes_equal(qxt.cpu().numpy(), oqxt, "X^T codes")
    assert_f32_bits_equal(sxt.cpu().numpy(), osxt, "X^T scale_inv")
    say("c5 gemm check")
    check_full(orc, dx, orc.gemm_by_rows(oqdy, 1, oqwt, 0, osdy, oswt), "dgrad")
    check_full(orc, dw, orc.gemm_by_rows(oqdyt, 1, oqxt, 0, osdyt, osxt), "wgrad")


def test_c4mx_moe_grouped_mx(fp8, orc):
    """The c4 tensors with MXFP8: tokens and expert weights through the MX
    quantizer (codes and scale records bit-exact on the whole tensors), every
    output of the grouped MX product, in the bench's launch configuration (expert
    weight records as a strided view of the stacked records)."""
    say("c4mx generate")
    w = workloads.c4()
    offsets = w["offsets"]
    g, n, k = w["w"].shape
    T = int(offsets[-1])
    wflat = w["w"].reshape(g * n, k)
    say("c4mx quantize")
    qx = torch.empty((T, k), dtype=torch.uint8, device="cuda:0")
    sx = fp8.mx_scale_records(T, k)
    qw = torch.empty((g * n, k), dtype=torch.uint8, device="cuda:0")
    sw = fp8.mx_scale_records(g * n, k)
    fp8.fp8_mx_quantize_row(dev_bf16(w["x"]), 0, qx, sx)
    fp8.fp8_mx_quantize_row(dev_bf16(wflat), 0, qw, sw)
    d = torch.empty((T, n), dtype=torch.bfloat16, device="cuda:0")
    swv = torch.as_strided(sw, (g, k // 128, n, 4), (4 * n, 4 * g * n, 4, 1))
    fp8.fp8_grouped_gemm_mx(qx, 0, sx, qw.view(g, n, k), 0, swv, torch.from_numpy(offsets).to("cuda:0"), d)
    torch.cuda.synchronize()
    oqx, osx = orc.mx_quantize_row(w["x"], 0)
    assert_codes_equal(qx.cpu().numpy(), oqx, "token codes")
    rec = lambda s: np.ascontiguousarray(s.reshape(s.shape[0], -1, 4).transpose(1, 0, 2))
    assert_codes_equal(sx.cpu().numpy(), rec(osx), "token scale records")
    oqw, osw = orc.mx_quantize_row(wflat, 0)
    assert_codes_equal(qw.cpu().numpy(), oqw, "expert weight codes")
    assert_codes_equal(sw.cpu().numpy(), rec(osw), "expert weight scale records")
    say("c4mx grouped gemm check")
    d = d.float().cpu().numpy()
    rows = 0
    for e in range(g):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            rows += check_full(orc, d, orc.mx_gemm_by_rows(oqx[lo:hi], 0, osx[lo:hi], oqw[e * n:(e + 1) * n], 0,
                                                           osw[e * n:(e + 1) * n]), f"c4mx expert {e}", row_offset=lo)
    assert rows == T
