"""GPU parity of the amax, quantizer and delayed-update kernels against the CPU
oracle, through the C ABI. Codes, scales, amax and the delayed state must be
bit-identical (the cast has a unique result)."""
import numpy as np
import pytest
import torch

import workloads
from helpers import (assert_codes_equal, assert_f32_bits_equal, check_guard, dev_bf16, dev_f32, guarded,
                     host_bits, say)

pytestmark = pytest.mark.gpu

FORMATS = [0, 1, 2, 3]
NAMES = {0: "e4m3", 1: "e5m2", 2: "e4m3fnuz", 3: "e5m2fnuz"}


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def rand_bf16(rows, cols, seed, spread=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-spread, spread + 1, size=(rows, 1))).astype(np.float32)
    return workloads.bf16_bits(x)


def gpu_row(fp8, xb, fmt, margin=0, ldq=None, col_amax=False):
    x = dev_bf16(xb)
    rows, cols = xb.shape
    q, qbuf, org = guarded(rows, cols, torch.uint8, ld=ldq)
    si = torch.full((rows,), -1.0, device="cuda:0")
    am = torch.full((rows,), -1.0, device="cuda:0")
    ca = torch.full((cols,), -1.0, device="cuda:0") if col_amax else None
    fp8.fp8_quantize_row(x, fmt, margin, q, si, am, ca)
    torch.cuda.synchronize()
    check_guard(qbuf, org, rows, cols)
    return q.cpu().numpy(), si.cpu().numpy(), am.cpu().numpy(), (ca.cpu().numpy() if col_amax else None)


def gpu_col(fp8, xb, fmt, margin=0, ldqt=None, ready=None, transpose=True):
    x = dev_bf16(xb)
    rows, cols = xb.shape
    qr, qc = (cols, rows) if transpose else (rows, cols)
    qt, qbuf, org = guarded(qr, qc, torch.uint8, ld=ldqt)
    si = torch.full((cols,), -1.0, device="cuda:0")
    ca = dev_f32(ready) if ready is not None else torch.full((cols,), -1.0, device="cuda:0")
    fp8.fp8_quantize_col(x, fmt, margin, qt, si, ca, col_amax_ready=ready is not None, transpose_out=transpose)
    torch.cuda.synchronize()
    check_guard(qbuf, org, qr, qc)
    return qt.cpu().numpy(), si.cpu().numpy(), ca.cpu().numpy()


# ------------------------------------------------------------------- the cast --

@pytest.mark.parametrize("fmt", FORMATS)
def test_cast_every_bf16_value_times_scales(fp8, orc, fmt):
    """All 65536 bf16 values (NaN, Inf, subnormals, both zeros, every tie
    between FP8 neighbours) cast with a range of scales, through the tensorwise
    quantizer with a given (delayed) scale."""
    xb = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    x = dev_bf16(xb)
    rng = np.random.default_rng(fmt)
    scales = [1.0, 2.0 ** -7, 2.0 ** 9, 0.75, 1.0 / 3.0, 3.0e-5, 1.0e5, float(np.float32(448.0 / 3.0)),
              float(np.float32(0.6)), 1.2e-38] + rng.uniform(0.01, 100.0, 6).tolist()
    for s in scales:
        s32 = np.float32(s)
        say("cast", NAMES[fmt], "scale", float(s32))
        q = torch.empty((256, 256), dtype=torch.uint8, device="cuda:0")
        si = torch.empty(1, device="cuda:0")
        am = torch.zeros(1, device="cuda:0")
        fp8.fp8_quantize_tensor(x, fmt, 0, dev_f32([s32]), q, si, am)
        torch.cuda.synchronize()
        oq, osi, oam = orc.quantize_tensor_scaled(xb, fmt, s32)
        assert_codes_equal(q.cpu().numpy(), oq, f"{NAMES[fmt]} s={s32}")
        assert_f32_bits_equal(si.cpu().numpy(), [osi], "scale_inv")
        assert_f32_bits_equal(am.cpu().numpy(), [oam], "amax")


@pytest.mark.parametrize("fmt", FORMATS)
def test_cast_products_next_to_every_tie(fp8, orc, fmt):
    """The hardware-convert path at the rounding boundaries: every FP8 tie
    (the midpoint of two neighbouring codes, in every binade and between
    subnormals) is a bf16 value, so with s = 1 + j 2^-23 and s = 1 - j 2^-24
    (j = 1..8) the fp32 products x s of all 65536 bf16 values x fall 1 to 16
    fp32 ulps above and below each tie, and with s = 1 exactly on it. Also the
    product-rounding witness s = 0x3F86F21C, for which fl32(1.0078125 s) is the
    tie 1.0625 exactly while the exact product lies above it (e4m3: 0x38, the
    even neighbour, only if the product is rounded to fp32 first)."""
    xb = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    x = dev_bf16(xb)
    scales = [np.float32(1.0)]
    for j in range(1, 9):
        scales += [np.float32(1.0 + j * 2.0 ** -23), np.float32(1.0 - j * 2.0 ** -24)]
    witness = np.array([0x3F86F21C], np.uint32).view(np.float32)[0]
    scales.append(witness)
    for s32 in scales:
        say("cast near ties", NAMES[fmt], "scale bits", hex(int(np.float32(s32).view(np.uint32))))
        q = torch.empty((256, 256), dtype=torch.uint8, device="cuda:0")
        si = torch.empty(1, device="cuda:0")
        am = torch.zeros(1, device="cuda:0")
        fp8.fp8_quantize_tensor(x, fmt, 0, dev_f32([s32]), q, si, am)
        torch.cuda.synchronize()
        oq, osi, _ = orc.quantize_tensor_scaled(xb, fmt, s32)
        got = q.cpu().numpy()
        assert_codes_equal(got, oq, f"{NAMES[fmt]} s=0x{int(np.float32(s32).view(np.uint32)):08X}")
        assert_f32_bits_equal(si.cpu().numpy(), [osi], "scale_inv")
    if fmt == 0:
        assert got[0x3F81 >> 8, 0x3F81 & 0xFF] == 0x38


# ----------------------------------------------------------------------- rows --

ROW_SHAPES = [(1, 16), (3, 48), (37, 200), (256, 512), (300, 4104), (64, 14336), (9, 16392), (5, 0)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", ROW_SHAPES)
def test_quantize_row_parity(fp8, orc, fmt, shape):
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=rows * 7 + cols)
    for margin in (0, 1, 2) if rows * cols < 2e5 else (0,):
        say("row", NAMES[fmt], shape, "margin", margin)
        q, si, am, _ = gpu_row(fp8, xb, fmt, margin)
        oq, osi, oam = orc.quantize_row(xb, fmt, margin)
        assert_codes_equal(q, oq, f"codes {shape}")
        assert_f32_bits_equal(si, osi, "scale_inv")
        assert_f32_bits_equal(am, oam, "amax")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(5, 37), (33, 203), (2, 1)])
def test_quantize_row_unaligned_layouts(fp8, orc, fmt, shape):
    """Widths that are not a multiple of 8 and a padded output stride take the
    scalar kernels."""
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=3)
    say("row scalar", NAMES[fmt], shape)
    q, si, am, _ = gpu_row(fp8, xb, fmt, 1, ldq=cols + 3)
    oq, osi, oam = orc.quantize_row(xb, fmt, 1)
    assert_codes_equal(q, oq, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(am, oam, "amax")


def special_rows():
    """Rows of zeros, NaN, +-Inf, bf16 subnormals, a single nonzero, huge and tiny values."""
    f = np.float32
    rows = [
        [0.0] * 16,
        [-0.0] * 8 + [0.0] * 8,
        [1.0, np.nan] + [2.0] * 14,
        [np.inf, -1.0] + [0.5] * 14,
        [-np.inf] + [0.0] * 15,
        [1e-40, -3e-41, 9e-39, 0.0] * 4,                     # bf16 subnormals
        [0.0] * 15 + [-7.0],
        [3.0e38, -1.0, 1.0, 2.0] * 4,
        [2.0 ** -133] + [0.0] * 15,                          # smallest bf16 subnormal: s overflows to FLT_MAX
        [448.0, 464.0, 480.0, 57344.0, 61440.0, -240.0, -232.0, 0.001] * 2,
    ]
    return workloads.bf16_bits(np.array(rows, dtype=f))


@pytest.mark.parametrize("fmt", FORMATS)
def test_quantize_row_special_values(fp8, orc, fmt):
    xb = special_rows()
    for margin in (0, 2):
        say("row specials", NAMES[fmt], margin)
        q, si, am, ca = gpu_row(fp8, xb, fmt, margin, col_amax=True)
        oq, osi, oam = orc.quantize_row(xb, fmt, margin)
        assert_codes_equal(q, oq, "codes")
        assert_f32_bits_equal(si, osi, "scale_inv")
        assert_f32_bits_equal(am, oam, "amax")
        assert_f32_bits_equal(ca, orc.amax(xb, orc.AXIS_COL), "col amax side output")


@pytest.mark.parametrize("shape", [(256, 512), (130, 72), (1, 8)])
def test_quantize_row_col_amax_side_output(fp8, orc, shape):
    xb = rand_bf16(*shape, seed=11)
    say("row + col amax", shape)
    q, si, am, ca = gpu_row(fp8, xb, 0, 0, col_amax=True)
    assert_f32_bits_equal(ca, orc.amax(xb, orc.AXIS_COL), "col amax")
    assert_codes_equal(q, orc.quantize_row(xb, 0)[0], "codes")


# -------------------------------------------------------------------- columns --

COL_SHAPES = [(1, 8), (128, 64), (130, 72), (257, 136), (1000, 520), (64, 4104), (3, 48)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(1, 8), (128, 64), (130, 72), (300, 1032), (1000, 520), (2100, 4104)])
def test_quantize_rowcol_parity(fp8, orc, fmt, shape):
    """Dual cast: rowwise codes and colwise-transposed codes of one tensor, as
    fp8_quantize_row and fp8_quantize_col give them (oracle), with ragged
    tiles, a NaN row and column, an Inf, an all-zero row and column, padded
    output strides and guard bands around both outputs."""
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=rows + 5 * cols)
    if rows > 3 and cols > 3:
        xb[1, 2] = 0x7FC0                                # NaN: row 1 and column 2
        xb[2, 3] = 0xFF80                                # -Inf: row 2 and column 3
        xb[3, :] = 0
        xb[:, 1] = 0x8000                                # a column of -0
    x = dev_bf16(xb)
    q, qbuf, qorg = guarded(rows, cols, torch.uint8, ld=cols + 8)
    qt, tbuf, torg = guarded(cols, rows, torch.uint8, ld=rows + 16 - rows % 16)
    si, am = torch.full((rows,), -1.0, device="cuda:0"), torch.full((rows,), -1.0, device="cuda:0")
    sc, ca = torch.full((cols,), -1.0, device="cuda:0"), torch.full((cols,), -1.0, device="cuda:0")
    say("rowcol", NAMES[fmt], shape)
    fp8.fp8_quantize_rowcol(x, fmt, 1, q, si, am, qt, sc, ca)
    torch.cuda.synchronize()
    check_guard(qbuf, qorg, rows, cols)
    check_guard(tbuf, torg, cols, rows)
    oq, osi, oam = orc.quantize_row(xb, fmt, 1)
    oqt, osc, oca = orc.quantize_col(xb, fmt, 1)
    assert_codes_equal(q.cpu().numpy(), oq, "row codes")
    assert_f32_bits_equal(si.cpu().numpy(), osi, "row scale_inv")
    assert_f32_bits_equal(am.cpu().numpy(), oam, "row amax")
    assert_codes_equal(qt.cpu().numpy(), oqt, "column codes")
    assert_f32_bits_equal(sc.cpu().numpy(), osc, "column scale_inv")
    assert_f32_bits_equal(ca.cpu().numpy(), oca, "column amax")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(1, 8), (300, 520), (257, 1032), (70, 37), (5, 3)])
def test_quantize_col_untransposed_parity(fp8, orc, fmt, shape):
    """transpose_out = 0: column scales with the codes in x's own layout (the
    oracle's transposed codes, transposed back), vector and scalar layouts,
    a padded output stride, a NaN column and an all-zero column."""
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=rows * 3 + cols)
    if rows > 2 and cols > 2:
        xb[rows // 2, 1] = 0x7FC0
        xb[:, 2] = 0
    for ready in (False, True):
        say("col untransposed", NAMES[fmt], shape, "ready", ready)
        oqt, osi, oam = orc.quantize_col(xb, fmt, 1)
        q, si, ca = gpu_col(fp8, xb, fmt, margin=1, ldqt=cols + 24, ready=oam if ready else None, transpose=False)
        assert_codes_equal(q, np.ascontiguousarray(oqt.T), f"codes {shape}")
        assert_f32_bits_equal(si, osi, "scale_inv")
        assert_f32_bits_equal(ca, oam, "col amax")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", COL_SHAPES)
def test_quantize_col_parity(fp8, orc, fmt, shape):
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=rows + 13 * cols)
    say("col", NAMES[fmt], shape)
    qt, si, ca = gpu_col(fp8, xb, fmt, margin=1)
    oqt, osi, oam = orc.quantize_col(xb, fmt, 1)
    assert_codes_equal(qt, oqt, f"codes {shape}")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(ca, oam, "col amax")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("shape,ldqt", [((130, 72), 136), ((100, 40), 103), ((33, 37), None), ((17, 3), None)])
def test_quantize_col_layouts(fp8, orc, fmt, shape, ldqt):
    """Output strides that break 16-byte stores, and widths off the 8-column
    grid (scalar kernel)."""
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=5)
    say("col layout", NAMES[fmt], shape, ldqt)
    qt, si, ca = gpu_col(fp8, xb, fmt, ldqt=ldqt)
    oqt, osi, oam = orc.quantize_col(xb, fmt, 0)
    assert_codes_equal(qt, oqt, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")


def test_quantize_col_over_65535_row_tiles(fp8, orc):
    """More row tiles of 128 than one launch's grid y holds (65535): the cast
    takes a second launch for the rows past 65535 * 128."""
    rows, cols = 65535 * 128 + 200, 16
    xb = rand_bf16(rows, cols, seed=23)
    say("col over 65535 row tiles", rows, cols)
    qt, si, ca = gpu_col(fp8, xb, 0, margin=1)
    oqt, osi, oam = orc.quantize_col(xb, 0, 1)
    assert_codes_equal(qt, oqt, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(ca, oam, "col amax")


def test_quantize_col_with_ready_amax(fp8, orc):
    xb = rand_bf16(300, 136, seed=9)
    ready = orc.amax(xb, orc.AXIS_COL)
    say("col ready amax")
    qt, si, ca = gpu_col(fp8, xb, 1, ready=ready)
    oqt, osi, _ = orc.quantize_col(xb, 1, 0)
    assert_codes_equal(qt, oqt, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")


def test_quantize_col_special_values(fp8, orc):
    xb = np.ascontiguousarray(special_rows().T)      # specials down the columns
    for fmt in FORMATS:
        say("col specials", NAMES[fmt])
        qt, si, ca = gpu_col(fp8, xb, fmt)
        oqt, osi, oam = orc.quantize_col(xb, fmt, 0)
        assert_codes_equal(qt, oqt, "codes")
        assert_f32_bits_equal(si, osi, "scale_inv")
        assert_f32_bits_equal(ca, oam, "amax")


# ----------------------------------------------------------------------- amax --

@pytest.mark.parametrize("shape", [(1, 8), (37, 200), (513, 1032), (7, 13), (0, 16), (16, 0)])
def test_amax_all_axes(fp8, orc, shape):
    xb = rand_bf16(*shape, seed=17) if shape[0] * shape[1] else np.zeros(shape, np.uint16)
    if xb.size:
        xb[shape[0] // 2, shape[1] // 3] = workloads.bf16_bits(np.float32([-1e30]))[0]
    x = dev_bf16(xb) if xb.size else torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
    for axis, n in ((0, 1), (1, shape[0]), (2, shape[1])):
        say("amax", shape, "axis", axis)
        out = torch.full((max(n, 1),), -1.0, device="cuda:0")
        fp8.fp8_amax(x, axis, out)
        torch.cuda.synchronize()
        want = orc.amax(xb, axis) if xb.size else np.zeros(n, np.float32)
        assert_f32_bits_equal(out.cpu().numpy()[:n], want, f"axis {axis}")


# ----------------------------------------------------------------- tensorwise --

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", [(37, 200), (300, 4104), (5, 37)])
def test_quantize_tensor_current(fp8, orc, fmt, shape):
    xb = rand_bf16(*shape, seed=23)
    x = dev_bf16(xb)
    say("tensor current", NAMES[fmt], shape)
    q = torch.empty(shape, dtype=torch.uint8, device="cuda:0")
    si = torch.empty(1, device="cuda:0")
    am = torch.full((1,), 123.0, device="cuda:0")      # overwritten in current mode
    fp8.fp8_quantize_tensor(x, fmt, 1, None, q, si, am)
    torch.cuda.synchronize()
    oq, osi, oam = orc.quantize_tensor_current(xb, fmt, 1)
    assert_codes_equal(q.cpu().numpy(), oq, "codes")
    assert_f32_bits_equal(si.cpu().numpy(), [osi], "scale_inv")
    assert_f32_bits_equal(am.cpu().numpy(), [oam], "amax")


@pytest.mark.parametrize("shape", [(1, 8), (7, 1024), (64, 16384), (3, 24000), (4096, 1032)])
def test_quantize_tensor_current_row_lengths(fp8, orc, shape):
    """Every register-resident row length (1 .. 32 chunks of 8 per lane), rows
    longer than that (strided fallback) and a tensor of many workgroups, whose
    amax is combined across workgroups; the largest magnitude sits in the last row."""
    xb = rand_bf16(*shape, seed=41)
    xb[-1, shape[1] // 2] = workloads.bf16_bits(np.float32([-7e4]))[0]
    x = dev_bf16(xb)
    say("tensor current row lengths", shape)
    q = torch.empty(shape, dtype=torch.uint8, device="cuda:0")
    si = torch.empty(1, device="cuda:0")
    am = torch.full((1,), 123.0, device="cuda:0")
    fp8.fp8_quantize_tensor(x, 0, 0, None, q, si, am)
    torch.cuda.synchronize()
    oq, osi, oam = orc.quantize_tensor_current(xb, 0, 0)
    assert_codes_equal(q.cpu().numpy(), oq, "codes")
    assert_f32_bits_equal(si.cpu().numpy(), [osi], "scale_inv")
    assert_f32_bits_equal(am.cpu().numpy(), [oam], "amax")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("shape", [(300, 4104), (2048, 512), (3, 24000), (37, 200)])
def test_quantize_tensor_delayed_parity(fp8, orc, fmt, shape):
    """Delayed (given-scale) cast of tensors with a NaN row and an Inf: codes,
    scale_inv and the amax folded into the running value, twice in a row (the
    second call folds into the first call's amax)."""
    xb = rand_bf16(*shape, seed=43)
    xb[1, 3] = 0x7FC1                                   # NaN (positive, payload)
    xb[-1, 0] = 0xFF80                                  # -Inf
    x = dev_bf16(xb)
    scale = np.float32(0.75)
    q = torch.empty(shape, dtype=torch.uint8, device="cuda:0")
    si = torch.empty(1, device="cuda:0")
    am = dev_f32([0.5])
    prev = np.float32(0.5)
    for call in range(2):
        say("tensor delayed", NAMES[fmt], shape, "call", call)
        fp8.fp8_quantize_tensor(x, fmt, 0, dev_f32([scale]), q, si, am)
        torch.cuda.synchronize()
        oq, osi, oam = orc.quantize_tensor_scaled(xb, fmt, scale, amax_in=prev)
        prev = oam
        assert_codes_equal(q.cpu().numpy(), oq, "codes")
        assert_f32_bits_equal(si.cpu().numpy(), [osi], "scale_inv")
        assert_f32_bits_equal(am.cpu().numpy(), [oam], "amax")


def test_quantize_tensor_delayed_folds_amax(fp8, orc):
    xb = rand_bf16(64, 96, seed=29)
    x = dev_bf16(xb)
    q = torch.empty((64, 96), dtype=torch.uint8, device="cuda:0")
    si = torch.empty(1, device="cuda:0")
    am = dev_f32([1e9])                                  # larger than the tensor's amax: kept
    say("tensor delayed fold")
    fp8.fp8_quantize_tensor(x, 0, 0, dev_f32([3.5]), q, si, am)
    torch.cuda.synchronize()
    oq, osi, oam = orc.quantize_tensor_scaled(xb, 0, np.float32(3.5), amax_in=1e9)
    assert am.item() == oam == np.float32(1e9)
    assert_codes_equal(q.cpu().numpy(), oq, "codes")


# ----------------------------------------------------------- delayed scaling --

def run_delayed(fp8, orc, amaxes, n, L, algo, margin, fmt):
    hist = torch.zeros((n, L), device="cuda:0")
    head = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    scale = torch.ones(n, device="cuda:0")
    scale_inv = torch.ones(n, device="cuda:0")
    cur = torch.zeros(n, device="cuda:0")
    st = orc.DelayedState(n, L)
    for t, a in enumerate(amaxes):
        cur.copy_(torch.from_numpy(np.asarray(a, np.float32)))
        st.cur_amax[:] = a
        fp8.fp8_delayed_scale_update(cur, hist, head, algo, margin, fmt, scale, scale_inv)
        st.update(algo, margin, fmt)
        if t % 97 == 0 or t == len(amaxes) - 1:
            torch.cuda.synchronize()
            assert_f32_bits_equal(scale.cpu().numpy(), st.scale, f"scale step {t}")
            assert_f32_bits_equal(scale_inv.cpu().numpy(), st.scale_inv, f"scale_inv step {t}")
            assert_f32_bits_equal(hist.cpu().numpy(), st.history, f"history step {t}")
            assert head.item() == st.head[0]
            assert not cur.any().item()


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_delayed_update_hand_sequence(fp8, orc, algo, fmt):
    say("delayed hand", algo, fmt)
    seq = [[8.0], [1.0], [1.0], [1.0], [1.0], [1.0], [0.0], [np.nan], [np.inf], [2.0]]
    run_delayed(fp8, orc, seq, 1, 4, algo, 1, fmt)


def test_delayed_update_wraps_at_1024(fp8, orc):
    rng = np.random.default_rng(2)
    amaxes = np.exp2(rng.uniform(-6, 6, (1100, 3))).astype(np.float32)
    amaxes[5] = [900.0, 1e-3, 0.0]
    say("delayed 1024 wrap")
    run_delayed(fp8, orc, amaxes, 3, 1024, 1, 0, 0)


def test_delayed_update_more_tensors_than_one_workgroup(fp8, orc):
    """Above 64 tensors the update runs one wavefront per tensor and a second
    launch advances the head."""
    rng = np.random.default_rng(4)
    amaxes = np.exp2(rng.uniform(-6, 6, (12, 130))).astype(np.float32)
    amaxes[3, 7] = 0.0
    say("delayed 130 tensors")
    run_delayed(fp8, orc, amaxes, 130, 8, 1, 0, 0)
    run_delayed(fp8, orc, amaxes, 130, 8, 0, 1, 1)


def test_delayed_update_many_tensors(fp8, orc):
    rng = np.random.default_rng(3)
    amaxes = np.exp2(rng.uniform(-6, 6, (20, 37))).astype(np.float32)
    say("delayed 37 tensors")
    run_delayed(fp8, orc, amaxes, 37, 16, 1, 2, 1)


# ------------------------------------------------------------- determinism --

def test_quantizers_deterministic(fp8):
    xb = rand_bf16(1000, 520, seed=31)
    say("determinism")
    a = gpu_row(fp8, xb, 0, col_amax=True)
    b = gpu_row(fp8, xb, 0, col_amax=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    c = gpu_col(fp8, xb, 1)
    d = gpu_col(fp8, xb, 1)
    for u, v in zip(c, d):
        assert np.array_equal(u, v)


# ------------------------------------------------------------ batched rowwise --

def gpu_row_batch(fp8, xbs, fmt, margin=0, ld_pad=0, amax_mask=None, col_mask=None):
    """fp8_quantize_row_batch over the tensors xbs (numpy bf16 bits, same cols);
    ld_pad > 0 pads the code rows (a layout that takes one launch per tensor);
    col_mask[j] asks for tensor j's column amax (then returned as a 4th list)."""
    cols = xbs[0].shape[1]
    xs = [dev_bf16(xb) for xb in xbs]
    views, bufs = [], []
    for xb in xbs:
        v, buf, org = guarded(xb.shape[0], cols, torch.uint8, ld=cols + ld_pad if ld_pad else cols)
        views.append(v)
        bufs.append((buf, org, xb.shape[0]))
    sis = [torch.full((max(xb.shape[0], 1),), -1.0, device="cuda:0") for xb in xbs]
    ams = [torch.full((max(xb.shape[0], 1),), -1.0, device="cuda:0") for xb in xbs]
    amax_outs = [a if (amax_mask is None or amax_mask[j]) else None for j, a in enumerate(ams)]
    cas = None
    if col_mask is not None:
        # one guard float after each column-amax output
        cabufs = [torch.full((cols + 1,), -1.0, device="cuda:0") for _ in xbs]
        cas = [b[:cols] if col_mask[j] else None for j, b in enumerate(cabufs)]
    fp8.fp8_quantize_row_batch(xs, fmt, margin, views, sis, amax_outs, cas)
    torch.cuda.synchronize()
    for buf, org, rows in bufs:
        check_guard(buf, org, rows, cols)
    out = ([v.cpu().numpy() for v in views], [s.cpu().numpy()[:xb.shape[0]] for s, xb in zip(sis, xbs)],
           [a.cpu().numpy()[:xb.shape[0]] for a, xb in zip(ams, xbs)])
    if col_mask is None:
        return out
    for b in cabufs:
        assert b[cols].item() == -1.0, "write past the column-amax output"
    return out + ([b.cpu().numpy()[:cols] for b in cabufs],)


def check_row_batch(orc, xbs, fmt, margin, got, amax_mask=None, col_mask=None):
    qs, sis, ams = got[:3]
    for j, xb in enumerate(xbs):
        if col_mask is not None and col_mask[j]:
            assert_f32_bits_equal(got[3][j], orc.amax(xb, orc.AXIS_COL), f"column amax of tensor {j} {xb.shape}")
        elif col_mask is not None:
            assert np.all(got[3][j] == -1.0), f"column amax of tensor {j} was written although not requested"
    for j, xb in enumerate(xbs):
        oq, osi, oam = orc.quantize_row(xb, fmt, margin)
        assert_codes_equal(qs[j], oq, f"codes of tensor {j} {xb.shape}")
        assert_f32_bits_equal(sis[j], osi, f"scale_inv of tensor {j}")
        if amax_mask is None or amax_mask[j]:
            assert_f32_bits_equal(ams[j], oam, f"amax of tensor {j}")
        else:
            assert np.all(ams[j] == -1.0), f"amax of tensor {j} was written although not requested"


@pytest.mark.parametrize("fmt", FORMATS)
def test_quantize_row_batch_parity(fp8, orc, fmt):
    """Eight tensors in one launch: ragged row counts (not multiples of the four
    rows of a workgroup), empty tensors in the middle and at the end, one row."""
    cols = 136
    sizes = [5, 0, 64, 1, 130, 3, 0, 257]
    xbs = [rand_bf16(r, cols, seed=100 + j) for j, r in enumerate(sizes)]
    mask = [True, True, False, True, True, False, True, True]
    say("row batch", NAMES[fmt], sizes, cols)
    got = gpu_row_batch(fp8, xbs, fmt, 1, amax_mask=mask)
    check_row_batch(orc, xbs, fmt, 1, got, mask)


@pytest.mark.parametrize("cols", [8, 4096, 14336, 16384])
def test_quantize_row_batch_linear_pair(fp8, orc, cols):
    """A linear layer's activation and weight (same K) at row lengths from one
    chunk per lane to the longest row held in registers."""
    m, n = (1030, 2050) if cols <= 4096 else (70, 133)
    xbs = [rand_bf16(m, cols, seed=7), rand_bf16(n, cols, seed=8)]
    say("row batch pair", (m, n, cols))
    got = gpu_row_batch(fp8, xbs, 0, 0)
    check_row_batch(orc, xbs, 0, 0, got)


@pytest.mark.parametrize("fmt", FORMATS)
def test_quantize_row_batch_col_amax_parity(fp8, orc, fmt):
    """The column-amax side output in the same pass: ragged row counts, empty
    tensors, a tensor that does not ask for it, special values (NaN and Inf
    columns); codes, scales and row amax unchanged."""
    cols = 136
    sizes = [5, 0, 64, 1, 130, 3, 0, 257]
    xbs = [rand_bf16(r, cols, seed=200 + j) for j, r in enumerate(sizes)]
    xbs[4][7:11] = np.pad(special_rows(), ((0, 0), (0, cols - 16)))[:4]    # NaN in column 1, Inf in 0
    xbs[4][20, 100] = 0x7FC1                             # a NaN in column 100
    cmask = [True, True, True, False, True, True, True, True]
    say("row batch col amax", NAMES[fmt], sizes, cols)
    got = gpu_row_batch(fp8, xbs, fmt, 1, col_mask=cmask)
    check_row_batch(orc, xbs, fmt, 1, got, col_mask=cmask)
    assert np.isnan(got[3][4][1]) and np.isnan(got[3][4][100]) and np.isinf(got[3][4][0])


def grouped_amax_oracle(orc, xb, offsets):
    """Per-group column amax [G x cols] from the oracle's grouped colwise cast
    (rows offsets[g] .. offsets[g+1]-1, clamped to the tensor)."""
    return orc.grouped_quantize_col(xb, 0, offsets, 256)[2]


GROUPED_AMAX = [
    (136, [5, 0, 64, 1, 130, 0, 257, 3], 0, 0),      # one chunk per lane, empty groups, groups of 1 row
    (1024, [300, 0, 1, 255, 257, 2000, 17], 5, 7),   # rows before the first group and after the last
    (2048, [991, 0, 785, 1, 2000, 30], 0, 3),         # the MoE output-gradient width: 4 chunks per lane
    (4096, [700, 0, 260, 1300, 2], 1, 0),            # 8 chunks per lane
    (7168, [4994, 118, 0, 2115, 1408, 3], 0, 0),     # the MoE token shape: 16 chunks per lane
    (16384, [300, 0, 129, 45], 0, 0),                # 32 chunks per lane (folded into LDS per row)
]


@pytest.mark.parametrize("cols,sizes,before,after", GROUPED_AMAX,
                         ids=["short_rows", "ungrouped_rows", "dy_width", "8_chunks", "moe_tokens", "32_chunks"])
def test_quantize_row_batch_grouped_col_amax(fp8, orc, cols, sizes, before, after):
    """The per-group column amax as a side output of the rowwise cast, in one
    batch with a tensor grouped by fixed blocks of rows (an expert's weight
    rows), an ungrouped column amax and a tensor without one: every group's
    amax bit-exact against the oracle's grouped colwise cast (empty groups 0,
    NaN / Inf columns inside a group), codes and scales unchanged, nothing
    written past the outputs."""
    rng = np.random.default_rng(cols)
    rows0 = before + sum(sizes) + after
    off0 = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64) + before
    x0 = rand_bf16(rows0, cols, seed=cols + 1)
    g_nan = int(np.argmax(np.array(sizes) > 2))          # a group with rows: NaN in column 3, Inf in 5
    r = int(off0[g_nan])
    x0[r, 3] = 0x7FC1
    x0[r + 1, 5] = 0xFF80
    experts, per = 4, 96
    x1 = rand_bf16(experts * per, cols, seed=cols + 2)
    off1 = (np.arange(experts + 1) * per).astype(np.int64)
    x2 = rand_bf16(33, cols, seed=cols + 3)
    x3 = rand_bf16(7, cols, seed=cols + 4)
    xbs = [x0, x1, x2, x3]
    G = [len(sizes), experts, 0, 0]
    xs = [dev_bf16(xb) for xb in xbs]
    qs = [torch.empty(xb.shape, dtype=torch.uint8, device="cuda:0") for xb in xbs]
    sis = [torch.empty(xb.shape[0], device="cuda:0") for xb in xbs]
    bufs = [torch.full((max(g, 1) * cols + 1,), -1.0, device="cuda:0") for g in G]
    cas = [bufs[0][:-1], bufs[1][:-1], bufs[2][:-1], None]
    offs = [torch.from_numpy(off0).to("cuda:0"), torch.from_numpy(off1).to("cuda:0"), None, None]
    say("row batch grouped col amax", cols, sizes, before, after)
    fp8.fp8_quantize_row_batch(xs, 1, 0, qs, sis, None, cas, offs)
    torch.cuda.synchronize()
    for b in bufs:
        assert b[-1].item() == -1.0, "write past a column-amax output"
    assert np.all(bufs[3].cpu().numpy() == -1.0)
    for j, xb in enumerate(xbs):
        oq, osi, _ = orc.quantize_row(xb, 1, 0)
        assert_codes_equal(qs[j].cpu().numpy(), oq, f"codes of tensor {j}")
        assert_f32_bits_equal(sis[j].cpu().numpy(), osi, f"scale_inv of tensor {j}")
    got0 = cas[0].cpu().numpy().reshape(len(sizes), cols)
    assert_f32_bits_equal(got0, grouped_amax_oracle(orc, x0, off0), "grouped column amax (token groups)")
    assert np.isnan(got0[g_nan, 3]) and np.isinf(got0[g_nan, 5])
    assert not got0[np.array(sizes) == 0].any(), "an empty group's amax is not 0"
    got1 = cas[1].cpu().numpy().reshape(experts, cols)
    assert_f32_bits_equal(got1, grouped_amax_oracle(orc, x1, off1), "grouped column amax (expert rows)")
    assert_f32_bits_equal(cas[2].cpu().numpy(), orc.amax(x2, orc.AXIS_COL), "ungrouped column amax")


@pytest.mark.parametrize("shape", [(3000, 8), (2500, 520), (5000, 4096), (2100, 8200), (2300, 14336),
                                   (900, 16384)])
def test_quantize_row_col_amax_row_lengths(fp8, orc, shape):
    """Single tensors from one chunk per lane to the longest row held in
    registers, with more rows than the grid's wavefronts (each wavefront
    folds several rows into its running column max)."""
    rows, cols = shape
    xb = rand_bf16(rows, cols, seed=rows + cols)
    say("row + col amax", shape)
    q, si, am, ca = gpu_row(fp8, xb, 1, 0, col_amax=True)
    oq, osi, oam = orc.quantize_row(xb, 1, 0)
    assert_codes_equal(q, oq, "codes")
    assert_f32_bits_equal(si, osi, "scale_inv")
    assert_f32_bits_equal(ca, orc.amax(xb, orc.AXIS_COL), "col amax")


@pytest.mark.parametrize("fmt", [0, 3])
def test_quantize_row_batch_per_tensor_layouts(fp8, orc, fmt):
    """Padded code rows (ldq not a multiple of 8), rows longer than the register
    kernels hold, and special values: one launch per tensor, same results."""
    say("row batch fallback", NAMES[fmt])
    xbs = [rand_bf16(9, 40, seed=1), np.ascontiguousarray(np.pad(special_rows(), ((0, 0), (0, 24))))]
    got = gpu_row_batch(fp8, xbs, fmt, 2, ld_pad=3)
    check_row_batch(orc, xbs, fmt, 2, got)
    long = [rand_bf16(3, 16392, seed=2), rand_bf16(5, 16392, seed=3)]
    got = gpu_row_batch(fp8, long, fmt, 0)
    check_row_batch(orc, long, fmt, 0, got)
    say("row batch fallback with col amax", NAMES[fmt])
    got = gpu_row_batch(fp8, long, fmt, 0, col_mask=[True, False])
    check_row_batch(orc, long, fmt, 0, got, col_mask=[True, False])
    got = gpu_row_batch(fp8, xbs, fmt, 2, ld_pad=3, col_mask=[True, True])
    check_row_batch(orc, xbs, fmt, 2, got, col_mask=[True, True])


def test_quantize_row_batch_special_values(fp8, orc):
    xbs = [special_rows(), special_rows()[::-1].copy()]
    for fmt in FORMATS:
        say("row batch specials", NAMES[fmt])
        got = gpu_row_batch(fp8, xbs, fmt, 0)
        check_row_batch(orc, xbs, fmt, 0, got)


def test_quantize_row_batch_matches_single_calls_at_llama3_8b(fp8, orc):
    """X [8192 x 4096] and W [14336 x 4096] of the Llama3-8B up-projection:
    the batched launch gives the bytes of two fp8_quantize_row calls, with and
    without the column-amax side outputs (compared with the oracle's column
    amax of both whole tensors)."""
    w = workloads.c2()
    say("row batch c2 full size")
    x, wt = dev_bf16(w["x"]), dev_bf16(w["w"])
    outs = []
    for batched, colmax in ((True, False), (False, False), (True, True)):
        qx = torch.empty(x.shape, dtype=torch.uint8, device="cuda:0")
        qw = torch.empty(wt.shape, dtype=torch.uint8, device="cuda:0")
        sx = torch.empty(x.shape[0], device="cuda:0")
        sw = torch.empty(wt.shape[0], device="cuda:0")
        cx = torch.full((x.shape[1],), -1.0, device="cuda:0")
        cw = torch.full((wt.shape[1],), -1.0, device="cuda:0")
        if batched:
            fp8.fp8_quantize_row_batch([x, wt], 0, 0, [qx, qw], [sx, sw], None, [cx, cw] if colmax else None)
        else:
            fp8.fp8_quantize_row(x, 0, 0, qx, sx)
            fp8.fp8_quantize_row(wt, 0, 0, qw, sw)
        torch.cuda.synchronize()
        outs.append((qx, qw, sx, sw))
    for ref in outs[1:]:
        for a, b in zip(outs[0], ref):
            assert torch.equal(a, b)
    assert_f32_bits_equal(cx.cpu().numpy(), orc.amax(w["x"], orc.AXIS_COL), "X column amax")
    assert_f32_bits_equal(cw.cpu().numpy(), orc.amax(w["w"], orc.AXIS_COL), "W column amax")


# ---------------------------------------------------- batched delayed tensorwise --

@pytest.mark.parametrize("fmt", FORMATS)
def test_quantize_tensor_batch_delayed_parity(fp8, orc, fmt):
    """Three tensors with their own delayed scales in one launch (ragged row
    counts, one tensor of one row): codes, scale_inv and the folded amax as
    fp8_quantize_tensor gives them, and as the oracle computes them."""
    cols = 264
    sizes = [37, 1, 600]
    xbs = [rand_bf16(r, cols, seed=40 + j, spread=3) for j, r in enumerate(sizes)]
    scales = [np.float32(v) for v in (3.5, 0.75, 1.0 / 24.0)]
    start = [np.float32(v) for v in (0.0, 1e6, 0.5)]      # a folded amax keeps a larger value already there
    say("tensor batch delayed", NAMES[fmt], sizes)
    xs = [dev_bf16(xb) for xb in xbs]
    outs = {}
    for batched in (True, False):
        qs = [torch.empty((r, cols), dtype=torch.uint8, device="cuda:0") for r in sizes]
        sc = [torch.tensor([v], device="cuda:0") for v in scales]
        si = [torch.full((1,), -1.0, device="cuda:0") for _ in sizes]
        am = [torch.tensor([v], device="cuda:0") for v in start]
        if batched:
            fp8.fp8_quantize_tensor_batch(xs, fmt, sc, qs, si, am)
        else:
            for j in range(len(sizes)):
                fp8.fp8_quantize_tensor(xs[j], fmt, 0, sc[j], qs[j], si[j], am[j])
        torch.cuda.synchronize()
        outs[batched] = ([q.cpu().numpy() for q in qs], [t.cpu().numpy() for t in si], [t.cpu().numpy() for t in am])
    for j, xb in enumerate(xbs):
        for part in range(3):
            assert np.array_equal(outs[True][part][j].view(np.uint8), outs[False][part][j].view(np.uint8)), (j, part)
        oq, osi, oam = orc.quantize_tensor_scaled(xb, fmt, scales[j], amax_in=start[j])
        assert_codes_equal(outs[True][0][j], oq, f"codes of tensor {j}")
        assert_f32_bits_equal(outs[True][1][j], [osi], f"scale_inv of tensor {j}")
        assert_f32_bits_equal(outs[True][2][j], [oam], f"amax of tensor {j}")


def test_quantize_tensor_batch_flux_mlp(fp8):
    """The Flux-12B MLP's X [4608 x 3072] and W [12288 x 3072] with their delayed
    scales: the batched launch gives the bytes of two fp8_quantize_tensor calls."""
    w = workloads.c3()
    _, xb = next(w["x_steps"]())
    say("tensor batch c3 full size")
    x, wt = dev_bf16(xb), dev_bf16(w["w"])
    res = []
    for batched in (True, False):
        qx = torch.empty(x.shape, dtype=torch.uint8, device="cuda:0")
        qw = torch.empty(wt.shape, dtype=torch.uint8, device="cuda:0")
        sc = [torch.tensor([112.0], device="cuda:0"), torch.tensor([3584.0], device="cuda:0")]
        si = [torch.empty(1, device="cuda:0") for _ in range(2)]
        am = [torch.zeros(1, device="cuda:0") for _ in range(2)]
        if batched:
            fp8.fp8_quantize_tensor_batch([x, wt], 0, sc, [qx, qw], si, am)
        else:
            fp8.fp8_quantize_tensor(x, 0, 0, sc[0], qx, si[0], am[0])
            fp8.fp8_quantize_tensor(wt, 0, 0, sc[1], qw, si[1], am[1])
        torch.cuda.synchronize()
        res.append([qx, qw] + si + am)
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_quantize_row_batch_single_and_empty(fp8, orc):
    """count = 1 (the batch entry point as a plain rowwise cast), and batches
    whose only rows sit in one tensor."""
    xb = rand_bf16(77, 520, seed=61)
    say("row batch count 1")
    check_row_batch(orc, [xb], 1, 0, gpu_row_batch(fp8, [xb], 1, 0))
    xbs = [rand_bf16(0, 520, seed=62), rand_bf16(0, 520, seed=63), xb]
    say("row batch empty leaders")
    check_row_batch(orc, xbs, 2, 1, gpu_row_batch(fp8, xbs, 2, 1))


@pytest.mark.parametrize("fmt", [1, 2])
def test_quantize_tensor_batch_per_tensor_paths(fp8, orc, fmt):
    """An empty tensor and a misaligned row stride send the batch to one launch
    per tensor: results as fp8_quantize_tensor's, the empty tensor still writes
    its scale_inv and leaves its amax target as it was."""
    cols = 40
    xbs = [rand_bf16(13, cols, seed=71, spread=2), rand_bf16(0, cols, seed=72)]
    scales = [np.float32(2.5), np.float32(0.125)]
    start = [np.float32(0.0), np.float32(7.0)]
    say("tensor batch fallback", NAMES[fmt])
    xs = [dev_bf16(xb) for xb in xbs]
    qbuf = torch.full((13, cols + 3), 0x5A, dtype=torch.uint8, device="cuda:0")
    qs = [qbuf[:, :cols], torch.empty((0, cols), dtype=torch.uint8, device="cuda:0")]
    sc = [torch.tensor([v], device="cuda:0") for v in scales]
    si = [torch.full((1,), -1.0, device="cuda:0") for _ in xbs]
    am = [torch.tensor([v], device="cuda:0") for v in start]
    fp8.fp8_quantize_tensor_batch(xs, fmt, sc, qs, si, am)
    torch.cuda.synchronize()
    oq, osi, oam = orc.quantize_tensor_scaled(xbs[0], fmt, scales[0], amax_in=start[0])
    assert_codes_equal(qs[0].cpu().numpy(), oq, "codes")
    assert np.all(qbuf[:, cols:].cpu().numpy() == 0x5A), "padding written"
    assert_f32_bits_equal(si[0].cpu().numpy(), [osi], "scale_inv")
    assert_f32_bits_equal(am[0].cpu().numpy(), [oam], "amax")
    assert_f32_bits_equal(si[1].cpu().numpy(), [np.float32(1.0) / scales[1]], "scale_inv of the empty tensor")
    assert_f32_bits_equal(am[1].cpu().numpy(), [start[1]], "amax of the empty tensor")


# ------------------------------------------------ delayed state checkpointing --

def test_delayed_state_checkpoint_resume_bitwise(fp8):
    """The delayed-scaling state is plain caller-owned device memory (history,
    head, scale, scale_inv, cur_amax): 16 steps straight give the same bytes as
    8 steps, a copy of the state to the host, fresh device buffers filled from
    that copy, and 8 more steps, at every step (codes, scale_inv, state)."""
    rng = np.random.default_rng(17)
    n_t, L, rows, cols = 2, 1024, 96, 264
    drift = np.cumprod(np.concatenate([[1.0], rng.uniform(0.5, 2.0, 15)])).astype(np.float32)
    xs = [workloads.bf16_bits(rng.standard_normal((2, rows, cols)).astype(np.float32) * d) for d in drift]

    def fresh(state=None):
        if state is None:
            return [torch.zeros((n_t, L), device="cuda:0"), torch.zeros(1, dtype=torch.int32, device="cuda:0"),
                    torch.ones(n_t, device="cuda:0"), torch.ones(n_t, device="cuda:0"),
                    torch.zeros(n_t, device="cuda:0")]
        return [torch.from_numpy(a.copy()).to("cuda:0") for a in state]

    def steps(st, t0, t1, log):
        hist, head, scale, scale_inv, cur = st
        for t in range(t0, t1):
            qs = [torch.empty((rows, cols), dtype=torch.uint8, device="cuda:0") for _ in range(n_t)]
            si = [torch.empty(1, device="cuda:0") for _ in range(n_t)]
            fp8.fp8_quantize_tensor_batch([dev_bf16(xs[t][j]) for j in range(n_t)], fp8.E4M3,
                                          [scale[j:j + 1] for j in range(n_t)], qs, si,
                                          [cur[j:j + 1] for j in range(n_t)])
            fp8.fp8_delayed_scale_update(cur, hist, head, fp8.AMAX_MAX, 0, fp8.E4M3, scale, scale_inv)
            torch.cuda.synchronize()
            log.append([q.cpu().numpy() for q in qs] + [s.cpu().numpy() for s in si] +
                       [a.cpu().numpy().copy() for a in (hist, head, scale, scale_inv, cur)])

    say("delayed checkpoint / resume, 16 steps")
    straight, resumed = [], []
    steps(fresh(), 0, 16, straight)
    first = fresh()
    steps(first, 0, 8, resumed)
    host = [a.cpu().numpy().copy() for a in first]      # the checkpoint
    del first
    steps(fresh(host), 8, 16, resumed)
    assert len(straight) == len(resumed) == 16
    for t, (a, b) in enumerate(zip(straight, resumed)):
        for i, (u, v) in enumerate(zip(a, b)):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"step {t}, output {i}"
    # the drift moves the scales: the sequence is not trivially constant
    assert len({float(x[-3][0]) for x in straight}) > 2


def test_wrong_max_is_not_used_by_the_library(fp8, orc):
    """The silent corruption of a scale computed against the wrong format max
    (448 for e4m3fnuz, whose largest value is 240) does not happen on the
    library path: x = 400 cast rowwise in e4m3fnuz gives the top code 0x7F with
    scale_inv = 400 / 240, so the dequantised value stays 400; in OCP e4m3 the
    top code is 0x7E (448). The fnuz and OCP bytes differ, and each decodes
    only in its own format."""
    xb = workloads.bf16_bits(np.array([[400.0, -400.0, 100.0, 0.0] * 4], np.float32))
    x = dev_bf16(xb)
    out = {}
    for fmt in (0, 2):
        q = torch.empty((1, 16), dtype=torch.uint8, device="cuda:0")
        si = torch.empty(1, device="cuda:0")
        say("wrong-max check", NAMES[fmt])
        fp8.fp8_quantize_row(x, fmt, 0, q, si)
        torch.cuda.synchronize()
        out[fmt] = (q.cpu().numpy()[0], si.cpu().numpy()[0])
    qf, sf = out[2]
    assert qf[0] == 0x7F and qf[1] == 0xFF                # +-240, fnuz's top codes
    assert abs(orc.decode(2, qf[:1])[0] * float(sf) - 400.0) < 1e-3
    assert abs(float(sf) - 400.0 / 240.0) < 1e-6          # not 400 / 448
    qo, so = out[0]
    assert qo[0] == 0x7E and qo[1] == 0xFE                # +-448, OCP e4m3's top codes
    assert abs(orc.decode(0, qo[:1])[0] * float(so) - 400.0) < 1e-3
    assert abs(orc.decode(2, qo[:1])[0] * float(so) - 400.0) > 100.0   # read as fnuz: wrong by half
