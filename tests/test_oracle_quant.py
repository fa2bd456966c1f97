"""Pins of the oracle's scale computation, quantizers and delayed-scaling update:
closed forms worked by hand, invariants of a saturating RNE cast, the reading of
the product rounding, the wrong-max corruption and hand-traced delayed
sequences. CPU only."""
import collections
import struct
from fractions import Fraction

import numpy as np
import pytest

import workloads

F32_MAX = float(np.finfo(np.float32).max)


def f32(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def bf(values):
    return workloads.bf16_bits(np.asarray(values, np.float32))


# --------------------------------------------------------------- closed forms --

def test_closed_form_row_e4m3_and_fnuz(orc):
    """Row [1, -2, 0.5, 0, -0, 1e-3] has amax 2. OCP e4m3: s = 448/2 = 224 and the
    codes are 224 -> 0x76, -448 -> 0xFE, 112 -> 0x6E, 0 -> 0x00, -0 -> 0x80 and
    bf16(1e-3)*224 = 0.22388 -> 1.75*2^-3 -> 0x26. e4m3fnuz: s = 120 and
    120 -> 0x77, -240 -> 0xFF, 60 -> 0x6F, 0, -0 -> 0x00 (no negative zero),
    0.11993 -> 1.875*2^-4 -> 0x27. Worked by hand from the bit layouts."""
    x = bf([[1.0, -2.0, 0.5, 0.0, -0.0, 1e-3]])
    q, si, am = orc.quantize_row(x, 0)
    assert q[0].tolist() == [0x76, 0xFE, 0x6E, 0x00, 0x80, 0x26]
    assert am[0] == 2.0 and si[0] == np.float32(1.0 / 224.0)
    q, si, am = orc.quantize_row(x, 2)
    assert q[0].tolist() == [0x77, 0xFF, 0x6F, 0x00, 0x00, 0x27]
    assert si[0] == np.float32(1.0 / 120.0)
    # margin 1 halves the scale: 1 * 112 -> 0x6E, -2 * 112 = -224 -> 0xF6
    q, si, _ = orc.quantize_row(x, 0, margin=1)
    assert q[0, :3].tolist() == [0x6E, 0xF6, 0x66]
    assert si[0] == np.float32(1.0 / 112.0)


def test_scale_rules(orc):
    # exact quotients
    assert orc.scale_current(0, 2.0) == 224.0
    assert orc.scale_current(1, 4.0) == 14336.0
    assert orc.scale_current(2, 400.0) == np.float32(0.6)
    # margin is a power of two
    assert orc.scale_current(0, 2.0, margin=2) == 56.0
    # amax zero or non-finite -> s = 1
    for a in (0.0, np.inf, np.nan):
        assert orc.scale_current(0, a) == 1.0
    # fp32 overflow of fmax/amax -> FLT_MAX (amax is an fp32 subnormal)
    assert orc.scale_current(0, 2.0 ** -140) == np.float32(F32_MAX)
    # correctly rounded division: 448/3 rounded once to fp32
    want = np.float32(Fraction(448, 3).__float__())
    assert orc.scale_current(0, 3.0) == want
    assert orc.reciprocal(np.float32(224.0)) == np.float32(1 / 224.0)


def test_product_rounding_witness(orc):
    """The cast sees fl32(x*s), not the exact product. x = bf16 0x3F81
    (1.0078125), s = fp32 0x3F86F21C: x*s = 1.0625 + 7*2^-28 exactly, just above
    the e4m3 tie 1.0625, but fl32(x*s) = 1.0625, which ties to even -> 0x38.
    Rounding the exact product once would give 0x39."""
    s = f32(0x3F86F21C)
    exact = Fraction(1.0078125) * Fraction(s)
    assert exact > Fraction(1.0625) and exact - Fraction(1.0625) == Fraction(7, 2 ** 28)
    assert orc.quantize_value(0, 0x3F81, s) == 0x38


def test_wrong_max_silently_clips(orc):
    """The corruption the TorchTitan/TorchAO post describes (scales computed
    against the wrong format max): with e4m3fnuz, x = 400, the right scale
    240/400 keeps 400 after dequantisation; a scale from 448 saturates the
    cast and dequantises to about 214 (-46%) without any error. Reading OCP codes
    as fnuz halves every value."""
    x = bf([[400.0]])
    q, si, _ = orc.quantize_row(x, 2)
    assert q[0, 0] == 0x7F
    assert abs(orc.decode(2, q[0])[0] * si[0] - 400.0) < 1e-3
    wrong_s = np.float32(448.0 / 400.0)
    qw = orc.quantize_value(2, int(x[0, 0]), wrong_s)
    assert qw == 0x7F                                   # saturated: no error raised
    deq = orc.decode(2, np.array([qw], np.uint8))[0] * float(np.float32(1.0 / wrong_s))
    assert 214.0 < deq < 214.5
    assert orc.decode(2, np.array([0x40], np.uint8))[0] == 1.0 and orc.decode(0, np.array([0x40], np.uint8))[0] == 2.0
    assert orc.decode(2, np.array([0x7E], np.uint8))[0] == 224.0 and orc.decode(0, np.array([0x7E], np.uint8))[0] == 448.0


# ------------------------------------------------------------------ invariants --

def _rows(seed=3, rows=64, cols=200):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-12, 12, size=(rows, 1))).astype(np.float32)
    return bf(x)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
@pytest.mark.parametrize("margin", [0, 1, 2])
def test_row_quantize_invariants(orc, fmt, margin):
    x = _rows()
    xf = workloads.bf16_to_f32(x).astype(np.float64)
    q, si, am = orc.quantize_row(x, fmt, margin)
    fmax = orc.fmt_info(fmt)[0]
    top = fmax * 2.0 ** -margin
    dq = orc.decode(fmt, q)
    # amax is the row's largest magnitude (exact)
    assert np.array_equal(am, np.abs(xf).max(axis=1).astype(np.float32))
    for i in range(x.shape[0]):
        # the largest element lands exactly on fmax * 2^-margin, nothing above it
        assert np.abs(dq[i]).max() == top
        assert dq[i, np.argmax(np.abs(xf[i]))] in (top, -top)
        # rounding is monotone
        order = np.argsort(xf[i], kind="stable")
        assert np.all(np.diff(dq[i][order]) >= 0)
        # error of the cast: within half a quantum of fl32(x*s) (plus fp32 rounding)
        s = 1.0 / float(si[i])
        p = xf[i] * s
        _, _, m, bias = orc.fmt_info(fmt)
        e = np.floor(np.log2(np.maximum(np.abs(p), 2.0 ** (1 - bias))))
        half_q = 2.0 ** (e - m - 1)
        assert np.all(np.abs(dq[i] - p) <= half_q * (1 + 1e-6) + np.abs(p) * 2.0 ** -23)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_row_quantize_power_of_two_invariance(orc, fmt):
    """Scaling a row by 2^j (exactly, within range) leaves the codes unchanged and
    scales scale_inv by 2^j."""
    x = _rows(seed=5)
    q0, si0, _ = orc.quantize_row(x, fmt)
    for j in (-3, 5):
        xs = bf(workloads.bf16_to_f32(x) * np.float32(2.0 ** j))
        q1, si1, _ = orc.quantize_row(xs, fmt)
        assert np.array_equal(q0, q1)
        assert np.array_equal(si1, (si0 * np.float32(2.0 ** j)).astype(np.float32))


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_col_equals_row_of_transpose(orc, fmt):
    x = _rows(seed=11, rows=37, cols=53)
    qt, si, am = orc.quantize_col(x, fmt, 1)
    qr, sir, amr = orc.quantize_row(np.ascontiguousarray(x.T), fmt, 1)
    assert np.array_equal(qt, qr) and np.array_equal(si, sir) and np.array_equal(am, amr)
    assert np.array_equal(orc.amax(x, orc.AXIS_COL), amr)
    assert np.array_equal(orc.amax(x, orc.AXIS_ROW), orc.quantize_row(x, fmt)[2])


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_tensor_current_is_one_row(orc, fmt):
    x = _rows(seed=13, rows=9, cols=31)
    q, si, am = orc.quantize_tensor_current(x, fmt, 0)
    qr, sir, amr = orc.quantize_row(x.reshape(1, -1), fmt)
    assert np.array_equal(q.reshape(1, -1), qr) and si == sir[0] and am == amr[0]
    assert am == orc.amax(x, orc.AXIS_TENSOR)[0]
    # delayed cast with the same scale gives the same codes and accumulates amax
    s = orc.scale_current(fmt, am)
    q2, si2, am2 = orc.quantize_tensor_scaled(x, fmt, s, amax_in=0.5)
    assert np.array_equal(q2, q) and si2 == si and am2 == max(am, np.float32(0.5))


def test_degenerate_rows(orc):
    x = bf([[0.0, -0.0, 0.0], [1.0, np.nan, -2.0], [np.inf, 1.0, -3.0], [-np.inf, 0.0, 0.0]])
    q, si, am = orc.quantize_row(x, 0)
    assert q[0].tolist() == [0x00, 0x80, 0x00] and si[0] == 1.0 and am[0] == 0.0
    assert np.isnan(am[1]) and si[1] == 1.0 and q[1].tolist() == [0x38, 0x7F, 0xC0]
    assert np.isinf(am[2]) and si[2] == 1.0 and q[2].tolist() == [0x7E, 0x38, 0xC4]
    assert q[3].tolist() == [0xFE, 0x00, 0x00]
    q, si, am = orc.quantize_row(x, 2)
    assert q[0].tolist() == [0, 0, 0] and q[1, 1] == 0x80


# ------------------------------------------------------------- delayed scaling --

def _run_delayed(orc, amaxes, L, algo, margin=0, fmt=0):
    """Returns the scale in force at each step (the one that step's cast uses)."""
    st = orc.DelayedState(1, L)
    used = []
    for a in amaxes:
        used.append(float(st.scale[0]))
        st.cur_amax[0] = a
        st.update(algo, margin, fmt)
        assert st.cur_amax[0] == 0.0
    return used, st


def test_delayed_hand_sequences(orc):
    """L = 4, amax per step 8, 1, 1, 1, 1, 1 (e4m3, fmax 448). 'max': steps 2-5
    use 448/8 = 56 and step 6 uses 448 once the 8 has left the window.
    'most_recent': step 2 uses 56, step 3 on use 448. Step 1 uses s0 = 1."""
    seq = [8.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    used, _ = _run_delayed(orc, seq, 4, orc.AMAX_MAX)
    assert used == [1.0, 56.0, 56.0, 56.0, 56.0, 448.0]
    used, _ = _run_delayed(orc, seq, 4, orc.AMAX_MOST_RECENT)
    assert used == [1.0, 56.0, 448.0, 448.0, 448.0, 448.0]
    used, _ = _run_delayed(orc, seq, 4, orc.AMAX_MAX, margin=1)
    assert used == [1.0, 28.0, 28.0, 28.0, 28.0, 224.0]


def test_delayed_keeps_scale_on_bad_amax(orc):
    for bad in (0.0, np.nan, np.inf):
        used, st = _run_delayed(orc, [8.0, bad, 2.0], 16, orc.AMAX_MOST_RECENT)
        assert used == [1.0, 56.0, 56.0]
        assert st.scale[0] == 224.0 and st.scale_inv[0] == np.float32(1 / 224.0)
    # with 'max', a NaN in the window freezes the scale until it leaves the window
    used, _ = _run_delayed(orc, [8.0, np.nan, 2.0, 2.0, 2.0, 2.0], 3, orc.AMAX_MAX)
    assert used == [1.0, 56.0, 56.0, 56.0, 56.0, 224.0]


def test_delayed_window_wraps_at_1024(orc):
    """1100 steps with L = 1024 and 'max': the scale in force equals fmax over the
    max of an explicit sliding window of the last 1024 amaxes."""
    rng = np.random.default_rng(1)
    amaxes = np.exp2(rng.uniform(-4, 4, 1100)).astype(np.float32)
    amaxes[3] = 1000.0
    used, st = _run_delayed(orc, amaxes, 1024, orc.AMAX_MAX)
    window = collections.deque(maxlen=1024)
    s = 1.0
    for t, a in enumerate(amaxes):
        assert used[t] == s, t
        window.append(float(a))
        s = float(np.float32(448.0 / max(window)))
    assert st.head[0] == 1100 % 1024
    assert 448.0 / 1000.0 == pytest.approx(used[500])
    assert used[1030] != used[1020]  # the outlier left the window at step 3 + 1024


def test_delayed_n_tensors_independent(orc):
    st = orc.DelayedState(3, 8)
    st.cur_amax[:] = [1.0, 2.0, 4.0]
    st.update(orc.AMAX_MAX, 0, 1)
    assert st.scale.tolist() == [57344.0, 28672.0, 14336.0]
    assert st.history[:, 0].tolist() == [1.0, 2.0, 4.0] and st.head[0] == 1
