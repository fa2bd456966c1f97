"""Pins of the oracle's FP8 codec against the format definitions, torch's float8
dtypes and brute force. CPU only.

The two maxima the pages print (448 for OCP e4m3, 240 for e4m3fnuz; "FP8 Training
on MI300X", section on the AMD FP8 dtype difference, and the TorchTitan/TorchAO
post's answer on silently wrong results) come from tests/golden/format_maxima.txt.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TORCH_DT = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2, 2: torch.float8_e4m3fnuz, 3: torch.float8_e5m2fnuz}
NAMES = {0: "e4m3fn", 1: "e5m2", 2: "e4m3fnuz", 3: "e5m2fnuz"}


def read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, *vals = line.split()
                rows[key] = vals
    return rows


def torch_table(fmt):
    return torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).to(torch.float64).numpy()


def brute_encode(table, fmt, v):
    """Nearest finite code by exhaustive search over the 256-code table, ties to
    the even code, zero keeping the sign of v in OCP; v clamped to +-fmax, NaN ->
    the canonical NaN code."""
    finite = np.isfinite(table)
    codes = np.nonzero(finite)[0]
    vals = table[codes]
    fmax = vals.max()
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    for lo in range(0, v.size, 4096):
        chunk = v.reshape(-1)[lo:lo + 4096]
        c = np.clip(chunk, -fmax, fmax)
        d = np.abs(c[:, None] - vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # among equidistant candidates prefer an even code (LSB 0); the two
        # zeros of OCP are both even, so zero is resolved by sign below
        even = (codes[None, :] & 1) == 0
        pick = np.where((cand & even).any(axis=1, keepdims=True), cand & even, cand)
        idx = pick.argmax(axis=1)
        res = codes[idx].astype(np.uint8)
        zero = vals[idx] == 0
        if fmt in (0, 1):
            res[zero] = np.where(np.signbit(chunk[zero]), 0x80, 0x00)
        else:
            res[zero] = 0x00
        nan = np.isnan(chunk)
        if fmt in (0, 1):
            res[nan] = np.where(np.signbit(chunk[nan]), 0xFF, 0x7F)
        else:
            res[nan] = 0x80
        out.reshape(-1)[lo:lo + 4096] = res
    return out


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_decode_table_matches_torch_dtypes(orc, fmt):
    ours = orc.decode_table(fmt)
    ref = torch_table(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zero: OCP has 0x80 = -0, fnuz has no negative zero
    assert np.signbit(ours[0x80]) == (fmt in (0, 1)) or fmt in (2, 3)


def test_format_maxima_from_pages(orc):
    gold = read_golden("format_maxima.txt")
    for fmt, name in NAMES.items():
        fmax, *_ = orc.fmt_info(fmt)
        assert fmax == float(gold[name][0]), name
        table = orc.decode_table(fmt)
        assert np.nanmax(table[np.isfinite(table)]) == fmax


@pytest.mark.parametrize("fmt,finite,nan_codes,inf_codes,min_normal,min_sub,max_code", [
    (0, 254, {0x7F, 0xFF}, set(), 2.0 ** -6, 2.0 ** -9, 0x7E),
    (1, 248, {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}, {0x7C, 0xFC}, 2.0 ** -14, 2.0 ** -16, 0x7B),
    (2, 255, {0x80}, set(), 2.0 ** -7, 2.0 ** -10, 0x7F),
    (3, 255, {0x80}, set(), 2.0 ** -15, 2.0 ** -17, 0x7F),
])
def test_format_table_structure(orc, fmt, finite, nan_codes, inf_codes, min_normal, min_sub, max_code):
    t = orc.decode_table(fmt)
    assert int(np.isfinite(t).sum()) == finite
    assert set(np.nonzero(np.isnan(t))[0].tolist()) == nan_codes
    assert set(np.nonzero(np.isinf(t))[0].tolist()) == inf_codes
    _, e, m, _ = orc.fmt_info(fmt)
    pos = t[:max_code + 1]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly up to the max"
    assert pos[1] == min_sub
    assert pos[1 << m] == min_normal
    # sign symmetry: code | 0x80 is the negation wherever both are finite and nonzero
    for c in range(1, max_code + 1):
        assert t[c | 0x80] == -t[c]


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_encode_all_bf16_times_scales_brute_force(orc, fmt):
    """Every bf16 value times a set of fp32 scales (the products rounded to fp32, as
    the cast sees them): oracle encode == exhaustive nearest-even search."""
    table = orc.decode_table(fmt)
    bf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    scales = np.array([1.0, 0.75, 3.0e-3, 224.0, 1.0 / 3.0, 2.0 ** -20], np.float32)
    for s in scales:
        with np.errstate(over="ignore", invalid="ignore"):
            p = (bf.astype(np.float64) * np.float64(s)).astype(np.float32)
        keep = np.isnan(p) | (np.abs(p.astype(np.float64)) < 2.0 * orc.fmt_info(fmt)[0]) | np.isinf(p)
        p = p[keep]
        got = orc.encode(fmt, p)
        want = brute_encode(table, fmt, p.astype(np.float64))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (s, p[bad[:5]], got[bad[:5]], want[bad[:5]])


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_encode_ties_and_neighbours(orc, fmt):
    """Every midpoint between adjacent finite values, and the fp32 values one ulp
    either side of it: ties go to the even code, neighbours to the nearer value."""
    table = orc.decode_table(fmt)
    vals = np.unique(table[np.isfinite(table)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (vals[:-1] + vals[1:]) / 2), "midpoints are fp32-exact"
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
                          vals.astype(np.float32)])
    got = orc.encode(fmt, pts)
    want = brute_encode(table, fmt, pts.astype(np.float64))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", [0, 1, 2, 3])
def test_encode_matches_torch_cast_in_range(orc, fmt):
    """Within [-fmax, fmax] torch's float8 cast is a round-to-nearest-even cast: a
    library routine independent of the oracle. (Outside it torch gives NaN/Inf
    instead of saturating, so the range is restricted.)"""
    fmax = orc.fmt_info(fmt)[0]
    rng = np.random.default_rng(7)
    mags = np.exp2(rng.uniform(-20, np.log2(fmax), 200000)).astype(np.float32)
    v = np.concatenate([mags, -mags, np.float32([0.0, -0.0, fmax, -fmax])])
    v = v[np.abs(v) <= fmax]
    ours = orc.encode(fmt, v)
    ref = torch.from_numpy(v).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_special_values(orc):
    enc = lambda f, v: int(orc.encode(f, np.array([v], np.float32))[0])
    # saturation, Inf included
    assert enc(0, 1e30) == 0x7E and enc(0, -1e30) == 0xFE
    assert enc(0, np.inf) == 0x7E and enc(0, -np.inf) == 0xFE
    assert enc(0, 464.0) == 0x7E
    assert enc(1, np.inf) == 0x7B and enc(1, -1e30) == 0xFB
    assert enc(3, -1e30) == 0xFF
    assert enc(2, 1e30) == 0x7F
    # NaN: sign | 0x7F for OCP, the single 0x80 for fnuz
    assert enc(0, np.nan) == 0x7F and enc(0, -np.nan) == 0xFF
    assert enc(1, np.nan) == 0x7F
    assert enc(2, np.nan) == 0x80 and enc(3, -np.nan) == 0x80
    # ties to even
    assert enc(0, 1.0625) == 0x38 and enc(0, 1.1875) == 0x3A
    assert enc(0, 2.0 ** -10) == 0x00 and enc(0, -(2.0 ** -10)) == 0x80
    assert enc(2, -(2.0 ** -11)) == 0x00 and enc(2, 3 * 2.0 ** -11) == 0x02
    # zeros
    assert enc(0, -0.0) == 0x80 and enc(2, -0.0) == 0x00 and enc(3, -1e-30) == 0x00
