"""ctypes wrapper over the CPU oracle (liboracle.so, built from fp8_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the tests, the smoke check and the
benchmark's CPU-baseline leg import this module. It takes and returns numpy
arrays; it never touches torch, the GPU or the HIP library.

Format codes: 0 = E4M3 (OCP e4m3fn), 1 = E5M2 (OCP), 2 = E4M3 FNUZ, 3 = E5M2 FNUZ.
bf16 tensors are passed as uint16 bit patterns; FP8 tensors as uint8 codes.
"""
import ctypes
import os
import subprocess

import numpy as np

E4M3, E5M2, E4M3_FNUZ, E5M2_FNUZ = 0, 1, 2, 3
FORMATS = (E4M3, E5M2, E4M3_FNUZ, E5M2_FNUZ)
AMAX_MOST_RECENT, AMAX_MAX = 0, 1
AXIS_TENSOR, AXIS_ROW, AXIS_COL = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build():
    """Compile liboracle.so with make (gcc, OpenMP)."""
    subprocess.run(["make", "-s", "-C", _HERE], check=True)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    F = ctypes.c_float
    sig = {
        "orc_fmt_info": (I, [I, P, P, P, P]),
        "orc_decode": (ctypes.c_double, [I, ctypes.c_uint8]),
        "orc_encode": (ctypes.c_uint8, [I, F]),
        "orc_encode_array": (None, [I, P, I64, P]),
        "orc_decode_array": (None, [I, P, I64, P]),
        "orc_scale_current": (F, [I, F, I]),
        "orc_reciprocal": (F, [F]),
        "orc_quantize_value": (ctypes.c_uint8, [I, ctypes.c_uint16, F]),
        "orc_amax": (None, [P, I64, I64, I64, I, P]),
        "orc_quantize_row": (None, [P, I64, I64, I64, I, I, P, I64, P, P]),
        "orc_quantize_col": (None, [P, I64, I64, I64, I, I, P, I64, P, P]),
        "orc_quantize_tensor_scaled": (None, [P, I64, I64, I64, I, F, P, I64, P, P]),
        "orc_quantize_tensor_current": (None, [P, I64, I64, I64, I, I, P, I64, P, P]),
        "orc_delayed_update": (None, [P, P, P, I64, I, I, I, I, P, P]),
        "orc_gemm": (None, [P, I, I64, P, I, I64, I64, I64, I64, P, I, P, I, P, P, P, I64, P]),
        "orc_gemm_entries": (None, [P, I, I64, P, I, I64, I64, P, I, P, I, P, P, I64, P, P]),
        "orc_grouped_gemm_entries": (None, [P, I, I64, P, I, I64, I64, P, I, I64, I64, P, P,
                                            P, P, I64, P, P]),
        "orc_mx_scale": (ctypes.c_uint8, [I, F]),
        "orc_mx_scale_value": (ctypes.c_double, [ctypes.c_uint8]),
        "orc_mx_quantize_row": (None, [P, I64, I64, I64, I, P, I64, P, I64]),
        "orc_mx_gemm": (None, [P, I, I64, P, I64, P, I, I64, P, I64, I64, I64, I64, P, P, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _vec_mode(scale, rows):
    """1 if scale holds one value per row, 0 if it is a single value."""
    if scale.size == rows:
        return 1
    if scale.size == 1:
        return 0
    raise ValueError(f"scale has {scale.size} entries for {rows} rows")


def fmt_info(fmt):
    """(fmax, ebits, mbits, bias) of an encoding."""
    fmax = ctypes.c_double()
    e, m, b = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    if _load().orc_fmt_info(fmt, ctypes.byref(fmax), ctypes.byref(e), ctypes.byref(m), ctypes.byref(b)):
        raise ValueError(f"unknown format {fmt}")
    return fmax.value, e.value, m.value, b.value


def decode(fmt, codes):
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().orc_decode_array(fmt, _p(codes), codes.size, _p(out))
    return out


def decode_table(fmt):
    return decode(fmt, np.arange(256, dtype=np.uint8))


def encode(fmt, values_f32):
    v = _c(values_f32, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_encode_array(fmt, _p(v), v.size, _p(out))
    return out


def scale_current(fmt, amax, margin=0):
    return np.float32(_load().orc_scale_current(fmt, float(np.float32(amax)), margin))


def reciprocal(s):
    return np.float32(_load().orc_reciprocal(float(np.float32(s))))


def quantize_value(fmt, x_bf16_bits, s):
    return _load().orc_quantize_value(fmt, int(x_bf16_bits), float(np.float32(s)))


def amax(x_bf16, axis):
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    n = {AXIS_TENSOR: 1, AXIS_ROW: rows, AXIS_COL: cols}[axis]
    out = np.empty(n, np.float32)
    _load().orc_amax(_p(x), rows, cols, cols, axis, _p(out))
    return out


def quantize_row(x_bf16, fmt, margin=0):
    """Per-row scales: returns (q [rows x cols] uint8, scale_inv [rows], amax [rows])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    si = np.empty(rows, np.float32)
    am = np.empty(rows, np.float32)
    _load().orc_quantize_row(_p(x), rows, cols, cols, fmt, margin, _p(q), cols, _p(si), _p(am))
    return q, si, am


def quantize_col(x_bf16, fmt, margin=0):
    """Per-column scales, transposed output: returns (qt [cols x rows], scale_inv [cols], amax [cols])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    qt = np.empty((cols, rows), np.uint8)
    si = np.empty(cols, np.float32)
    am = np.empty(cols, np.float32)
    _load().orc_quantize_col(_p(x), rows, cols, cols, fmt, margin, _p(qt), rows, _p(si), _p(am))
    return qt, si, am


def quantize_tensor_scaled(x_bf16, fmt, s, amax_in=0.0):
    """Given scale s: returns (q, scale_inv_used, amax_acc) with amax_acc = max(amax_in, amax(x))."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    si = np.empty(1, np.float32)
    am = np.array([amax_in], np.float32)
    _load().orc_quantize_tensor_scaled(_p(x), rows, cols, cols, fmt, float(np.float32(s)), _p(q), cols,
                                       _p(si), _p(am))
    return q, si[0], am[0]


def quantize_tensor_current(x_bf16, fmt, margin=0):
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    si = np.empty(1, np.float32)
    am = np.empty(1, np.float32)
    _load().orc_quantize_tensor_current(_p(x), rows, cols, cols, fmt, margin, _p(q), cols, _p(si), _p(am))
    return q, si[0], am[0]


class DelayedState:
    """n delayed-scaling states in the layout the library uses: history [n x L]
    ring with a shared head, scale[n], scale_inv[n], cur_amax[n]."""

    def __init__(self, n, L):
        self.n, self.L = n, L
        self.history = np.zeros((n, L), np.float32)
        self.head = np.zeros(1, np.int32)
        self.scale = np.ones(n, np.float32)
        self.scale_inv = np.ones(n, np.float32)
        self.cur_amax = np.zeros(n, np.float32)

    def update(self, algo, margin, fmt):
        _load().orc_delayed_update(_p(self.cur_amax), _p(self.history), _p(self.head), self.n, self.L, algo,
                                   margin, fmt, _p(self.scale), _p(self.scale_inv))


def gemm(a, fa, b, fb, a_scale, b_scale, with_bound=True):
    """Y = (A B^T) * sa * sb in fp64; a [m x k], b [n x k] uint8 codes; scales are
    fp32 vectors ([m] / [n]) or single values. Returns (y, bound)."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    sa = _c(np.atleast_1d(a_scale), np.float32)
    sb = _c(np.atleast_1d(b_scale), np.float32)
    a_vec = _vec_mode(sa, m)
    b_vec = _vec_mode(sb, n)
    ad = np.empty(max(m * k, 1), np.float64)
    bd = np.empty(max(n * k, 1), np.float64)
    y = np.empty((m, n), np.float64)
    bound = np.empty((m, n), np.float64) if with_bound else None
    _load().orc_gemm(_p(a), fa, k, _p(b), fb, k, m, n, k, _p(sa), a_vec, _p(sb), b_vec, _p(ad), _p(bd),
                     _p(y), n, _p(bound))
    return y, bound


def gemm_entries(a, fa, b, fb, a_scale, b_scale, ii, jj):
    """Selected outputs Y[ii[e], jj[e]] of the dense product; returns (y, bound)."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    m, k = a.shape
    n = b.shape[0]
    sa = _c(np.atleast_1d(a_scale), np.float32)
    sb = _c(np.atleast_1d(b_scale), np.float32)
    a_vec = _vec_mode(sa, m)
    b_vec = _vec_mode(sb, n)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    y = np.empty(ii.size, np.float64)
    bound = np.empty(ii.size, np.float64)
    _load().orc_gemm_entries(_p(a), fa, k, _p(b), fb, k, k, _p(sa), a_vec, _p(sb), b_vec, _p(ii), _p(jj),
                             ii.size, _p(y), _p(bound))
    return y, bound


def grouped_gemm_entries(a, fa, b, fb, offsets, a_scale, b_scale, ii, jj):
    """Selected outputs of the grouped product. a [total_m x k], b [g x n x k],
    offsets int64 [g+1], a_scale [total_m], b_scale [g x n]."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    g, n, k = b.shape
    offsets = _c(offsets, np.int64)
    sa = _c(a_scale, np.float32)
    sb = _c(b_scale, np.float32).reshape(-1)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    y = np.empty(ii.size, np.float64)
    bound = np.empty(ii.size, np.float64)
    _load().orc_grouped_gemm_entries(_p(a), fa, k, _p(b), fb, k, n * k, _p(offsets), g, n, k, _p(sa), _p(sb),
                                     _p(ii), _p(jj), ii.size, _p(y), _p(bound))
    return y, bound


def grouped_gemm(a, fa, b, fb, offsets, a_scale, b_scale):
    """Whole grouped product as the per-group dense oracle: rows of group g are
    A[offsets[g]:offsets[g+1]] times B_g^T with scales a_scale[rows], b_scale[g]."""
    a = _c(a, np.uint8)
    g, n, k = b.shape
    total_m = a.shape[0]
    y = np.full((total_m, n), np.nan)
    bound = np.full((total_m, n), np.nan)
    for gg in range(g):
        lo, hi = int(offsets[gg]), int(offsets[gg + 1])
        if hi > lo:
            y[lo:hi], bound[lo:hi] = gemm(a[lo:hi], fa, b[gg], fb, a_scale[lo:hi], b_scale[gg])
    return y, bound


# ------------------------------------------------------------------ MX blocks --
# MXFP8 (block-32 scales along K, E8M0 power-of-two): see the MX block section
# of fp8_oracle.c for the reading of the format.
MX_BLOCK = 32


def mx_scale(fmt, amax):
    """Biased E8M0 exponent of a block with the given amax (0xFF: NaN)."""
    return int(_load().orc_mx_scale(fmt, float(amax)))


def mx_scale_value(s):
    return _load().orc_mx_scale_value(int(s))


def mx_quantize_row(x_bf16, fmt):
    """Rowwise MX quantization: returns (codes [rows x cols], scales uint8 [rows x cols/32])."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    assert cols % MX_BLOCK == 0
    q = np.empty((rows, cols), np.uint8)
    sc = np.empty((rows, cols // MX_BLOCK), np.uint8)
    _load().orc_mx_quantize_row(_p(x), rows, cols, cols, fmt, _p(q), cols, _p(sc), cols // MX_BLOCK)
    return q, sc


def mx_gemm(a, fa, sa, b, fb, sb):
    """Y = A B^T with per-block E8M0 scales, fp64: a [m x k], sa [m x k/32], b [n x k],
    sb [n x k/32]. Returns (y, bound)."""
    a = _c(a, np.uint8)
    b = _c(b, np.uint8)
    sa = _c(sa, np.uint8)
    sb = _c(sb, np.uint8)
    m, k = a.shape
    n = b.shape[0]
    ad = np.empty(max(m * k, 1), np.float64)
    bd = np.empty(max(n * k, 1), np.float64)
    y = np.empty((m, n), np.float64)
    bound = np.empty((m, n), np.float64)
    _load().orc_mx_gemm(_p(a), fa, k, _p(sa), k // MX_BLOCK, _p(b), fb, k, _p(sb), k // MX_BLOCK, m, n, k, _p(ad),
                        _p(bd), _p(y), n, _p(bound))
    return y, bound


def mx_grouped_gemm(a, fa, sa, b, fb, sb, offsets):
    """Grouped MX product: rows offsets[g] .. offsets[g+1] of a (scales sa) times
    b[g]^T (scales sb[g]); returns (y [total_m x n], bound)."""
    a = _c(a, np.uint8)
    g, n, k = b.shape
    y = np.full((a.shape[0], n), np.nan)
    bound = np.full((a.shape[0], n), np.nan)
    for gg in range(g):
        lo, hi = int(offsets[gg]), int(offsets[gg + 1])
        if hi > lo:
            y[lo:hi], bound[lo:hi] = mx_gemm(a[lo:hi], fa, sa[lo:hi], b[gg], fb, sb[gg])
    return y, bound


def mx_scale_values(s):
    """E8M0 bytes -> 2^(s - 127) in fp64; 255 -> NaN."""
    s = np.asarray(s)
    return np.where(s == 255, np.nan, np.exp2(s.astype(np.float64) - 127.0))


def mx_gemm_entries(a, fa, sa, b, fb, sb, ii, jj, chunk=1024):
    """Selected outputs Y[ii[e], jj[e]] of the MX product, from its definition:
    per 32-element block the dot product of the decoded codes times both block
    scales, summed over the blocks (fp64). Returns (y, bound)."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    ii = np.asarray(ii, np.int64)
    jj = np.asarray(jj, np.int64)
    k = a.shape[1]
    nb = k // MX_BLOCK
    y = np.empty(ii.size, np.float64)
    bound = np.empty(ii.size, np.float64)
    for lo in range(0, ii.size, chunk):
        i, j = ii[lo:lo + chunk], jj[lo:lo + chunk]
        p = decode(fa, a[i]).reshape(-1, nb, MX_BLOCK) * decode(fb, b[j]).reshape(-1, nb, MX_BLOCK)
        x = mx_scale_values(np.asarray(sa)[i]) * mx_scale_values(np.asarray(sb)[j])
        y[lo:lo + chunk] = (x * p.sum(axis=2)).sum(axis=1)
        bound[lo:lo + chunk] = (x * np.abs(p).sum(axis=2)).sum(axis=1)
    return y, bound


def mx_grouped_gemm_entries(a, fa, sa, b, fb, sb, offsets, ii, jj):
    """Selected outputs of the grouped MX product: row i belongs to the group g
    with offsets[g] <= i < offsets[g+1], whose weights are b[g] (scales sb[g])."""
    g, n, k = b.shape
    grp = np.searchsorted(np.asarray(offsets, np.int64), np.asarray(ii, np.int64), side="right") - 1
    rows_b = grp * n + np.asarray(jj, np.int64)
    return mx_gemm_entries(a, fa, sa, np.asarray(b).reshape(g * n, k), fb,
                           np.asarray(sb).reshape(g * n, k // MX_BLOCK), ii, rows_b)


# ---------------------------------------------------------------- MoE backward --
# The MoE backward ("FP8 Training on AMD GPUs with TorchTitan and TorchAO": the
# backward-pass speedup of the MoE model, colwise scales, grouped GEMM) needs the
# expert-local transposed operands of the weight gradient: for expert g with
# tokens offsets[g] .. offsets[g+1], dW_g = dY_g^T X_g contracts over that
# group's tokens. Reading used here (the pages give no layout): each group's
# codes sit transposed in one matrix, group g at columns P_g .. P_g + m_g, where
# P_g = sum over h < g of roundup(m_h, align); columns m_g .. roundup(m_g, align)
# of the group hold zero codes, which add nothing to a contraction.

def padded_offsets(offsets, align):
    """P_g = sum_{h<g} roundup(m_h, align), g = 0..G (int64 [G+1])."""
    offsets = np.asarray(offsets, np.int64)
    sizes = np.diff(offsets)
    padded = (sizes + align - 1) // align * align
    out = np.zeros(offsets.size, np.int64)
    out[1:] = np.cumsum(padded)
    return out


def grouped_quantize_col(x_bf16, fmt, offsets, align, margin=0):
    """Colwise quantization per group of rows: group g's rows get their own
    per-column scales (amax over the group's rows only) and are written
    transposed at columns P_g .. P_g + m_g of qt [cols x P_G], zero codes after.
    An empty group has amax 0, hence scale 1. Returns (qt, scale_inv [G x cols],
    amax [G x cols])."""
    x = _c(x_bf16, np.uint16)
    offsets = np.asarray(offsets, np.int64)
    G = offsets.size - 1
    cols = x.shape[1]
    P = padded_offsets(offsets, align)
    qt = np.zeros((cols, int(P[-1])), np.uint8)
    si = np.ones((G, cols), np.float32)
    am = np.zeros((G, cols), np.float32)
    for g in range(G):
        lo, hi = int(offsets[g]), int(offsets[g + 1])
        if hi > lo:
            qg, si[g], am[g] = quantize_col(x[lo:hi], fmt, margin)
            qt[:, P[g]:P[g] + (hi - lo)] = qg
    return qt, si, am


def grouped_gemm_ragged_k(a_t, fa, b_t, fb, offsets, align, a_scale, b_scale):
    """Weight-gradient form of the grouped product: for each group g,
    D_g = (A[:, P_g : P_g + m_g] . B[:, P_g : P_g + m_g]^T) * a_scale[g][:, None] * b_scale[g][None, :]
    in fp64, with a_t [m x L] and b_t [n x L] codes in the padded grouped
    layout and a_scale [G x m], b_scale [G x n]. An empty group gives zeros.
    Returns (d [G x m x n], bound [G x m x n])."""
    a_t = _c(a_t, np.uint8)
    b_t = _c(b_t, np.uint8)
    offsets = np.asarray(offsets, np.int64)
    G = offsets.size - 1
    m, n = a_t.shape[0], b_t.shape[0]
    P = padded_offsets(offsets, align)
    d = np.zeros((G, m, n))
    bound = np.zeros((G, m, n))
    for g in range(G):
        kg = int(offsets[g + 1] - offsets[g])
        if kg > 0:
            sl = slice(int(P[g]), int(P[g]) + kg)
            d[g], bound[g] = gemm(a_t[:, sl], fa, b_t[:, sl], fb, a_scale[g], b_scale[g])
    return d, bound


def gemm_within_bound(gpu, y, bound, out_bf16=True):
    """The acceptance rule: |gpu - y| <= 1e-3 * bound + 2^-8 |y| (the last term only
    for bf16 output). NaN matches NaN. Returns a boolean array."""
    gpu = np.asarray(gpu, np.float64)
    tol = 1e-3 * bound + (2.0 ** -8 * np.abs(y) if out_bf16 else 0.0)
    ok = np.abs(gpu - y) <= tol
    both_nan = np.isnan(gpu) & np.isnan(y)
    same_inf = np.isinf(gpu) & np.isinf(y) & (np.sign(gpu) == np.sign(y))
    return ok | both_nan | same_inf


# ------------------------------------------------------------- MoE layer forward --
# The per-layer MoE path ("How PyTorch FP8 Optimizations on AMD GPUs Reduce LLM
# Cost ...": What Happened, the per-MoE-layer latency; "FP8 Training on AMD GPUs
# with TorchTitan and TorchAO": fused quantization kernels, FP8 grouped GEMM for
# MoE). The pages give no layer definition; the reading used here is the
# plainest MoE feed-forward layer: each token goes to its top-k experts, every
# expert applies a SwiGLU FFN, and the k results are summed with the router's
# weights. Steps: route (expert-sorted order), permute + rowwise quantize,
# grouped GEMM with the stacked gate|up weights, SwiGLU + rowwise quantize,
# grouped GEMM with the down weights, unpermute + weighted combine.

def moe_route(expert_idx, num_experts):
    """expert_idx int [T x k] -> (offsets int64 [E+1], dest int32 [T x k]):
    a counting sort of the T*k (token, slot) entries by expert, stable in
    (token, slot) order. dest[t, j] is the row of entry (t, j) in the
    expert-sorted order; expert e owns rows offsets[e] .. offsets[e+1]-1. An
    index outside [0, E) drops its entry (dest -1, not counted)."""
    idx = np.asarray(expert_idx, np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(num_experts, np.int64)
    for e in flat:                                      # histogram
        if 0 <= e < num_experts:
            counts[e] += 1
    offsets = np.zeros(num_experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    nxt = offsets[:-1].copy()                           # next free row of each expert
    dest = np.full(flat.size, -1, np.int64)
    for i, e in enumerate(flat):                        # entries in (token, slot) order
        if 0 <= e < num_experts:
            dest[i] = nxt[e]
            nxt[e] += 1
    return offsets, dest.reshape(T, k).astype(np.int32)


def moe_permute_quantize_row(x_bf16, dest, fmt, margin=0):
    """Rowwise quantization of every token, its codes and scale placed at each
    of its k destination rows: returns (q [T*k x H], scale_inv [T*k])."""
    q_tok, si_tok, _ = quantize_row(x_bf16, fmt, margin)
    dest = np.asarray(dest, np.int64)
    T, k = dest.shape
    q = np.empty((T * k, q_tok.shape[1]), np.uint8)
    si = np.empty(T * k, np.float32)
    for t in range(T):
        for j in range(k):
            if dest[t, j] >= 0:
                q[dest[t, j]] = q_tok[t]
                si[dest[t, j]] = si_tok[t]
    return q, si


def silu(x):
    """x * sigmoid(x) in fp64."""
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_quantize_row(h_bf16, fmt, margin=0):
    """h [rows x 2I] bf16 holding gate (columns 0 .. I-1) | up (I .. 2I-1):
    a = silu(gate) * up in fp64, rounded once to fp32; then rowwise current
    scaling of the fp32 rows (amax, s = scale rule, code = cast(fl32(a * s))).
    Returns (q [rows x I], scale_inv [rows], a32 [rows x I])."""
    h = bf16_to_f64(h_bf16)
    inter = h.shape[1] // 2
    a32 = (silu(h[:, :inter]) * h[:, inter:]).astype(np.float32)
    rows = a32.shape[0]
    q = np.empty((rows, inter), np.uint8)
    si = np.empty(rows, np.float32)
    for r in range(rows):
        row = a32[r]
        am = np.float32(np.nan) if np.isnan(row).any() else np.abs(row).max(initial=np.float32(0))
        s = scale_current(fmt, am, margin)
        q[r] = encode(fmt, row * s)                      # fp32 product, then the saturating RNE cast
        si[r] = reciprocal(s)
    return q, si, a32


def moe_unpermute_combine(y_bf16, dest, weights):
    """out[t] = sum over slots j of weights[t, j] * y[dest[t, j]] in fp64
    (returned unrounded, with the sum of magnitudes as the bound's base);
    slots whose destination is outside y's rows add nothing."""
    y = bf16_to_f64(y_bf16)
    dest = np.asarray(dest, np.int64)
    w = np.asarray(weights, np.float64)
    T, k = dest.shape
    out = np.zeros((T, y.shape[1]))
    mag = np.zeros((T, y.shape[1]))
    for j in range(k):
        ok = (dest[:, j] >= 0) & (dest[:, j] < y.shape[0])
        term = np.where(ok[:, None], w[:, j:j + 1] * y[np.where(ok, dest[:, j], 0)], 0.0)
        out += term
        mag += np.abs(term)
    return out, mag


def bf16_to_f64(bits):
    """bf16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x):
    """fp64 -> bf16 bit patterns, round to nearest even. Goes through fp32
    rounded to odd (truncate toward zero, then set the last bit if anything
    was dropped), which keeps the bf16 decision that of the fp64 value."""
    x = np.asarray(x, np.float64)
    f = x.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    u = f.view(np.uint32).copy()
    inexact = (f.astype(np.float64) != x) & np.isfinite(x)
    u[inexact] |= 1
    u64 = u.astype(np.uint64)
    r = ((u64 + 0x7FFF + ((u64 >> 16) & 1)) >> 16).astype(np.uint16)
    r[np.isnan(x)] = 0x7FC0
    return r


# ------------------------------------------------------------------- blockwise --
# The blockwise recipe ("FP8 training for Flux models", Configuration: blockwise
# among the recipes; no block shapes or scale rule on the pages). Reading used
# here: tiles of 1 x 128 along K for activations and gradients and 128 x 128 for
# weights share one scale; the scale is the current-scaling rule's fmax / amax
# (with its zero / non-finite / overflow conventions, no margin) rounded down
# to a power of two, so that no element saturates and the block scale is exact
# as a power of two. Stored as the E8M0 byte of the dequantization factor
# 1 / s (= 127 - log2 s, within 0 .. 247); codes are cast(x * s).
BLOCK = 128


def pow2_scale(fmt, amax):
    """The block scale: the current-scaling scale rounded down to a power of two."""
    s = float(scale_current(fmt, amax, 0))
    return 2.0 ** np.floor(np.log2(s))


def _block_codes(xv_bits, fmt, s):
    """Cast of a block of bf16 values at scale s (fp32 product, then the
    saturating RNE cast)."""
    vals = (np.asarray(xv_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return encode(fmt, vals * np.float32(s))


def blockwise_quantize_act(x_bf16, fmt):
    """1 x 128 blocks: returns (q [rows x K], e8 bytes [rows x K/128])."""
    x = np.asarray(x_bf16, np.uint16)
    rows, K = x.shape
    assert K % BLOCK == 0
    q = np.empty((rows, K), np.uint8)
    e8 = np.empty((rows, K // BLOCK), np.uint8)
    for r in range(rows):
        for b in range(K // BLOCK):
            blk = x[r, b * BLOCK:(b + 1) * BLOCK]
            am = amax(blk[None, :], AXIS_TENSOR)[0]
            s = pow2_scale(fmt, am)
            q[r, b * BLOCK:(b + 1) * BLOCK] = _block_codes(blk, fmt, s)
            e8[r, b] = 127 - int(np.log2(s))
    return q, e8


def blockwise_quantize_weight(w_bf16, fmt):
    """128 x 128 tiles (the last row tile may be shorter): returns
    (q [n x K], e8 bytes [ceil(n/128) x K/128])."""
    w = np.asarray(w_bf16, np.uint16)
    n, K = w.shape
    assert K % BLOCK == 0
    nt = (n + BLOCK - 1) // BLOCK
    q = np.empty((n, K), np.uint8)
    e8 = np.empty((nt, K // BLOCK), np.uint8)
    for t in range(nt):
        r0, r1 = t * BLOCK, min(n, (t + 1) * BLOCK)
        for b in range(K // BLOCK):
            tile = np.ascontiguousarray(w[r0:r1, b * BLOCK:(b + 1) * BLOCK])
            am = amax(tile.reshape(1, -1), AXIS_TENSOR)[0]
            s = pow2_scale(fmt, am)
            q[r0:r1, b * BLOCK:(b + 1) * BLOCK] = _block_codes(tile, fmt, s)
            e8[t, b] = 127 - int(np.log2(s))
    return q, e8


def blockwise_gemm(a, fa, ea, b, fb, eb_tiles):
    """Y = sum over 128-deep K blocks kb of 2^(ea[i,kb]-127) 2^(eb[j//128,kb]-127)
    * sum_{k in kb} dec(a_ik) dec(b_jk), fp64. Returns (y, bound)."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    m, K = a.shape
    n = b.shape[0]
    nb = K // BLOCK
    ad = decode(fa, a).reshape(m, nb, BLOCK)
    bd = decode(fb, b).reshape(n, nb, BLOCK)
    xa = np.exp2(np.asarray(ea, np.float64) - 127.0)                       # [m x nb]
    xb = np.exp2(np.asarray(eb_tiles, np.float64) - 127.0)[np.arange(n) // BLOCK]   # [n x nb]
    y = np.zeros((m, n))
    bound = np.zeros((m, n))
    for kb in range(nb):
        p = ad[:, kb, :] @ bd[:, kb, :].T
        pm = np.abs(ad[:, kb, :]) @ np.abs(bd[:, kb, :]).T
        x = xa[:, kb:kb + 1] * xb[None, :, kb]
        y += x * p
        bound += x * pm
    return y, bound


def blockwise_gemm_entries(a, fa, ea, b, fb, eb_tiles, ii, jj, chunk=1024):
    """Selected outputs Y[ii[e], jj[e]] of blockwise_gemm, from the same
    definition evaluated per entry. Returns (y, bound)."""
    a = np.asarray(a, np.uint8)
    b = np.asarray(b, np.uint8)
    ii = np.asarray(ii, np.int64)
    jj = np.asarray(jj, np.int64)
    nb = a.shape[1] // BLOCK
    y = np.empty(ii.size)
    bound = np.empty(ii.size)
    for lo in range(0, ii.size, chunk):
        i, j = ii[lo:lo + chunk], jj[lo:lo + chunk]
        p = decode(fa, a[i]).reshape(-1, nb, BLOCK) * decode(fb, b[j]).reshape(-1, nb, BLOCK)
        x = np.exp2(np.asarray(ea, np.float64)[i] - 127.0) * np.exp2(np.asarray(eb_tiles, np.float64)[j // BLOCK] - 127.0)
        y[lo:lo + chunk] = (x * p.sum(axis=2)).sum(axis=1)
        bound[lo:lo + chunk] = (x * np.abs(p).sum(axis=2)).sum(axis=1)
    return y, bound


# ------------------------------------------------------ whole products by rows --
# The products above evaluated on every output of a full-size workload, in
# blocks of rows so that the fp64 results of a block fit in memory. Same
# definition ("FP8 Training on AMD GPUs with TorchTitan and TorchAO": rowwise /
# colwise scaled FP8 linear layers and grouped GEMM; the MX and blockwise
# readings above): the decoded codes form fp64 matrices and numpy's fp64 matrix
# product is the library step that sums over k. Every product of two decoded
# codes is exact in fp64, so only the summation order differs from the loops
# of fp8_oracle.c (a relative error of at most k * 2^-53 of the bound term).
# For the block-scaled forms, each decoded code is first multiplied by its
# block's power-of-two factor (exact in fp64: the factors lie in 2^-127 ..
# 2^127 and the codes' magnitudes in 2^-17 .. 2^16), which turns the sum over
# blocks of scaled block sums into one plain sum over k.

def _scaled_rows(codes, fmt, e8, block):
    """Decoded codes [r x k] times 2^(e8 - 127) of their K block (e8 [r x k/block]; 255 -> NaN)."""
    dec = decode(fmt, codes)
    x = mx_scale_values(np.asarray(e8))
    return dec * np.repeat(x, block, axis=1)


def _product(ad, bd, bd_abs, sa, sb):
    """(y, bound) of decoded operand rows ad [r x k], bd [n x k] (bd_abs = |bd|)
    with the dequantisation factors sa [r] / sb [n] (or single values):
    y = (ad bd^T) * sa * sb, bound = |sa * sb| * (|ad| |bd|^T)."""
    sa = np.asarray(sa, np.float64).reshape(-1, 1) if np.size(sa) > 1 else np.float64(np.asarray(sa).reshape(-1)[0])
    sb = np.asarray(sb, np.float64).reshape(1, -1) if np.size(sb) > 1 else np.float64(np.asarray(sb).reshape(-1)[0])
    s = ad @ bd.T
    t = np.abs(ad) @ bd_abs.T
    return s * sa * sb, np.abs(sa * sb) * t


def gemm_by_rows(a, fa, b, fb, a_scale, b_scale, chunk=1024):
    """Every output of Y = (A B^T) * sa * sb (the oracle's gemm), yielded as
    (r0, r1, y [r1-r0 x n], bound) over blocks of `chunk` rows of A."""
    a = np.asarray(a, np.uint8)
    m = a.shape[0]
    sa = np.asarray(np.atleast_1d(a_scale), np.float32)
    sb = np.asarray(np.atleast_1d(b_scale), np.float32)
    bd = decode(fb, b)
    bd_abs = np.abs(bd)
    for r0 in range(0, m, chunk):
        r1 = min(m, r0 + chunk)
        y, bound = _product(decode(fa, a[r0:r1]), bd, bd_abs, sa[r0:r1] if sa.size > 1 else sa, sb)
        yield r0, r1, y, bound


def mx_gemm_by_rows(a, fa, sa, b, fb, sb, chunk=1024):
    """Every output of the MX product (mx_gemm): a [m x k] with E8M0 block
    scales sa [m x k/32], b [n x k] with sb [n x k/32]; yields (r0, r1, y, bound)."""
    a = np.asarray(a, np.uint8)
    bd = _scaled_rows(b, fb, sb, MX_BLOCK)
    bd_abs = np.abs(bd)
    for r0 in range(0, a.shape[0], chunk):
        r1 = min(a.shape[0], r0 + chunk)
        y, bound = _product(_scaled_rows(a[r0:r1], fa, np.asarray(sa)[r0:r1], MX_BLOCK), bd, bd_abs, 1.0, 1.0)
        yield r0, r1, y, bound


def blockwise_gemm_by_rows(a, fa, ea, b, fb, eb_tiles, chunk=1024):
    """Every output of the blockwise product (blockwise_gemm): ea [m x k/128]
    per activation row, eb_tiles [ceil(n/128) x k/128] per weight tile;
    yields (r0, r1, y, bound)."""
    a = np.asarray(a, np.uint8)
    n = np.asarray(b).shape[0]
    eb_rows = np.asarray(eb_tiles)[np.arange(n) // BLOCK]
    bd = _scaled_rows(b, fb, eb_rows, BLOCK)
    bd_abs = np.abs(bd)
    for r0 in range(0, a.shape[0], chunk):
        r1 = min(a.shape[0], r0 + chunk)
        y, bound = _product(_scaled_rows(a[r0:r1], fa, np.asarray(ea)[r0:r1], BLOCK), bd, bd_abs, 1.0, 1.0)
        yield r0, r1, y, bound
