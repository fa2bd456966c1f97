"""Python binding of libfp8amax (the MI355X FP8 linear-layer library).

Thin ctypes marshalling over the C ABI declared in include/fp8amax.h: the
functions below carry the same names and arguments; torch tensors supply
device memory (data_ptr, strides) and the stream (torch's current stream).
Every step of the computation runs in the library's HIP kernels. If the
library is missing or fails to load, importing this package raises.

bf16 inputs are torch.bfloat16 tensors; FP8 codes are any 1-byte tensors
(torch.uint8 or a torch.float8_* dtype); scales and amax are float32.
"""
import ctypes
import os

import torch

__all__ = [
    "E4M3", "E5M2", "E4M3_FNUZ", "E5M2_FNUZ", "AXIS_TENSOR", "AXIS_ROW", "AXIS_COL",
    "AMAX_MOST_RECENT", "AMAX_MAX", "SCALE_TENSOR", "SCALE_VECTOR", "OUT_BF16", "OUT_F32",
    "Fp8Error", "LIB_PATH", "lib", "fp8_query_device", "fp8_status_string", "fp8_amax",
    "fp8_quantize_tensor", "fp8_quantize_tensor_batch", "fp8_quantize_row", "fp8_quantize_row_batch",
    "fp8_quantize_col", "fp8_quantize_rowcol", "fp8_delayed_scale_update",
    "fp8_gemm_scaled", "fp8_grouped_gemm_scaled", "fp8_grouped_quantize_col", "fp8_grouped_gemm_ragged_k",
    "grouped_layout_width", "GROUP_K_ALIGN", "MX_BLOCK", "fp8_mx_quantize_row", "fp8_gemm_mx",
    "fp8_grouped_gemm_mx", "mx_scale_records", "fp8_moe_route", "fp8_moe_permute_quantize_row",
    "fp8_swiglu_quantize_row", "fp8_moe_unpermute_combine", "fp8_blockwise_quantize_act",
    "fp8_blockwise_quantize_weight", "EXPORTED_SYMBOLS",
]

E4M3, E5M2, E4M3_FNUZ, E5M2_FNUZ = 0, 1, 2, 3
AXIS_TENSOR, AXIS_ROW, AXIS_COL = 0, 1, 2
AMAX_MOST_RECENT, AMAX_MAX = 0, 1
SCALE_TENSOR, SCALE_VECTOR = 0, 1
OUT_BF16, OUT_F32 = 0, 1

EXPORTED_SYMBOLS = (
    "fp8_query_device", "fp8_status_string", "fp8_last_error", "fp8_amax", "fp8_quantize_tensor",
    "fp8_quantize_row", "fp8_quantize_row_batch", "fp8_quantize_tensor_batch", "fp8_quantize_col",
    "fp8_quantize_rowcol", "fp8_delayed_scale_update", "fp8_gemm_scaled",
    "fp8_grouped_gemm_scaled", "fp8_grouped_quantize_col", "fp8_grouped_gemm_ragged_k",
    "fp8_mx_quantize_row", "fp8_gemm_mx", "fp8_grouped_gemm_mx", "fp8_moe_route", "fp8_moe_permute_quantize_row",
    "fp8_swiglu_quantize_row", "fp8_moe_unpermute_combine", "fp8_blockwise_quantize_act",
    "fp8_blockwise_quantize_weight",
)

GROUP_K_ALIGN = 256     # FP8_GROUP_K_ALIGN of the C header
MAX_ROW_BATCH = 8       # FP8_MAX_ROW_BATCH of the C header
MX_BLOCK = 32           # FP8_MX_BLOCK of the C header

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp8amax.so")


class Fp8Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class _DeviceInfo(ctypes.Structure):
    _fields_ = [("arch", ctypes.c_char * 64), ("is_gfx950", ctypes.c_int32), ("native_e4m3", ctypes.c_int32),
                ("native_e5m2", ctypes.c_int32), ("compute_units", ctypes.c_int32),
                ("lds_bytes_per_block", ctypes.c_int32), ("global_mem_bytes", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (or make -C "
                          f"{os.path.dirname(LIB_PATH)}) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    sigs = {
        "fp8_query_device": [I, ctypes.POINTER(_DeviceInfo)],
        "fp8_amax": [P, I64, I64, I64, I, P, P],
        "fp8_quantize_tensor": [P, I64, I64, I64, I, I32, P, P, I64, P, P, P],
        "fp8_quantize_row": [P, I64, I64, I64, I, I32, P, I64, P, P, P, P],
        "fp8_quantize_row_batch": [I32, P, P, I64, P, I, I32, P, P, P, P, P, P, P, P],
        "fp8_quantize_tensor_batch": [I32, P, P, I64, P, I, P, P, P, P, P, P],
        "fp8_quantize_col": [P, I64, I64, I64, I, I32, I32, P, I64, P, P, I32, P],
        "fp8_quantize_rowcol": [P, I64, I64, I64, I, I32, P, I64, P, P, P, I64, P, P, P],
        "fp8_delayed_scale_update": [P, P, P, I64, I32, I, I32, I, P, P, P],
        "fp8_gemm_scaled": [P, I, I64, P, I, I64, I64, I64, I64, P, I, P, I, P, I, I64, P],
        "fp8_grouped_gemm_scaled": [P, I, I64, P, I, I64, I64, P, I32, I64, I64, I64, P, P, P, I, I64, P],
        "fp8_grouped_quantize_col": [P, I64, I64, I64, I, I32, P, I32, P, I64, P, P, I32, P],
        "fp8_grouped_gemm_ragged_k": [P, I, I64, P, I, I64, P, I32, I64, I64, I64, P, P, P, I, I64, I64, P],
        "fp8_mx_quantize_row": [P, I64, I64, I64, I, P, I64, P, I64, P],
        "fp8_gemm_mx": [P, I, I64, P, I64, P, I, I64, P, I64, I64, I64, I64, P, I, I64, P],
        "fp8_grouped_gemm_mx": [P, I, I64, P, I64, P, I, I64, I64, P, I64, I64, P, I32, I64, I64, I64, P, I, I64, P],
        "fp8_moe_route": [P, I64, I32, I32, P, P, P],
        "fp8_blockwise_quantize_act": [P, I64, I64, I64, I, P, I64, P, I64, P],
        "fp8_blockwise_quantize_weight": [P, I64, I64, I64, I, P, I64, P, I64, P],
        "fp8_moe_permute_quantize_row": [P, I64, I64, I64, P, I32, I64, I, I32, P, I64, P, P],
        "fp8_swiglu_quantize_row": [P, I64, I64, I64, I, I32, P, I64, P, P],
        "fp8_moe_unpermute_combine": [P, I64, I64, I64, P, P, I64, I32, P, I64, P],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = I
    L.fp8_status_string.argtypes = [I]
    L.fp8_status_string.restype = ctypes.c_char_p
    L.fp8_last_error.argtypes = []
    L.fp8_last_error.restype = ctypes.c_char_p
    return L


lib = _load()


def _status_name(status):
    return lib.fp8_status_string(status).decode()


def fp8_status_string(status):
    return _status_name(status)


def _check(status):
    if status != 0:
        raise Fp8Error(status, lib.fp8_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t=None):
    dev = t.device if t is not None and t.is_cuda else None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _mat(t, name, elem_size=None):
    """(rows, cols, ld) of a 2-D row-major tensor with unit column stride."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if elem_size is not None and t.element_size() != elem_size:
        raise ValueError(f"{name} must have {elem_size}-byte elements, got {t.dtype}")
    if t.numel() > 0 and t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    return t.shape[0], t.shape[1], max(t.stride(0), t.shape[1], 1)


def _bf16(t, name="x"):
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be torch.bfloat16, got {t.dtype}")
    return _mat(t, name, 2)


def fp8_query_device(device=0):
    """Properties of HIP device `device` as a dict."""
    info = _DeviceInfo()
    _check(lib.fp8_query_device(int(device), ctypes.byref(info)))
    return {"arch": info.arch.decode(), "is_gfx950": bool(info.is_gfx950), "native_e4m3": info.native_e4m3,
            "native_e5m2": info.native_e5m2, "compute_units": info.compute_units,
            "lds_bytes_per_block": info.lds_bytes_per_block, "global_mem_bytes": info.global_mem_bytes}


def fp8_amax(x, axis, amax_out):
    rows, cols, ldx = _bf16(x)
    _check(lib.fp8_amax(_ptr(x), rows, cols, ldx, axis, _ptr(amax_out), _stream(x)))


def fp8_quantize_tensor(x, fmt, margin, scale, q, scale_inv_out, amax_out):
    rows, cols, ldx = _bf16(x)
    _, _, ldq = _mat(q, "q", 1)
    _check(lib.fp8_quantize_tensor(_ptr(x), rows, cols, ldx, fmt, margin, _ptr(scale), _ptr(q), ldq,
                                   _ptr(scale_inv_out), _ptr(amax_out), _stream(x)))


def fp8_quantize_row(x, fmt, margin, q, scale_inv_out, amax_out=None, col_amax_out=None):
    rows, cols, ldx = _bf16(x)
    _, _, ldq = _mat(q, "q", 1)
    _check(lib.fp8_quantize_row(_ptr(x), rows, cols, ldx, fmt, margin, _ptr(q), ldq, _ptr(scale_inv_out),
                                _ptr(amax_out), _ptr(col_amax_out), _stream(x)))


def fp8_quantize_row_batch(xs, fmt, margin, qs, scale_inv_outs, amax_outs=None, col_amax_outs=None,
                           col_group_offsets=None):
    """Rowwise casts of the bf16 tensors xs (same number of columns) in one
    launch; col_amax_outs[j] (fp32 [cols] or None) receives tensor j's column
    amax. With col_group_offsets[j] (a device int64 tensor [G + 1], or None),
    col_amax_outs[j] is fp32 [G x cols] and receives the column amax of each
    group of rows."""
    count = len(xs)
    if not (len(qs) == len(scale_inv_outs) == count) or (amax_outs is not None and len(amax_outs) != count) or (
            col_amax_outs is not None and len(col_amax_outs) != count) or (
            col_group_offsets is not None and len(col_group_offsets) != count):
        raise ValueError("xs, qs, scale_inv_outs (and amax_outs, col_amax_outs, col_group_offsets) must have the "
                         "same length")
    if count == 0:
        raise ValueError("no tensors")
    shapes = [_bf16(x) for x in xs]
    cols = shapes[0][1]
    if any(c != cols for _, c, _ in shapes):
        raise ValueError("the tensors of one batch share their number of columns")
    P64, PP = ctypes.c_int64 * count, ctypes.c_void_p * count
    xp = PP(*[_ptr(x) for x in xs])
    rows = P64(*[r for r, _, _ in shapes])
    ldx = P64(*[ld for _, _, ld in shapes])
    qp = PP(*[_ptr(q) for q in qs])
    ldq = P64(*[_mat(q, "q", 1)[2] for q in qs])
    sp = PP(*[_ptr(s) for s in scale_inv_outs])
    ap = PP(*[_ptr(a) for a in amax_outs]) if amax_outs is not None else None
    cp = PP(*[_ptr(c) for c in col_amax_outs]) if col_amax_outs is not None else None
    gp, gn = None, None
    if col_group_offsets is not None:
        for o in col_group_offsets:
            if o is not None and (o.dtype != torch.int64 or o.dim() != 1 or o.numel() < 2 or not o.is_contiguous()):
                raise ValueError("col_group_offsets entries are contiguous int64 tensors [G + 1]")
        gp = PP(*[_ptr(o) for o in col_group_offsets])
        gn = (ctypes.c_int32 * count)(*[o.numel() - 1 if o is not None else 0 for o in col_group_offsets])
    _check(lib.fp8_quantize_row_batch(count, xp, rows, cols, ldx, fmt, margin, qp, ldq, sp, ap, cp, gp, gn,
                                      _stream(xs[0])))


def fp8_quantize_tensor_batch(xs, fmt, scales, qs, scale_inv_outs, amax_outs):
    """Delayed tensorwise casts of the bf16 tensors xs (same number of columns)
    in one launch; scales[j] (device fp32 [1]) is tensor j's delayed scale."""
    count = len(xs)
    if count == 0 or not (len(scales) == len(qs) == len(scale_inv_outs) == len(amax_outs) == count):
        raise ValueError("xs, scales, qs, scale_inv_outs and amax_outs must have the same, nonzero length")
    shapes = [_bf16(x) for x in xs]
    cols = shapes[0][1]
    if any(c != cols for _, c, _ in shapes):
        raise ValueError("the tensors of one batch share their number of columns")
    P64, PP = ctypes.c_int64 * count, ctypes.c_void_p * count
    _check(lib.fp8_quantize_tensor_batch(
        count, PP(*[_ptr(x) for x in xs]), P64(*[r for r, _, _ in shapes]), cols, P64(*[ld for _, _, ld in shapes]),
        fmt, PP(*[_ptr(t) for t in scales]), PP(*[_ptr(q) for q in qs]), P64(*[_mat(q, "q", 1)[2] for q in qs]),
        PP(*[_ptr(t) for t in scale_inv_outs]), PP(*[_ptr(t) for t in amax_outs]), _stream(xs[0])))


def fp8_quantize_col(x, fmt, margin, q, scale_inv_out, col_amax, col_amax_ready=False, transpose_out=True):
    """Colwise scales; q is [cols x rows] (transpose_out) or [rows x cols]."""
    rows, cols, ldx = _bf16(x)
    _, _, ldq = _mat(q, "q", 1)
    _check(lib.fp8_quantize_col(_ptr(x), rows, cols, ldx, fmt, margin, int(bool(transpose_out)), _ptr(q), ldq,
                                _ptr(scale_inv_out), _ptr(col_amax), int(bool(col_amax_ready)), _stream(x)))


def fp8_quantize_rowcol(x, fmt, margin, q, scale_inv_out, amax_out, qt, col_scale_inv_out, col_amax_out):
    """Rowwise codes q [rows x cols] and colwise-transposed codes qt [cols x rows] of x in two passes."""
    rows, cols, ldx = _bf16(x)
    _, _, ldq = _mat(q, "q", 1)
    _, _, ldqt = _mat(qt, "qt", 1)
    _check(lib.fp8_quantize_rowcol(_ptr(x), rows, cols, ldx, fmt, margin, _ptr(q), ldq, _ptr(scale_inv_out),
                                   _ptr(amax_out), _ptr(qt), ldqt, _ptr(col_scale_inv_out), _ptr(col_amax_out),
                                   _stream(x)))


def fp8_delayed_scale_update(cur_amax, history, head, algo, margin, fmt, scale, scale_inv):
    """history: float32 [n x L]; head: int32 [1]; cur_amax, scale, scale_inv: float32 [n]."""
    n, L = history.shape
    _check(lib.fp8_delayed_scale_update(_ptr(cur_amax), _ptr(history), _ptr(head), n, L, algo, margin, fmt,
                                        _ptr(scale), _ptr(scale_inv), _stream(history)))


def fp8_gemm_scaled(a, fa, b, fb, a_scale_inv, a_mode, b_scale_inv, b_mode, d):
    """d [m x n] = (a [m x k] codes) * (b [n x k] codes)^T, scaled; d bf16 or float32."""
    m, k, lda = _mat(a, "a", 1)
    n, kb, ldb = _mat(b, "b", 1)
    if kb != k:
        raise ValueError(f"a has k = {k} but b has k = {kb}")
    _, _, ldd = _mat(d, "d")
    d_type = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[d.dtype]
    _check(lib.fp8_gemm_scaled(_ptr(a), fa, lda, _ptr(b), fb, ldb, m, n, k, _ptr(a_scale_inv), a_mode,
                               _ptr(b_scale_inv), b_mode, _ptr(d), d_type, ldd, _stream(a)))


def fp8_grouped_gemm_scaled(a, fa, b, fb, group_offsets, a_scale_inv, b_scale_inv, d):
    """a [total_m x k] codes sorted by group; b [g x n x k] codes; group_offsets int64 [g+1]
    on the device; a_scale_inv [total_m]; b_scale_inv [g x n]; d [total_m x n]."""
    total_m, k, lda = _mat(a, "a", 1)
    if b.dim() != 3 or b.element_size() != 1 or (b.numel() > 0 and b.shape[2] > 1 and b.stride(2) != 1):
        raise ValueError("b must be a [g x n x k] 1-byte tensor with unit last stride")
    g, n, kb = b.shape
    if kb != k:
        raise ValueError(f"a has k = {k} but b has k = {kb}")
    _, _, ldd = _mat(d, "d")
    d_type = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[d.dtype]
    if group_offsets.dtype != torch.int64 or group_offsets.numel() != g + 1:
        raise ValueError("group_offsets must be int64 with g + 1 entries")
    _check(lib.fp8_grouped_gemm_scaled(_ptr(a), fa, lda, _ptr(b), fb, max(b.stride(1), k), b.stride(0),
                                       _ptr(group_offsets), g, total_m, n, k, _ptr(a_scale_inv),
                                       _ptr(b_scale_inv), _ptr(d), d_type, ldd, _stream(a)))


def grouped_layout_width(total_m, g):
    """Columns that always hold the grouped transposed layout of total_m rows in
    g groups (each group padded to GROUP_K_ALIGN), rounded up to 16."""
    w = total_m + g * (GROUP_K_ALIGN - 1)
    return (w + 15) // 16 * 16


def fp8_grouped_quantize_col(x, fmt, margin, group_offsets, qt, scale_inv_out, col_amax, col_amax_ready=False):
    """x bf16 [total_m x cols], rows sorted by group; group_offsets int64 [g+1] on the
    device; qt codes [cols x L] with L >= the layout width (grouped_layout_width
    always suffices); scale_inv_out and col_amax fp32 [g x cols]."""
    total_m, cols, ldx = _bf16(x)
    qr, _, ldqt = _mat(qt, "qt", 1)
    if qr != cols:
        raise ValueError(f"qt must have {cols} rows (one per column of x), got {qr}")
    if group_offsets.dtype != torch.int64 or group_offsets.dim() != 1:
        raise ValueError("group_offsets must be a 1-D int64 tensor")
    g = group_offsets.numel() - 1
    _check(lib.fp8_grouped_quantize_col(_ptr(x), total_m, cols, ldx, fmt, margin, _ptr(group_offsets), g, _ptr(qt),
                                        ldqt, _ptr(scale_inv_out), _ptr(col_amax), int(bool(col_amax_ready)),
                                        _stream(x)))


def fp8_grouped_gemm_ragged_k(a, fa, b, fb, group_offsets, total_m, a_scale_inv, b_scale_inv, d):
    """a codes [m x L], b codes [n x L] in the grouped transposed layout of total_m
    rows; group_offsets int64 [g+1] on the device; a_scale_inv fp32 [g x m],
    b_scale_inv fp32 [g x n]; d [g x m x n] bf16 or fp32 (unit last stride)."""
    m, _, lda = _mat(a, "a", 1)
    n, _, ldb = _mat(b, "b", 1)
    if d.dim() != 3 or (d.numel() > 0 and d.shape[2] > 1 and d.stride(2) != 1):
        raise ValueError("d must be a [g x m x n] tensor with unit last stride")
    g = group_offsets.numel() - 1
    if tuple(d.shape) != (g, m, n):
        raise ValueError(f"d must have shape {(g, m, n)}, got {tuple(d.shape)}")
    d_type = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[d.dtype]
    ldd = max(d.stride(1), n, 1)
    _check(lib.fp8_grouped_gemm_ragged_k(_ptr(a), fa, lda, _ptr(b), fb, ldb, _ptr(group_offsets), g, total_m, m, n,
                                         _ptr(a_scale_inv), _ptr(b_scale_inv), _ptr(d), d_type, ldd, d.stride(0),
                                         _stream(a)))


def mx_scale_records(rows, cols, device="cuda:0"):
    """An empty uint8 [ceil(cols/128) x rows x 4] tensor: the MX scale records
    of a [rows x cols] matrix (record (j, r) holds the scales of blocks
    4j .. 4j+3 of row r)."""
    return torch.empty(((cols + 127) // 128, rows, 4), dtype=torch.uint8, device=device)


def _records(t, name):
    """(record rows J, rows, ld) of a uint8 [J x rows x 4] record tensor."""
    if t.dim() != 3 or t.element_size() != 1 or t.shape[2] != 4:
        raise ValueError(f"{name} must be a 1-byte [J x rows x 4] tensor, got {tuple(t.shape)} {t.dtype}")
    if t.numel() > 0 and (t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != 4) or
                          (t.shape[0] > 1 and t.stride(0) % 4 != 0)):
        raise ValueError(f"{name} must hold contiguous 4-byte records, rows contiguous")
    ld = t.stride(0) // 4 if t.shape[0] > 1 else t.shape[1]
    return t.shape[0], t.shape[1], max(ld, t.shape[1], 1)


def fp8_mx_quantize_row(x, fmt, q, scale_e8m0):
    """x bf16 [rows x cols] (cols % 32 == 0); q codes [rows x cols]; scale_e8m0
    uint8 records [ceil(cols/128) x rows x 4] (mx_scale_records)."""
    rows, cols, ldx = _bf16(x)
    _, _, ldq = _mat(q, "q", 1)
    J, r, lds = _records(scale_e8m0, "scale_e8m0")
    if r != rows or J != (cols + 127) // 128:
        raise ValueError(f"scale_e8m0 must be [{(cols + 127) // 128} x {rows} x 4], got {tuple(scale_e8m0.shape)}")
    _check(lib.fp8_mx_quantize_row(_ptr(x), rows, cols, ldx, fmt, _ptr(q), ldq, _ptr(scale_e8m0), lds, _stream(x)))


def fp8_gemm_mx(a, fa, a_scale, b, fb, b_scale, d):
    """d [m x n] = block-scaled (a [m x k] codes, a_scale records [k/128 x m x 4])
    times (b [n x k] codes, b_scale records [k/128 x n x 4])^T; d bf16 or float32."""
    m, k, lda = _mat(a, "a", 1)
    n, kb, ldb = _mat(b, "b", 1)
    if kb != k:
        raise ValueError(f"a has k = {k} but b has k = {kb}")
    _, _, ldas = _records(a_scale, "a_scale")
    _, _, ldbs = _records(b_scale, "b_scale")
    _, _, ldd = _mat(d, "d")
    d_type = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[d.dtype]
    _check(lib.fp8_gemm_mx(_ptr(a), fa, lda, _ptr(a_scale), ldas, _ptr(b), fb, ldb, _ptr(b_scale), ldbs, m, n, k,
                           _ptr(d), d_type, ldd, _stream(a)))


def fp8_grouped_gemm_mx(a, fa, a_scale, b, fb, b_scale, group_offsets, d):
    """a [total_m x k] codes sorted by group with a_scale records [k/128 x total_m x 4];
    b [g x n x k] codes (unit last stride) with b_scale records [g x k/128 x n x 4];
    group_offsets int64 [g+1] on the device; d [total_m x n]."""
    total_m, k, lda = _mat(a, "a", 1)
    _, _, ldas = _records(a_scale, "a_scale")
    if b.dim() != 3 or b.element_size() != 1 or (b.numel() > 0 and b.shape[2] > 1 and b.stride(2) != 1):
        raise ValueError("b must be a [g x n x k] 1-byte tensor with unit last stride")
    g, n, kb = b.shape
    if b_scale.dim() != 4 or b_scale.shape[0] != g:
        raise ValueError(f"b_scale must be [{g} x k/128 x {n} x 4], got {tuple(b_scale.shape)}")
    _, nb, ldbs = _records(b_scale[0], "b_scale[g]")
    if kb != k or nb != n:
        raise ValueError(f"b {tuple(b.shape)} / b_scale {tuple(b_scale.shape)} do not match a's k = {k}")
    _, _, ldd = _mat(d, "d")
    d_type = {torch.bfloat16: OUT_BF16, torch.float32: OUT_F32}[d.dtype]
    if group_offsets.dtype != torch.int64 or group_offsets.numel() != g + 1:
        raise ValueError("group_offsets must be int64 with g + 1 entries")
    _check(lib.fp8_grouped_gemm_mx(_ptr(a), fa, lda, _ptr(a_scale), ldas, _ptr(b), fb, max(b.stride(1), k),
                                   b.stride(0), _ptr(b_scale), ldbs, b_scale.stride(0), _ptr(group_offsets), g,
                                   total_m, n, k, _ptr(d), d_type, ldd, _stream(a)))


def _i32_2d(t, name):
    if t.dim() != 2 or t.dtype != torch.int32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 [tokens x topk] tensor")
    return t.shape[0], t.shape[1]


def fp8_moe_route(expert_idx, num_experts, offsets_out, dest_out):
    """expert_idx int32 [T x k] -> offsets_out int64 [E+1], dest_out int32 [T x k]."""
    T, k = _i32_2d(expert_idx, "expert_idx")
    if tuple(dest_out.shape) != (T, k) or dest_out.dtype != torch.int32 or not dest_out.is_contiguous():
        raise ValueError(f"dest_out must be a contiguous int32 [{T} x {k}] tensor")
    if offsets_out.dtype != torch.int64 or offsets_out.numel() != num_experts + 1:
        raise ValueError(f"offsets_out must be int64 with {num_experts + 1} entries")
    _check(lib.fp8_moe_route(_ptr(expert_idx), T, k, num_experts, _ptr(offsets_out), _ptr(dest_out),
                             _stream(expert_idx)))


def fp8_moe_permute_quantize_row(x, dest, fmt, margin, q, scale_inv_out):
    """x bf16 [T x H]; dest int32 [T x k] (fp8_moe_route); q codes [rows_out x H];
    scale_inv_out fp32 [rows_out]."""
    T, H, ldx = _bf16(x)
    Td, k = _i32_2d(dest, "dest")
    if Td != T:
        raise ValueError(f"dest has {Td} rows, x has {T}")
    rows_out, qc, ldq = _mat(q, "q", 1)
    if qc != H:
        raise ValueError(f"q must have {H} columns")
    _check(lib.fp8_moe_permute_quantize_row(_ptr(x), T, H, ldx, _ptr(dest), k, rows_out, fmt, margin, _ptr(q), ldq,
                                            _ptr(scale_inv_out), _stream(x)))


def fp8_swiglu_quantize_row(h, fmt, margin, q, scale_inv_out):
    """h bf16 [rows x 2I] (gate | up); q codes [rows x I]; scale_inv_out fp32 [rows]."""
    rows, two_i, ldh = _bf16(h, "h")
    if two_i % 2:
        raise ValueError("h must have an even number of columns (gate | up)")
    _, _, ldq = _mat(q, "q", 1)
    _check(lib.fp8_swiglu_quantize_row(_ptr(h), rows, two_i // 2, ldh, fmt, margin, _ptr(q), ldq,
                                       _ptr(scale_inv_out), _stream(h)))


def fp8_moe_unpermute_combine(y, dest, weights, out):
    """y bf16 [rows x H] in expert order; dest int32 [T x k]; weights fp32 [T x k];
    out bf16 [T x H]."""
    rows, H, ldy = _bf16(y, "y")
    T, k = _i32_2d(dest, "dest")
    if tuple(weights.shape) != (T, k) or weights.dtype != torch.float32 or not weights.is_contiguous():
        raise ValueError(f"weights must be a contiguous float32 [{T} x {k}] tensor")
    To, Ho, ldo = _bf16(out, "out")
    if (To, Ho) != (T, H):
        raise ValueError(f"out must be [{T} x {H}]")
    _check(lib.fp8_moe_unpermute_combine(_ptr(y), rows, H, ldy, _ptr(dest), _ptr(weights), T, k, _ptr(out), ldo,
                                         _stream(y)))


def _blockwise(fn, x, fmt, q, scale_records):
    rows, cols, ldx = _bf16(x)
    _, _, ldq = _mat(q, "q", 1)
    J, r, lds = _records(scale_records, "scale_records")
    if r != rows or J != (cols + 127) // 128:
        raise ValueError(f"scale_records must be [{(cols + 127) // 128} x {rows} x 4]")
    _check(fn(_ptr(x), rows, cols, ldx, fmt, _ptr(q), ldq, _ptr(scale_records), lds, _stream(x)))


def fp8_blockwise_quantize_act(x, fmt, q, scale_records):
    """1 x 128 blocks: x bf16 [rows x cols] (cols % 128 == 0); q codes; scale
    records uint8 [cols/128 x rows x 4] (mx_scale_records), for fp8_gemm_mx."""
    _blockwise(lib.fp8_blockwise_quantize_act, x, fmt, q, scale_records)


def fp8_blockwise_quantize_weight(w, fmt, q, scale_records):
    """128 x 128 tiles: as fp8_blockwise_quantize_act, one scale per tile."""
    _blockwise(lib.fp8_blockwise_quantize_weight, w, fmt, q, scale_records)
