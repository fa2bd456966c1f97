"""The C ABI library loads, exports every function include/fp8amax.h declares,
and rejects bad arguments on the host before anything is launched. CPU only:
no call here reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8amax.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fp8_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def fp8():
    import fp8_scaled_gemm_amax_amd as m
    return m


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("fp8_amax", "fp8_quantize_tensor", "fp8_quantize_row", "fp8_quantize_col",
                     "fp8_delayed_scale_update", "fp8_gemm_scaled", "fp8_grouped_gemm_scaled",
                     "fp8_query_device", "fp8_status_string", "fp8_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol(fp8):
    lib = ctypes.CDLL(fp8.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fp8.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (fp8_\w+)", out.stdout))
    assert set(declared_functions()) <= exported
    assert set(fp8.EXPORTED_SYMBOLS) == set(declared_functions())


def test_library_has_gfx950_code_object(fp8):
    """The embedded offload bundle carries a gfx950 code object (bundle entry id)."""
    blob = open(fp8.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings(fp8):
    assert fp8.fp8_status_string(0) == "FP8_OK"
    assert fp8.fp8_status_string(1) == "FP8_ERR_INVALID_ARG"
    assert fp8.fp8_status_string(3) == "FP8_ERR_UNSUPPORTED"


def _call(fp8, name, *args):
    st = getattr(fp8.lib, name)(*args)
    return st, fp8.lib.fp8_last_error().decode()


FAKE = ctypes.c_void_p(0x10000)     # never dereferenced: every call below fails validation first


def test_gemm_rejects_bad_arguments(fp8):
    g = "fp8_gemm_scaled"
    # k not a multiple of 16
    st, msg = _call(fp8, g, FAKE, 0, 32, FAKE, 0, 32, 8, 8, 24, FAKE, 1, FAKE, 1, FAKE, 0, 8, None)
    assert st == 1 and "multiple of 16" in msg
    # negative size
    st, _ = _call(fp8, g, FAKE, 0, 32, FAKE, 0, 32, -1, 8, 32, FAKE, 1, FAKE, 1, FAKE, 0, 8, None)
    assert st == 1
    # misaligned operand
    st, _ = _call(fp8, g, ctypes.c_void_p(0x10001), 0, 32, FAKE, 0, 32, 8, 8, 32, FAKE, 1, FAKE, 1, FAKE, 0, 8, None)
    assert st == 2
    # lda not a multiple of 16
    st, _ = _call(fp8, g, FAKE, 0, 40, FAKE, 0, 32, 8, 8, 32, FAKE, 1, FAKE, 1, FAKE, 0, 8, None)
    assert st == 2
    # fnuz operands are accepted (the bf16 compatibility path) and validated like
    # the others: here ldd < n
    st, msg = _call(fp8, g, FAKE, 2, 32, FAKE, 3, 32, 8, 8, 32, FAKE, 1, FAKE, 1, FAKE, 0, 4, None)
    assert st == 1 and "leading dimension" in msg
    # unknown format / output type / scale mode
    assert _call(fp8, g, FAKE, 7, 32, FAKE, 0, 32, 8, 8, 32, FAKE, 1, FAKE, 1, FAKE, 0, 8, None)[0] == 1
    assert _call(fp8, g, FAKE, 0, 32, FAKE, 0, 32, 8, 8, 32, FAKE, 1, FAKE, 1, FAKE, 5, 8, None)[0] == 1
    assert _call(fp8, g, FAKE, 0, 32, FAKE, 0, 32, 8, 8, 32, FAKE, 4, FAKE, 1, FAKE, 0, 8, None)[0] == 1
    # NULL output
    assert _call(fp8, g, FAKE, 0, 32, FAKE, 0, 32, 8, 8, 32, FAKE, 1, FAKE, 1, None, 0, 8, None)[0] == 1


def test_grouped_gemm_rejects_bad_arguments(fp8):
    g = "fp8_grouped_gemm_scaled"
    ok_args = [FAKE, 0, 32, FAKE, 0, 32, 8 * 32, FAKE, 4, 64, 8, 32, FAKE, FAKE, FAKE, 0, 8, None]
    bad = list(ok_args)
    bad[8] = 0                      # no groups
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[7] = None                   # no offsets
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[6] = -16                    # negative group stride (smaller ones may interleave, by design)
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[6] = 8                      # group stride off the 16-byte grid
    assert _call(fp8, g, *bad)[0] == 2
    bad = list(ok_args)
    bad[7] = ctypes.c_void_p(0x10004)
    assert _call(fp8, g, *bad)[0] == 2


def test_grouped_quantize_col_rejects_bad_arguments(fp8):
    g = "fp8_grouped_quantize_col"
    # x [64 x 32] bf16, 4 groups, qt [32 x 1088]
    ok_args = [FAKE, 64, 32, 32, 0, 0, FAKE, 4, FAKE, 1088, FAKE, FAKE, 0, None]
    bad = list(ok_args)
    bad[7] = 0                      # no groups
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[7] = 5000                   # too many groups
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[6] = None                   # no offsets
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[9] = 48                     # ldqt < total_m
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[9] = 1096                   # ldqt off the 16-byte grid
    assert _call(fp8, g, *bad)[0] == 2
    bad = list(ok_args)
    bad[2], bad[3] = 36, 36         # cols not a multiple of 8
    assert _call(fp8, g, *bad)[0] == 2
    bad = list(ok_args)
    bad[10] = None                  # no scale output
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[12] = 2                     # col_amax_ready not 0 / 1
    assert _call(fp8, g, *bad)[0] == 1


def test_grouped_gemm_ragged_k_rejects_bad_arguments(fp8):
    g = "fp8_grouped_gemm_ragged_k"
    # a [64 x 1088], b [96 x 1088], 4 groups over 64 tokens, d [4 x 64 x 96]
    ok_args = [FAKE, 1, 1088, FAKE, 0, 1088, FAKE, 4, 64, 64, 96, FAKE, FAKE, FAKE, 0, 96, 64 * 96, None]
    bad = list(ok_args)
    bad[1] = 2                      # fnuz operand
    assert _call(fp8, g, *bad)[0] == 3
    bad = list(ok_args)
    bad[7] = 0                      # no groups
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[2] = 32                     # lda < total_m
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[16] = 64 * 96 - 1           # output groups overlap
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[6] = None                   # no offsets
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_args)
    bad[0] = ctypes.c_void_p(0x10008)
    assert _call(fp8, g, *bad)[0] == 2


def test_quantizers_reject_bad_arguments(fp8):
    # margin out of range
    st, msg = _call(fp8, "fp8_quantize_row", FAKE, 4, 16, 16, 0, 33, FAKE, 16, FAKE, None, None, None)
    assert st == 1 and "margin" in msg
    # ld smaller than the row
    assert _call(fp8, "fp8_quantize_row", FAKE, 4, 16, 8, 0, 0, FAKE, 16, FAKE, None, None, None)[0] == 1
    # unknown format
    assert _call(fp8, "fp8_quantize_row", FAKE, 4, 16, 16, 9, 0, FAKE, 16, FAKE, None, None, None)[0] == 1
    # x misaligned for bf16
    assert _call(fp8, "fp8_quantize_row", ctypes.c_void_p(0x10001), 4, 16, 16, 0, 0, FAKE, 16, FAKE, None, None,
                 None)[0] == 2
    # tensorwise needs scale_inv_out and amax_out
    assert _call(fp8, "fp8_quantize_tensor", FAKE, 4, 16, 16, 0, 0, None, FAKE, 16, None, FAKE, None)[0] == 1
    # colwise: transposed output needs ldq >= rows, untransposed ldq >= cols;
    # col_amax_ready and transpose_out must be 0/1
    assert _call(fp8, "fp8_quantize_col", FAKE, 64, 16, 16, 0, 0, 1, FAKE, 32, FAKE, FAKE, 0, None)[0] == 1
    assert _call(fp8, "fp8_quantize_col", FAKE, 64, 16, 16, 0, 0, 1, FAKE, 64, FAKE, FAKE, 2, None)[0] == 1
    st, msg = _call(fp8, "fp8_quantize_col", FAKE, 64, 16, 16, 0, 0, 0, FAKE, 8, FAKE, FAKE, 0, None)
    assert st == 1 and "leading dimension" in msg
    st, msg = _call(fp8, "fp8_quantize_col", FAKE, 64, 16, 16, 0, 0, 2, FAKE, 64, FAKE, FAKE, 0, None)
    assert st == 1 and "transpose_out" in msg
    # amax: unknown axis
    assert _call(fp8, "fp8_amax", FAKE, 4, 16, 16, 3, FAKE, None)[0] == 1


def test_quantize_row_batch_rejects_bad_arguments(fp8):
    f = "fp8_quantize_row_batch"
    PP, P64 = ctypes.c_void_p * 2, ctypes.c_int64 * 2
    x, q, s = PP(FAKE, FAKE), PP(FAKE, FAKE), PP(FAKE, FAKE)
    rows, ld = P64(4, 8), P64(16, 16)

    def call(count=2, x=x, rows=rows, cols=16, ldx=ld, fmt=0, margin=0, q=q, ldq=ld, s=s, a=None, ca=None, go=None,
             gn=None):
        return _call(fp8, f, count, x, rows, cols, ldx, fmt, margin, q, ldq, s, a, ca, go, gn, None)

    st, msg = call(count=0)
    assert st == 1 and "count" in msg
    assert call(count=fp8.MAX_ROW_BATCH + 1)[0] == 1
    assert call(x=None)[0] == 1                                   # a host array is missing
    assert call(margin=33)[0] == 1
    assert call(fmt=9)[0] == 1
    st, msg = call(ldx=P64(16, 8))                                # tensor 1: ld smaller than the row
    assert st == 1 and "leading dimension" in msg
    assert call(s=PP(FAKE, None))[0] == 1                         # tensor 1 has rows but no scale output
    assert call(x=PP(FAKE, ctypes.c_void_p(0x10001)))[0] == 2     # tensor 1 misaligned for bf16
    assert call(a=PP(None, ctypes.c_void_p(0x10002)))[0] == 2     # misaligned amax output
    assert call(ca=PP(ctypes.c_void_p(0x10002), None))[0] == 2    # misaligned column-amax output
    # grouped column amax: group counts 0..4096, offsets required and 8-byte aligned, an output for every grouped
    # tensor, the vector layout and cols <= 16384
    G32 = ctypes.c_int32 * 2
    ca = PP(FAKE, FAKE)
    st, msg = call(ca=ca, go=PP(FAKE, None), gn=G32(4097, 0))
    assert st == 1 and "col_groups" in msg
    assert call(ca=ca, go=PP(None, None), gn=G32(3, 0))[0] == 1
    assert call(ca=ca, go=None, gn=G32(3, 0))[0] == 1
    assert call(ca=PP(None, FAKE), go=PP(FAKE, None), gn=G32(3, 0))[0] == 1
    assert call(ca=ca, go=PP(ctypes.c_void_p(0x10004), None), gn=G32(3, 0))[0] == 2
    assert call(ca=ca, go=PP(FAKE, None), gn=G32(3, 0), cols=12, ldx=P64(12, 12), ldq=P64(12, 12))[0] == 2
    assert call(ca=ca, go=PP(FAKE, None), gn=G32(3, 0), cols=16392, ldx=P64(16392, 16392),
                ldq=P64(16392, 16392))[0] == 3


def test_quantize_tensor_batch_rejects_bad_arguments(fp8):
    f = "fp8_quantize_tensor_batch"
    PP, P64 = ctypes.c_void_p * 2, ctypes.c_int64 * 2
    two = PP(FAKE, FAKE)
    rows, ld = P64(4, 8), P64(16, 16)

    def call(count=2, x=two, rows=rows, ldx=ld, fmt=0, sc=two, ldq=ld, si=two, am=two):
        return _call(fp8, f, count, x, rows, 16, ldx, fmt, sc, two, ldq, si, am, None)

    st, msg = call(count=9)
    assert st == 1 and "count" in msg
    assert call(sc=None)[0] == 1                                   # the scale array is required
    st, msg = call(sc=PP(FAKE, None))                              # tensor 1 without its delayed scale
    assert st == 1 and "required" in msg
    assert call(am=PP(FAKE, None))[0] == 1
    assert call(fmt=7)[0] == 1
    assert call(ldq=P64(16, 4))[0] == 1
    assert call(si=PP(FAKE, ctypes.c_void_p(0x10002)))[0] == 2


def test_delayed_update_rejects_bad_arguments(fp8):
    f = "fp8_delayed_scale_update"
    assert _call(fp8, f, FAKE, FAKE, FAKE, 2, 0, 1, 0, 0, FAKE, FAKE, None)[0] == 1        # L = 0
    assert _call(fp8, f, FAKE, FAKE, FAKE, 2, 1024, 2, 0, 0, FAKE, FAKE, None)[0] == 1     # algo
    assert _call(fp8, f, FAKE, FAKE, None, 2, 1024, 1, 0, 0, FAKE, FAKE, None)[0] == 1     # head
    assert _call(fp8, f, FAKE, FAKE, FAKE, 2, 1024, 1, -1, 0, FAKE, FAKE, None)[0] == 1    # margin


def test_query_device_rejects_null(fp8):
    assert fp8.lib.fp8_query_device(0, None) == 1


def test_mx_entry_points_reject_bad_arguments(fp8):
    q = "fp8_mx_quantize_row"
    # x [4 x 64] bf16, q [4 x 64], one K step of 4 scale records
    ok_q = [FAKE, 4, 64, 64, 0, FAKE, 64, FAKE, 4, None]
    bad = list(ok_q)
    bad[2], bad[3], bad[6] = 48, 64, 64      # cols not a multiple of 32
    assert _call(fp8, q, *bad)[0] == 1
    bad = list(ok_q)
    bad[4] = 2                               # fnuz elements
    assert _call(fp8, q, *bad)[0] == 1
    bad = list(ok_q)
    bad[8] = 3                               # record stride < rows
    assert _call(fp8, q, *bad)[0] == 1
    bad = list(ok_q)
    bad[7] = ctypes.c_void_p(0x10002)        # scale records off the dword grid
    assert _call(fp8, q, *bad)[0] == 2
    bad = list(ok_q)
    bad[5] = ctypes.c_void_p(0x10004)        # q off the 8-byte grid
    assert _call(fp8, q, *bad)[0] == 2
    bad = list(ok_q)
    bad[1] = bad[8] = 1 << 26                # too many rows
    assert _call(fp8, q, *bad)[0] == 3
    g = "fp8_gemm_mx"
    # a [64 x 512], b [32 x 512], scale records with ld = rows, d [64 x 32]
    ok_g = [FAKE, 0, 512, FAKE, 64, FAKE, 0, 512, FAKE, 32, 64, 32, 512, FAKE, 0, 32, None]
    bad = list(ok_g)
    bad[12], bad[2], bad[7] = 384, 384, 384  # k not a multiple of 256
    st, msg = _call(fp8, g, *bad)
    assert st == 3 and "256" in msg
    bad = list(ok_g)
    bad[4] = 63                              # record stride < m
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_g)
    bad[8] = ctypes.c_void_p(0x10006)        # scale records off the dword grid
    assert _call(fp8, g, *bad)[0] == 2
    bad = list(ok_g)
    bad[3] = None                            # no scales
    assert _call(fp8, g, *bad)[0] == 1
    bad = list(ok_g)
    bad[6] = 3                               # fnuz operand
    assert _call(fp8, g, *bad)[0] == 3
    gg = "fp8_grouped_gemm_mx"
    # a [64 x 512], 4 groups of b [32 x 512], scale records with ld = rows
    ok_gg = [FAKE, 0, 512, FAKE, 64, FAKE, 1, 512, 32 * 512, FAKE, 32, 4 * 32 * 4, FAKE, 4, 64, 32, 512, FAKE, 0, 32,
             None]
    bad = list(ok_gg)
    bad[13] = 0                              # no groups
    assert _call(fp8, gg, *bad)[0] == 1
    bad = list(ok_gg)
    bad[11] = 514                            # scale group stride off the dword grid
    assert _call(fp8, gg, *bad)[0] == 2
    bad = list(ok_gg)
    bad[11] = -4                             # negative scale group stride
    assert _call(fp8, gg, *bad)[0] == 1
    bad = list(ok_gg)
    bad[12] = None                           # no offsets
    assert _call(fp8, gg, *bad)[0] == 1


def test_moe_layer_entry_points_reject_bad_arguments(fp8):
    r = "fp8_moe_route"
    ok_r = [FAKE, 100, 8, 32, FAKE, FAKE, None]
    for i, v, st in ((2, 0, 1), (2, 65, 1), (3, 0, 1), (3, 1025, 1), (1, -1, 1), (4, None, 1),
                     (4, ctypes.c_void_p(0x10004), 2), (5, ctypes.c_void_p(0x10002), 2)):
        bad = list(ok_r)
        bad[i] = v
        assert _call(fp8, r, *bad)[0] == st, (i, v)
    bad = list(ok_r)
    bad[1], bad[2] = 1 << 30, 2               # 2^31 entries
    assert _call(fp8, r, *bad)[0] == 3
    p = "fp8_moe_permute_quantize_row"
    # x [100 x 64], dest [100 x 8], q [800 x 64]
    ok_p = [FAKE, 100, 64, 64, FAKE, 8, 800, 0, 0, FAKE, 64, FAKE, None]
    for i, v, st in ((5, 0, 1), (8, 33, 1), (7, 9, 1), (10, 32, 1), (4, None, 1), (11, None, 1),
                     (9, ctypes.c_void_p(0x10004), 2), (0, ctypes.c_void_p(0x10008), 2)):
        bad = list(ok_p)
        bad[i] = v
        assert _call(fp8, p, *bad)[0] == st, (i, v)
    bad = list(ok_p)
    bad[2], bad[3], bad[10] = 16392, 16392, 16392          # rows longer than 16384
    assert _call(fp8, p, *bad)[0] == 3
    s = "fp8_swiglu_quantize_row"
    # h [64 x 2*256], q [64 x 256]
    ok_s = [FAKE, 64, 256, 512, 0, 0, FAKE, 256, FAKE, None]
    for i, v, st in ((3, 256, 1), (8, None, 1), (2, 252, 2), (6, ctypes.c_void_p(0x10004), 2), (4, 7, 1)):
        bad = list(ok_s)
        bad[i] = v
        assert _call(fp8, s, *bad)[0] == st, (i, v)
    bad = list(ok_s)
    bad[2], bad[3], bad[7] = 4104, 8208, 4104              # intermediate size above 4096
    assert _call(fp8, s, *bad)[0] == 3
    c = "fp8_moe_unpermute_combine"
    # y [800 x 64], dest / weights [100 x 8], out [100 x 64]
    ok_c = [FAKE, 800, 64, 64, FAKE, FAKE, 100, 8, FAKE, 64, None]
    for i, v, st in ((7, 0, 1), (4, None, 1), (5, None, 1), (9, 32, 1), (8, ctypes.c_void_p(0x10008), 2),
                     (2, 60, 2)):
        bad = list(ok_c)
        bad[i] = v
        assert _call(fp8, c, *bad)[0] == st, (i, v)


def test_blockwise_entry_points_reject_bad_arguments(fp8):
    for f in ("fp8_blockwise_quantize_act", "fp8_blockwise_quantize_weight"):
        ok = [FAKE, 4, 256, 256, 0, FAKE, 256, FAKE, 4, None]
        for i, v, st in ((2, 192, 1), (4, 2, 1), (8, 3, 1), (7, None, 1), (7, ctypes.c_void_p(0x10002), 2),
                         (5, ctypes.c_void_p(0x10004), 2), (3, 260, 2)):
            bad = list(ok)
            bad[i] = v
            if i == 2:
                bad[3], bad[6] = 192, 192
            assert _call(fp8, f, *bad)[0] == st, (f, i, v)
