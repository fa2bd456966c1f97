// api.cpp - the C ABI of include/fp8amax.h: argument validation (before any
// launch), the per-device properties cache, and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/fp8amax.h"
#include "kernels.hpp"

namespace fp8amax {

namespace {

thread_local char g_err[512] = "";

fp8_status_t fail(fp8_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

fp8_status_t ok() {
    g_err[0] = '\0';
    return FP8_OK;
}

constexpr int kMaxDevices = 64;
struct PropsSlot {
    std::once_flag once;
    DeviceProps props{};
    bool gfx950 = false;
    hipError_t err = hipSuccess;
};
PropsSlot g_props[kMaxDevices];

PropsSlot* slot_for_current(int* dev_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    PropsSlot& s = g_props[dev];
    std::call_once(s.once, [&s, dev]() {
        hipDeviceProp_t p;
        s.err = hipGetDeviceProperties(&p, dev);
        if (s.err == hipSuccess) {
            s.props.cus = p.multiProcessorCount;
            s.gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        }
    });
    if (dev_out) *dev_out = dev;
    return &s;
}

bool valid_fmt(int f) { return f >= FP8_E4M3 && f <= FP8_E5M2_FNUZ; }
bool ocp_fmt(int f) { return f == FP8_E4M3 || f == FP8_E5M2; }
bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Device check shared by every compute entry point (after argument checks).
fp8_status_t check_device() {
    int dev = 0;
    PropsSlot* s = slot_for_current(&dev);
    if (!s) return fail(FP8_ERR_HIP, "cannot query the current HIP device");
    if (s->err != hipSuccess) return fail(FP8_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(s->err));
    if (!s->gfx950) return fail(FP8_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X); this library is built for gfx950 only", dev);
    return FP8_OK;
}

fp8_status_t launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

fp8_status_t check_matrix(const char* fn, const char* name, const void* p, int64_t rows, int64_t cols, int64_t ld) {
    if (rows < 0 || cols < 0) return fail(FP8_ERR_INVALID_ARG, "%s: %s has negative size %lld x %lld", fn, name,
                                          (long long)rows, (long long)cols);
    if (ld < cols || ld < 1) return fail(FP8_ERR_INVALID_ARG, "%s: leading dimension of %s (%lld) < max(cols, 1) (%lld)",
                                        fn, name, (long long)ld, (long long)cols);
    if (!p && rows > 0 && cols > 0) return fail(FP8_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
    return FP8_OK;
}

#define FP8_TRY(expr)                          \
    do {                                       \
        fp8_status_t _s = (expr);              \
        if (_s != FP8_OK) return _s;           \
    } while (0)

fp8_status_t check_common_quant(const char* fn, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                int margin) {
    FP8_TRY(check_matrix(fn, "x", x, rows, cols, ldx));
    if (!valid_fmt(fmt)) return fail(FP8_ERR_INVALID_ARG, "%s: unknown format %d", fn, fmt);
    if (margin < 0 || margin > 32) return fail(FP8_ERR_INVALID_ARG, "%s: margin %d outside 0..32", fn, margin);
    if (!aligned(x, 2)) return fail(FP8_ERR_ALIGNMENT, "%s: x is not 2-byte aligned", fn);
    return FP8_OK;
}

// fnuz_ok: the product has the bf16 compatibility path for fnuz operands
// (dense and grouped scaled GEMMs); the MX and ragged-K products take OCP only.
fp8_status_t check_gemm_operands(const char* fn, const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb,
                                 int64_t ldb, int64_t m, int64_t n, int64_t k, const void* d, int d_type, int64_t ldd,
                                 bool fnuz_ok = false) {
    if (m < 0 || n < 0 || k < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative size m=%lld n=%lld k=%lld", fn,
                                             (long long)m, (long long)n, (long long)k);
    if (!valid_fmt(fa) || !valid_fmt(fb)) return fail(FP8_ERR_INVALID_ARG, "%s: unknown format (%d, %d)", fn, fa, fb);
    if (d_type != FP8_OUT_BF16 && d_type != FP8_OUT_F32) return fail(FP8_ERR_INVALID_ARG, "%s: unknown output type %d", fn, d_type);
    if (k % 16 != 0) return fail(FP8_ERR_INVALID_ARG, "%s: k = %lld is not a multiple of 16", fn, (long long)k);
    if (lda < k || ldb < k || ldd < n || ldd < 1)
        return fail(FP8_ERR_INVALID_ARG, "%s: leading dimension smaller than the row", fn);
    if (m > 0 && n > 0) {
        if (!d) return fail(FP8_ERR_INVALID_ARG, "%s: d is NULL", fn);
        if (k > 0 && (!a || !b)) return fail(FP8_ERR_INVALID_ARG, "%s: a or b is NULL", fn);
    }
    if (k > 0 && (!aligned(a, 16) || !aligned(b, 16) || lda % 16 != 0 || ldb % 16 != 0))
        return fail(FP8_ERR_ALIGNMENT, "%s: a, b must be 16-byte aligned with lda, ldb multiples of 16", fn);
    if (!aligned(d, 4)) return fail(FP8_ERR_ALIGNMENT, "%s: d must be 4-byte aligned", fn);
    if (!fnuz_ok && (!ocp_fmt(fa) || !ocp_fmt(fb)))
        return fail(FP8_ERR_UNSUPPORTED,
                    "%s: fnuz operands (%d, %d): this product takes the OCP e4m3/e5m2 encodings only", fn, fa, fb);
    return FP8_OK;
}

fp8_status_t check_blockwise(const char* fn, const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                             const uint8_t* q, int64_t ldq, const uint8_t* scale, int64_t ld_scale) {
    FP8_TRY(check_common_quant(fn, x, rows, cols, ldx, fmt, 0));
    if (!ocp_fmt(fmt)) return fail(FP8_ERR_INVALID_ARG, "%s: blockwise codes are OCP e4m3 or e5m2 (format %d)", fn, fmt);
    if (cols % 128 != 0) return fail(FP8_ERR_INVALID_ARG, "%s: cols = %lld is not a multiple of 128", fn, (long long)cols);
    FP8_TRY(check_matrix(fn, "q", q, rows, cols, ldq));
    if (rows > 0 && cols > 0 && !scale) return fail(FP8_ERR_INVALID_ARG, "%s: scale records are NULL", fn);
    if (ld_scale < rows || ld_scale < 1)
        return fail(FP8_ERR_INVALID_ARG, "%s: scale record stride %lld < rows", fn, (long long)ld_scale);
    if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(q, 8) || ldq % 8 != 0 || !aligned(scale, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: x must be 16-byte aligned with ldx a multiple of 8, q 8-byte aligned with "
                    "ldq a multiple of 8, the scale records 4-byte aligned", fn);
    if (rows >= ((int64_t)1 << 26)) return fail(FP8_ERR_UNSUPPORTED, "%s: 2^26 rows or more", fn);
    return FP8_OK;
}

// Shared checks of the MX products: k % 256, the E8M0 scale records (one
// dword per row and 128-deep K step, ld records apart per step), and the
// 32-bit tile offsets.
fp8_status_t check_mx(const char* fn, int64_t rows_a, int64_t rows_b, int64_t k, int64_t lda, int64_t ldb,
                      const uint8_t* xa, int64_t ld_xa, const uint8_t* xb, int64_t ld_xb) {
    if (k % 256 != 0) return fail(FP8_ERR_UNSUPPORTED, "%s: k = %lld is not a multiple of 256", fn, (long long)k);
    if (k > 0) {
        if (rows_a > 0 && rows_b > 0 && (!xa || !xb)) return fail(FP8_ERR_INVALID_ARG, "%s: scale is NULL", fn);
        if (ld_xa < rows_a || ld_xb < rows_b || ld_xa < 1 || ld_xb < 1)
            return fail(FP8_ERR_INVALID_ARG, "%s: scale record stride smaller than the row count", fn);
        if (!aligned(xa, 4) || !aligned(xb, 4)) return fail(FP8_ERR_ALIGNMENT, "%s: scales must be 4-byte aligned", fn);
    }
    if (lda >= (1 << 24) || ldb >= (1 << 24))
        return fail(FP8_ERR_UNSUPPORTED, "%s: lda, ldb must be < 2^24 (256-row tiles use 32-bit offsets)", fn);
    return FP8_OK;
}

}  // namespace

const DeviceProps& current_device_props() {
    static DeviceProps fallback{256};
    PropsSlot* s = slot_for_current(nullptr);
    return (s && s->err == hipSuccess) ? s->props : fallback;
}

}  // namespace fp8amax

using namespace fp8amax;

extern "C" {

const char* fp8_status_string(fp8_status_t status) {
    switch (status) {
        case FP8_OK: return "FP8_OK";
        case FP8_ERR_INVALID_ARG: return "FP8_ERR_INVALID_ARG";
        case FP8_ERR_ALIGNMENT: return "FP8_ERR_ALIGNMENT";
        case FP8_ERR_UNSUPPORTED: return "FP8_ERR_UNSUPPORTED";
        case FP8_ERR_HIP: return "FP8_ERR_HIP";
    }
    return "FP8_ERR_UNKNOWN";
}

const char* fp8_last_error(void) { return g_err; }

fp8_status_t fp8_query_device(int device, fp8_device_info_t* info) {
    if (!info) return fail(FP8_ERR_INVALID_ARG, "fp8_query_device: info is NULL");
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "hipGetDeviceCount: %s", hipGetErrorString(e));
    if (device < 0 || device >= count)
        return fail(FP8_ERR_INVALID_ARG, "fp8_query_device: device %d outside [0, %d)", device, count);
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, device);
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    std::memset(info, 0, sizeof *info);
    std::strncpy(info->arch, p.gcnArchName, sizeof info->arch - 1);
    info->is_gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    const bool fnuz_native = std::strncmp(p.gcnArchName, "gfx94", 5) == 0;
    info->native_e4m3 = fnuz_native ? FP8_E4M3_FNUZ : FP8_E4M3;
    info->native_e5m2 = fnuz_native ? FP8_E5M2_FNUZ : FP8_E5M2;
    info->compute_units = p.multiProcessorCount;
    info->lds_bytes_per_block = (int32_t)p.sharedMemPerBlock;
    info->global_mem_bytes = (int64_t)p.totalGlobalMem;
    return ok();
}

fp8_status_t fp8_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_axis_t axis, float* amax_out,
                      void* stream) {
    const char* fn = "fp8_amax";
    FP8_TRY(check_matrix(fn, "x", x, rows, cols, ldx));
    if (axis != FP8_AXIS_TENSOR && axis != FP8_AXIS_ROW && axis != FP8_AXIS_COL)
        return fail(FP8_ERR_INVALID_ARG, "%s: unknown axis %d", fn, (int)axis);
    const int64_t nout = axis == FP8_AXIS_TENSOR ? 1 : (axis == FP8_AXIS_ROW ? rows : cols);
    if (nout > 0 && !amax_out) return fail(FP8_ERR_INVALID_ARG, "%s: amax_out is NULL", fn);
    if (!aligned(x, 2) || !aligned(amax_out, 4)) return fail(FP8_ERR_ALIGNMENT, "%s: misaligned pointer", fn);
    FP8_TRY(check_device());
    return launched(launch_amax(x, rows, cols, ldx, (int)axis, amax_out, (hipStream_t)stream), fn);
}

fp8_status_t fp8_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                                 int32_t margin, const float* scale, uint8_t* q, int64_t ldq, float* scale_inv_out,
                                 float* amax_out, void* stream) {
    const char* fn = "fp8_quantize_tensor";
    FP8_TRY(check_common_quant(fn, x, rows, cols, ldx, (int)fmt, margin));
    FP8_TRY(check_matrix(fn, "q", q, rows, cols, ldq));
    if (!scale_inv_out || !amax_out) return fail(FP8_ERR_INVALID_ARG, "%s: scale_inv_out and amax_out are required", fn);
    if (!aligned(scale_inv_out, 4) || !aligned(amax_out, 4) || !aligned(scale, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer", fn);
    FP8_TRY(check_device());
    return launched(launch_quant_tensor(x, rows, cols, ldx, (int)fmt, margin, scale, q, ldq, scale_inv_out, amax_out,
                                        (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                              int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out, float* amax_out,
                              float* col_amax_out, void* stream) {
    const char* fn = "fp8_quantize_row";
    FP8_TRY(check_common_quant(fn, x, rows, cols, ldx, (int)fmt, margin));
    FP8_TRY(check_matrix(fn, "q", q, rows, cols, ldq));
    if (rows > 0 && !scale_inv_out) return fail(FP8_ERR_INVALID_ARG, "%s: scale_inv_out is NULL", fn);
    if (!aligned(scale_inv_out, 4) || !aligned(amax_out, 4) || !aligned(col_amax_out, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer", fn);
    FP8_TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    if (col_amax_out)       // the column amax as a side output of the same pass (a batch of one)
        return launched(launch_quant_row_batch(1, &x, &rows, cols, &ldx, (int)fmt, margin, &q, &ldq, &scale_inv_out,
                                               &amax_out, &col_amax_out, nullptr, nullptr, st),
                        fn);
    return launched(launch_quant_row(x, rows, cols, ldx, (int)fmt, margin, q, ldq, scale_inv_out, amax_out, false, st),
                    fn);
}

fp8_status_t fp8_quantize_row_batch(int32_t count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                    const int64_t* ldx, fp8_format_t fmt, int32_t margin, uint8_t* const* q,
                                    const int64_t* ldq, float* const* scale_inv_out, float* const* amax_out,
                                    float* const* col_amax_out, const int64_t* const* col_group_offsets,
                                    const int32_t* col_groups, void* stream) {
    const char* fn = "fp8_quantize_row_batch";
    if (count < 1 || count > FP8_MAX_ROW_BATCH)
        return fail(FP8_ERR_INVALID_ARG, "%s: count %d outside 1..%d", fn, (int)count, FP8_MAX_ROW_BATCH);
    if (!x || !rows || !ldx || !q || !ldq || !scale_inv_out)
        return fail(FP8_ERR_INVALID_ARG, "%s: a required host array is NULL", fn);
    for (int j = 0; j < count; ++j) {
        FP8_TRY(check_common_quant(fn, x[j], rows[j], cols, ldx[j], (int)fmt, margin));
        FP8_TRY(check_matrix(fn, "q", q[j], rows[j], cols, ldq[j]));
        if (rows[j] > 0 && !scale_inv_out[j]) return fail(FP8_ERR_INVALID_ARG, "%s: scale_inv_out[%d] is NULL", fn, j);
        if (!aligned(scale_inv_out[j], 4) || (amax_out && !aligned(amax_out[j], 4)) ||
            (col_amax_out && !aligned(col_amax_out[j], 4)))
            return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer (tensor %d)", fn, j);
    }
    bool grouped = false;
    for (int j = 0; j < count && col_groups; ++j) {
        if (col_groups[j] < 0 || col_groups[j] > 4096)
            return fail(FP8_ERR_INVALID_ARG, "%s: col_groups[%d] = %d outside 0..4096", fn, j, (int)col_groups[j]);
        if (col_groups[j] == 0) continue;
        grouped = true;
        if (!col_amax_out || !col_amax_out[j])
            return fail(FP8_ERR_INVALID_ARG, "%s: tensor %d has column groups but no col_amax_out", fn, j);
        if (!col_group_offsets || !col_group_offsets[j])
            return fail(FP8_ERR_INVALID_ARG, "%s: col_group_offsets[%d] is NULL", fn, j);
        if (!aligned(col_group_offsets[j], 8))
            return fail(FP8_ERR_ALIGNMENT, "%s: col_group_offsets[%d] must be 8-byte aligned", fn, j);
    }
    if (grouped) {      // the single-pass kernel only: every tensor in the vector layout, rows <= 16384 columns
        if (cols > 16384)
            return fail(FP8_ERR_UNSUPPORTED, "%s: grouped column amax needs cols <= 16384 (cols = %lld)", fn,
                        (long long)cols);
        for (int j = 0; j < count; ++j)
            if (cols % 8 != 0 || ldx[j] % 8 != 0 || ldq[j] % 8 != 0 || !aligned(x[j], 16) || !aligned(q[j], 8))
                return fail(FP8_ERR_ALIGNMENT, "%s: grouped column amax needs every tensor's x 16-byte and q 8-byte "
                            "aligned, ldx, ldq, cols multiples of 8 (tensor %d)", fn, j);
    }
    FP8_TRY(check_device());
    return launched(launch_quant_row_batch(count, x, rows, cols, ldx, (int)fmt, margin, q, ldq, scale_inv_out,
                                           amax_out, col_amax_out, grouped ? col_group_offsets : nullptr,
                                           grouped ? col_groups : nullptr, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_quantize_tensor_batch(int32_t count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                       const int64_t* ldx, fp8_format_t fmt, const float* const* scale,
                                       uint8_t* const* q, const int64_t* ldq, float* const* scale_inv_out,
                                       float* const* amax_out, void* stream) {
    const char* fn = "fp8_quantize_tensor_batch";
    if (count < 1 || count > FP8_MAX_ROW_BATCH)
        return fail(FP8_ERR_INVALID_ARG, "%s: count %d outside 1..%d", fn, (int)count, FP8_MAX_ROW_BATCH);
    if (!x || !rows || !ldx || !scale || !q || !ldq || !scale_inv_out || !amax_out)
        return fail(FP8_ERR_INVALID_ARG, "%s: a host array is NULL", fn);
    for (int j = 0; j < count; ++j) {
        FP8_TRY(check_common_quant(fn, x[j], rows[j], cols, ldx[j], (int)fmt, 0));
        FP8_TRY(check_matrix(fn, "q", q[j], rows[j], cols, ldq[j]));
        if (!scale[j] || !scale_inv_out[j] || !amax_out[j])
            return fail(FP8_ERR_INVALID_ARG, "%s: scale, scale_inv_out and amax_out of tensor %d are required", fn, j);
        if (!aligned(scale[j], 4) || !aligned(scale_inv_out[j], 4) || !aligned(amax_out[j], 4))
            return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer (tensor %d)", fn, j);
    }
    FP8_TRY(check_device());
    return launched(launch_quant_tensor_batch(count, x, rows, cols, ldx, (int)fmt, scale, q, ldq, scale_inv_out,
                                              amax_out, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_quantize_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                              int32_t margin, int32_t transpose_out, uint8_t* q, int64_t ldq, float* scale_inv_out,
                              float* col_amax, int32_t col_amax_ready, void* stream) {
    const char* fn = "fp8_quantize_col";
    FP8_TRY(check_common_quant(fn, x, rows, cols, ldx, (int)fmt, margin));
    if (transpose_out != 0 && transpose_out != 1)
        return fail(FP8_ERR_INVALID_ARG, "%s: transpose_out must be 0 or 1", fn);
    if (transpose_out)
        FP8_TRY(check_matrix(fn, "q", q, cols, rows, ldq));
    else
        FP8_TRY(check_matrix(fn, "q", q, rows, cols, ldq));
    if (cols > 0 && (!scale_inv_out || !col_amax))
        return fail(FP8_ERR_INVALID_ARG, "%s: scale_inv_out and col_amax are required", fn);
    if (col_amax_ready != 0 && col_amax_ready != 1)
        return fail(FP8_ERR_INVALID_ARG, "%s: col_amax_ready must be 0 or 1", fn);
    if (!aligned(scale_inv_out, 4) || !aligned(col_amax, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer", fn);
    FP8_TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (!col_amax_ready) e = launch_amax(x, rows, cols, ldx, FP8_AXIS_COL, col_amax, st);
    if (e == hipSuccess)
        e = launch_quant_col(x, rows, cols, ldx, (int)fmt, margin, transpose_out, q, ldq, scale_inv_out, col_amax, st);
    return launched(e, fn);
}

fp8_status_t fp8_quantize_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                                 int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out, float* amax_out,
                                 uint8_t* qt, int64_t ldqt, float* col_scale_inv_out, float* col_amax_out,
                                 void* stream) {
    const char* fn = "fp8_quantize_rowcol";
    FP8_TRY(check_common_quant(fn, x, rows, cols, ldx, (int)fmt, margin));
    FP8_TRY(check_matrix(fn, "q", q, rows, cols, ldq));
    FP8_TRY(check_matrix(fn, "qt", qt, cols, rows, ldqt));
    if ((rows > 0 && (!scale_inv_out || !amax_out)) || (cols > 0 && (!col_scale_inv_out || !col_amax_out)))
        return fail(FP8_ERR_INVALID_ARG, "%s: scale and amax outputs are required", fn);
    if (!aligned(scale_inv_out, 4) || !aligned(amax_out, 4) || !aligned(col_scale_inv_out, 4) ||
        !aligned(col_amax_out, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer", fn);
    if (!aligned(x, 16) || ldx % 8 != 0 || cols % 8 != 0 || !aligned(q, 8) || ldq % 8 != 0)
        return fail(FP8_ERR_ALIGNMENT, "%s: x must be 16-byte aligned with ldx, cols multiples of 8; q 8-byte "
                    "aligned with ldq a multiple of 8", fn);
    FP8_TRY(check_device());
    return launched(launch_quant_rowcol(x, rows, cols, ldx, (int)fmt, margin, q, ldq, scale_inv_out, amax_out, qt,
                                        ldqt, col_scale_inv_out, col_amax_out, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_delayed_scale_update(float* cur_amax, float* history, int32_t* head, int64_t n, int32_t L,
                                      fp8_amax_algo_t algo, int32_t margin, fp8_format_t fmt, float* scale,
                                      float* scale_inv, void* stream) {
    const char* fn = "fp8_delayed_scale_update";
    if (n < 0) return fail(FP8_ERR_INVALID_ARG, "%s: n < 0", fn);
    if (L < 1 || L > 65536) return fail(FP8_ERR_INVALID_ARG, "%s: history length %d outside 1..65536", fn, L);
    if (algo != FP8_AMAX_MOST_RECENT && algo != FP8_AMAX_MAX)
        return fail(FP8_ERR_INVALID_ARG, "%s: unknown amax algo %d", fn, (int)algo);
    if (margin < 0 || margin > 32) return fail(FP8_ERR_INVALID_ARG, "%s: margin %d outside 0..32", fn, margin);
    if (!valid_fmt((int)fmt)) return fail(FP8_ERR_INVALID_ARG, "%s: unknown format %d", fn, (int)fmt);
    if (!head) return fail(FP8_ERR_INVALID_ARG, "%s: head is NULL", fn);
    if (n > 0 && (!cur_amax || !history || !scale || !scale_inv))
        return fail(FP8_ERR_INVALID_ARG, "%s: state pointer is NULL", fn);
    if (!aligned(cur_amax, 4) || !aligned(history, 4) || !aligned(head, 4) || !aligned(scale, 4) ||
        !aligned(scale_inv, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned state pointer", fn);
    FP8_TRY(check_device());
    return launched(launch_delayed_update(cur_amax, history, head, n, L, (int)algo, margin, (int)fmt, scale, scale_inv,
                                          (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_gemm_scaled(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* b, fp8_format_t fb,
                             int64_t ldb, int64_t m, int64_t n, int64_t k, const float* a_scale_inv,
                             fp8_scale_mode_t a_mode, const float* b_scale_inv, fp8_scale_mode_t b_mode, void* d,
                             fp8_out_t d_type, int64_t ldd, void* stream) {
    const char* fn = "fp8_gemm_scaled";
    FP8_TRY(check_gemm_operands(fn, a, (int)fa, lda, b, (int)fb, ldb, m, n, k, d, (int)d_type, ldd, true));
    if ((a_mode != FP8_SCALE_TENSOR && a_mode != FP8_SCALE_VECTOR) ||
        (b_mode != FP8_SCALE_TENSOR && b_mode != FP8_SCALE_VECTOR))
        return fail(FP8_ERR_INVALID_ARG, "%s: unknown scale mode", fn);
    if (m > 0 && n > 0 && (!a_scale_inv || !b_scale_inv)) return fail(FP8_ERR_INVALID_ARG, "%s: scale is NULL", fn);
    if (!aligned(a_scale_inv, 4) || !aligned(b_scale_inv, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned scale pointer", fn);
    FP8_TRY(check_device());
    if (!ocp_fmt((int)fa) || !ocp_fmt((int)fb))
        return launched(launch_gemm_compat(a, (int)fa, lda, b, (int)fb, ldb, m, n, k, a_scale_inv,
                                           a_mode == FP8_SCALE_VECTOR, b_scale_inv, b_mode == FP8_SCALE_VECTOR, d,
                                           d_type == FP8_OUT_F32, ldd, (hipStream_t)stream),
                        fn);
    return launched(launch_gemm(a, (int)fa, lda, b, (int)fb, ldb, m, n, k, a_scale_inv, a_mode == FP8_SCALE_VECTOR,
                                b_scale_inv, b_mode == FP8_SCALE_VECTOR, d, d_type == FP8_OUT_F32, ldd,
                                (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_grouped_gemm_scaled(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* b,
                                     fp8_format_t fb, int64_t ldb, int64_t b_group_stride,
                                     const int64_t* group_offsets, int32_t g, int64_t total_m, int64_t n, int64_t k,
                                     const float* a_scale_inv, const float* b_scale_inv, void* d, fp8_out_t d_type,
                                     int64_t ldd, void* stream) {
    const char* fn = "fp8_grouped_gemm_scaled";
    FP8_TRY(check_gemm_operands(fn, a, (int)fa, lda, b, (int)fb, ldb, total_m, n, k, d, (int)d_type, ldd, true));
    if (g < 1 || g > 4096) return fail(FP8_ERR_INVALID_ARG, "%s: group count %d outside 1..4096", fn, g);
    if (!group_offsets) return fail(FP8_ERR_INVALID_ARG, "%s: group_offsets is NULL", fn);
    if (!aligned(group_offsets, 8)) return fail(FP8_ERR_ALIGNMENT, "%s: group_offsets must be 8-byte aligned", fn);
    if (b_group_stride < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative b_group_stride", fn);
    if (b_group_stride % 16 != 0) return fail(FP8_ERR_ALIGNMENT, "%s: b_group_stride must be a multiple of 16", fn);
    if (total_m > 0 && n > 0 && (!a_scale_inv || !b_scale_inv))
        return fail(FP8_ERR_INVALID_ARG, "%s: scale is NULL", fn);
    if (!aligned(a_scale_inv, 4) || !aligned(b_scale_inv, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned scale pointer", fn);
    FP8_TRY(check_device());
    if (!ocp_fmt((int)fa) || !ocp_fmt((int)fb))
        return launched(launch_grouped_gemm_compat(a, (int)fa, lda, b, (int)fb, ldb, b_group_stride, group_offsets, g,
                                                   total_m, n, k, a_scale_inv, b_scale_inv, d, d_type == FP8_OUT_F32,
                                                   ldd, (hipStream_t)stream),
                        fn);
    return launched(launch_grouped_gemm(a, (int)fa, lda, b, (int)fb, ldb, b_group_stride, group_offsets, g, total_m,
                                        n, k, a_scale_inv, b_scale_inv, d, d_type == FP8_OUT_F32, ldd,
                                        (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_grouped_quantize_col(const uint16_t* x, int64_t total_m, int64_t cols, int64_t ldx,
                                      fp8_format_t fmt, int32_t margin, const int64_t* group_offsets, int32_t g,
                                      uint8_t* qt, int64_t ldqt, float* scale_inv_out, float* col_amax,
                                      int32_t col_amax_ready, void* stream) {
    const char* fn = "fp8_grouped_quantize_col";
    FP8_TRY(check_common_quant(fn, x, total_m, cols, ldx, (int)fmt, margin));
    FP8_TRY(check_matrix(fn, "qt", qt, cols, total_m, ldqt));
    if (g < 1 || g > 4096) return fail(FP8_ERR_INVALID_ARG, "%s: group count %d outside 1..4096", fn, g);
    if (!group_offsets) return fail(FP8_ERR_INVALID_ARG, "%s: group_offsets is NULL", fn);
    if (!aligned(group_offsets, 8)) return fail(FP8_ERR_ALIGNMENT, "%s: group_offsets must be 8-byte aligned", fn);
    if (cols > 0 && (!scale_inv_out || !col_amax))
        return fail(FP8_ERR_INVALID_ARG, "%s: scale_inv_out and col_amax are required", fn);
    if (col_amax_ready != 0 && col_amax_ready != 1)
        return fail(FP8_ERR_INVALID_ARG, "%s: col_amax_ready must be 0 or 1", fn);
    if (!aligned(scale_inv_out, 4) || !aligned(col_amax, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned fp32 pointer", fn);
    if (!aligned(x, 16) || ldx % 8 != 0 || cols % 8 != 0 || !aligned(qt, 16) || ldqt % 16 != 0)
        return fail(FP8_ERR_ALIGNMENT, "%s: x must be 16-byte aligned with ldx, cols multiples of 8, "
                    "qt 16-byte aligned with ldqt a multiple of 16", fn);
    FP8_TRY(check_device());
    return launched(launch_grouped_quant_col(x, total_m, cols, ldx, (int)fmt, margin, group_offsets, g, qt, ldqt,
                                             scale_inv_out, col_amax, col_amax_ready, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_grouped_gemm_ragged_k(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* b,
                                       fp8_format_t fb, int64_t ldb, const int64_t* group_offsets, int32_t g,
                                       int64_t total_m, int64_t m, int64_t n, const float* a_scale_inv,
                                       const float* b_scale_inv, void* d, fp8_out_t d_type, int64_t ldd,
                                       int64_t d_group_stride, void* stream) {
    const char* fn = "fp8_grouped_gemm_ragged_k";
    if (total_m < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative total_m", fn);
    // the contraction runs over the grouped layout's columns: lda, ldb >= total_m
    // (checked as k = total_m rounded down to 16, the operand width requirement)
    FP8_TRY(check_gemm_operands(fn, a, (int)fa, lda, b, (int)fb, ldb, m, n, total_m / 16 * 16, d, (int)d_type, ldd));
    if (lda < total_m || ldb < total_m) return fail(FP8_ERR_INVALID_ARG, "%s: lda, ldb must be >= total_m", fn);
    if (lda >= (1 << 24) || ldb >= (1 << 24))
        return fail(FP8_ERR_UNSUPPORTED, "%s: lda, ldb must be < 2^24 (256-row tiles use 32-bit offsets)", fn);
    if (m > 0 && n > 0 && (!a || !b)) return fail(FP8_ERR_INVALID_ARG, "%s: a or b is NULL", fn);
    if (!aligned(a, 16) || !aligned(b, 16) || lda % 16 != 0 || ldb % 16 != 0)
        return fail(FP8_ERR_ALIGNMENT, "%s: a, b must be 16-byte aligned with lda, ldb multiples of 16", fn);
    if (g < 1 || g > 4096) return fail(FP8_ERR_INVALID_ARG, "%s: group count %d outside 1..4096", fn, g);
    if (!group_offsets) return fail(FP8_ERR_INVALID_ARG, "%s: group_offsets is NULL", fn);
    if (!aligned(group_offsets, 8)) return fail(FP8_ERR_ALIGNMENT, "%s: group_offsets must be 8-byte aligned", fn);
    if (g > 1 && m > 0 && d_group_stride < m * ldd)
        return fail(FP8_ERR_INVALID_ARG, "%s: d_group_stride %lld < m * ldd", fn, (long long)d_group_stride);
    if (d_group_stride < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative d_group_stride", fn);
    if (m > 0 && n > 0 && (!a_scale_inv || !b_scale_inv)) return fail(FP8_ERR_INVALID_ARG, "%s: scale is NULL", fn);
    if (!aligned(a_scale_inv, 4) || !aligned(b_scale_inv, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned scale pointer", fn);
    FP8_TRY(check_device());
    return launched(launch_grouped_gemm_ragged_k(a, (int)fa, lda, b, (int)fb, ldb, group_offsets, g, total_m, m, n,
                                                 a_scale_inv, b_scale_inv, d, d_type == FP8_OUT_F32, ldd,
                                                 d_group_stride, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_mx_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                                 uint8_t* q, int64_t ldq, uint8_t* scale_e8m0, int64_t ld_scale, void* stream) {
    const char* fn = "fp8_mx_quantize_row";
    FP8_TRY(check_common_quant(fn, x, rows, cols, ldx, (int)fmt, 0));
    if (!ocp_fmt((int)fmt)) return fail(FP8_ERR_INVALID_ARG, "%s: MX elements are OCP e4m3 or e5m2 (format %d)", fn, (int)fmt);
    if (cols % FP8_MX_BLOCK != 0) return fail(FP8_ERR_INVALID_ARG, "%s: cols = %lld is not a multiple of %d", fn,
                                              (long long)cols, FP8_MX_BLOCK);
    FP8_TRY(check_matrix(fn, "q", q, rows, cols, ldq));
    if (rows > 0 && cols > 0 && !scale_e8m0) return fail(FP8_ERR_INVALID_ARG, "%s: scale_e8m0 is NULL", fn);
    if (ld_scale < rows || ld_scale < 1)
        return fail(FP8_ERR_INVALID_ARG, "%s: scale record stride %lld < rows", fn, (long long)ld_scale);
    if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(q, 8) || ldq % 8 != 0 || !aligned(scale_e8m0, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: x must be 16-byte aligned with ldx a multiple of 8, q 8-byte aligned with "
                    "ldq a multiple of 8, scale_e8m0 4-byte aligned", fn);
    if (rows >= ((int64_t)1 << 26)) return fail(FP8_ERR_UNSUPPORTED, "%s: 2^26 rows or more", fn);
    FP8_TRY(check_device());
    return launched(launch_mx_quant_row(x, rows, cols, ldx, (int)fmt, q, ldq, scale_e8m0, ld_scale,
                                        (hipStream_t)stream),
                    fn);
}


fp8_status_t fp8_gemm_mx(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* a_scale, int64_t ld_as,
                         const uint8_t* b, fp8_format_t fb, int64_t ldb, const uint8_t* b_scale, int64_t ld_bs,
                         int64_t m, int64_t n, int64_t k, void* d, fp8_out_t d_type, int64_t ldd, void* stream) {
    const char* fn = "fp8_gemm_mx";
    FP8_TRY(check_gemm_operands(fn, a, (int)fa, lda, b, (int)fb, ldb, m, n, k, d, (int)d_type, ldd));
    FP8_TRY(check_mx(fn, m, n, k, lda, ldb, a_scale, ld_as, b_scale, ld_bs));
    if (((m + 255) / 256) * ((n + 255) / 256) >= ((int64_t)1 << 24))
        return fail(FP8_ERR_UNSUPPORTED, "%s: 2^24 or more tiles of 256 x 256", fn);
    FP8_TRY(check_device());
    return launched(launch_gemm_mx(a, (int)fa, lda, a_scale, ld_as, b, (int)fb, ldb, b_scale, ld_bs, m, n, k, d,
                                   d_type == FP8_OUT_F32, ldd, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_grouped_gemm_mx(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* a_scale,
                                 int64_t ld_as, const uint8_t* b, fp8_format_t fb, int64_t ldb, int64_t b_group_stride,
                                 const uint8_t* b_scale, int64_t ld_bs, int64_t b_scale_group_stride,
                                 const int64_t* group_offsets, int32_t g, int64_t total_m, int64_t n, int64_t k,
                                 void* d, fp8_out_t d_type, int64_t ldd, void* stream) {
    const char* fn = "fp8_grouped_gemm_mx";
    FP8_TRY(check_gemm_operands(fn, a, (int)fa, lda, b, (int)fb, ldb, total_m, n, k, d, (int)d_type, ldd));
    FP8_TRY(check_mx(fn, total_m, n, k, lda, ldb, a_scale, ld_as, b_scale, ld_bs));
    if (g < 1 || g > 4096) return fail(FP8_ERR_INVALID_ARG, "%s: group count %d outside 1..4096", fn, g);
    if (!group_offsets) return fail(FP8_ERR_INVALID_ARG, "%s: group_offsets is NULL", fn);
    if (!aligned(group_offsets, 8)) return fail(FP8_ERR_ALIGNMENT, "%s: group_offsets must be 8-byte aligned", fn);
    if (b_group_stride < 0 || b_scale_group_stride < 0)
        return fail(FP8_ERR_INVALID_ARG, "%s: negative group stride", fn);
    if (b_group_stride % 16 != 0 || b_scale_group_stride % 4 != 0)
        return fail(FP8_ERR_ALIGNMENT, "%s: b_group_stride must be a multiple of 16, b_scale_group_stride of 4", fn);
    if (((total_m + 255) / 256 + g) * ((n + 255) / 256) >= ((int64_t)1 << 24))
        return fail(FP8_ERR_UNSUPPORTED, "%s: 2^24 or more tiles of 256 x 256", fn);
    FP8_TRY(check_device());
    return launched(launch_grouped_gemm_mx(a, (int)fa, lda, a_scale, ld_as, b, (int)fb, ldb, b_group_stride, b_scale,
                                           ld_bs, b_scale_group_stride, group_offsets, g, total_m, n, k, d,
                                           d_type == FP8_OUT_F32, ldd, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_moe_route(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t num_experts,
                           int64_t* offsets_out, int32_t* dest_out, void* stream) {
    const char* fn = "fp8_moe_route";
    if (tokens < 0) return fail(FP8_ERR_INVALID_ARG, "%s: negative token count", fn);
    if (topk < 1 || topk > kMoeMaxTopk) return fail(FP8_ERR_INVALID_ARG, "%s: topk %d outside 1..%d", fn, topk, kMoeMaxTopk);
    if (num_experts < 1 || num_experts > kMoeMaxExperts)
        return fail(FP8_ERR_INVALID_ARG, "%s: expert count %d outside 1..%d", fn, num_experts, kMoeMaxExperts);
    if (tokens * topk >= ((int64_t)1 << 31)) return fail(FP8_ERR_UNSUPPORTED, "%s: 2^31 or more entries", fn);
    if (!offsets_out || (tokens > 0 && (!expert_idx || !dest_out)))
        return fail(FP8_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(expert_idx, 4) || !aligned(dest_out, 4) || !aligned(offsets_out, 8))
        return fail(FP8_ERR_ALIGNMENT, "%s: misaligned pointer", fn);
    FP8_TRY(check_device());
    return launched(launch_moe_route(expert_idx, tokens, topk, num_experts, offsets_out, dest_out,
                                     (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_moe_permute_quantize_row(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ldx,
                                          const int32_t* dest, int32_t topk, int64_t rows_out, fp8_format_t fmt,
                                          int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out,
                                          void* stream) {
    const char* fn = "fp8_moe_permute_quantize_row";
    FP8_TRY(check_common_quant(fn, x, tokens, cols, ldx, (int)fmt, margin));
    FP8_TRY(check_matrix(fn, "q", q, rows_out, cols, ldq));
    if (topk < 1 || topk > kMoeMaxTopk) return fail(FP8_ERR_INVALID_ARG, "%s: topk %d outside 1..%d", fn, topk, kMoeMaxTopk);
    if (tokens > 0 && cols > 0 && (!dest || !scale_inv_out)) return fail(FP8_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || ldx % 8 != 0 || cols % 8 != 0 || !aligned(q, 8) || ldq % 8 != 0 || !aligned(dest, 4) ||
        !aligned(scale_inv_out, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: x must be 16-byte aligned with ldx, cols multiples of 8; q 8-byte "
                    "aligned with ldq a multiple of 8", fn);
    if (cols > 16384) return fail(FP8_ERR_UNSUPPORTED, "%s: rows longer than 16384 columns", fn);
    if (tokens >= ((int64_t)1 << 31)) return fail(FP8_ERR_UNSUPPORTED, "%s: 2^31 or more tokens", fn);
    FP8_TRY(check_device());
    return launched(launch_moe_permute_quant_row(x, tokens, cols, ldx, dest, topk, rows_out, (int)fmt, margin, q, ldq,
                                                 scale_inv_out, (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_swiglu_quantize_row(const uint16_t* h, int64_t rows, int64_t inter, int64_t ldh, fp8_format_t fmt,
                                     int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out, void* stream) {
    const char* fn = "fp8_swiglu_quantize_row";
    FP8_TRY(check_common_quant(fn, h, rows, 2 * inter, ldh, (int)fmt, margin));
    FP8_TRY(check_matrix(fn, "q", q, rows, inter, ldq));
    if (rows > 0 && inter > 0 && !scale_inv_out) return fail(FP8_ERR_INVALID_ARG, "%s: scale_inv_out is NULL", fn);
    if (!aligned(h, 16) || ldh % 8 != 0 || inter % 8 != 0 || !aligned(q, 8) || ldq % 8 != 0 ||
        !aligned(scale_inv_out, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: h must be 16-byte aligned with ldh, inter multiples of 8; q 8-byte "
                    "aligned with ldq a multiple of 8", fn);
    if (inter > kSwigluMaxChunks * 512)
        return fail(FP8_ERR_UNSUPPORTED, "%s: intermediate size above %d", fn, kSwigluMaxChunks * 512);
    if (rows >= ((int64_t)1 << 31)) return fail(FP8_ERR_UNSUPPORTED, "%s: 2^31 or more rows", fn);
    FP8_TRY(check_device());
    return launched(launch_swiglu_quant_row(h, rows, inter, ldh, (int)fmt, margin, q, ldq, scale_inv_out,
                                            (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_moe_unpermute_combine(const uint16_t* y, int64_t rows, int64_t cols, int64_t ldy,
                                       const int32_t* dest, const float* weights, int64_t tokens, int32_t topk,
                                       uint16_t* out, int64_t ldo, void* stream) {
    const char* fn = "fp8_moe_unpermute_combine";
    FP8_TRY(check_matrix(fn, "y", y, rows, cols, ldy));
    FP8_TRY(check_matrix(fn, "out", out, tokens, cols, ldo));
    if (topk < 1 || topk > kMoeMaxTopk) return fail(FP8_ERR_INVALID_ARG, "%s: topk %d outside 1..%d", fn, topk, kMoeMaxTopk);
    if (tokens > 0 && cols > 0 && (!dest || !weights)) return fail(FP8_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(y, 16) || ldy % 8 != 0 || cols % 8 != 0 || !aligned(out, 16) || ldo % 8 != 0 ||
        !aligned(dest, 4) || !aligned(weights, 4))
        return fail(FP8_ERR_ALIGNMENT, "%s: y and out must be 16-byte aligned with ldy, ldo, cols multiples of 8",
                    fn);
    if (tokens >= ((int64_t)1 << 31)) return fail(FP8_ERR_UNSUPPORTED, "%s: 2^31 or more tokens", fn);
    FP8_TRY(check_device());
    return launched(launch_moe_unpermute_combine(y, rows, cols, ldy, dest, weights, tokens, topk, out, ldo,
                                                 (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_blockwise_quantize_act(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                        fp8_format_t fmt, uint8_t* q, int64_t ldq, uint8_t* scale_records,
                                        int64_t ld_scale, void* stream) {
    const char* fn = "fp8_blockwise_quantize_act";
    FP8_TRY(check_blockwise(fn, x, rows, cols, ldx, (int)fmt, q, ldq, scale_records, ld_scale));
    FP8_TRY(check_device());
    return launched(launch_blockwise_quant(x, rows, cols, ldx, (int)fmt, 0, q, ldq, scale_records, ld_scale,
                                           (hipStream_t)stream),
                    fn);
}

fp8_status_t fp8_blockwise_quantize_weight(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw,
                                           fp8_format_t fmt, uint8_t* q, int64_t ldq, uint8_t* scale_records,
                                           int64_t ld_scale, void* stream) {
    const char* fn = "fp8_blockwise_quantize_weight";
    FP8_TRY(check_blockwise(fn, w, rows, cols, ldw, (int)fmt, q, ldq, scale_records, ld_scale));
    if (cols / 128 > 65535) return fail(FP8_ERR_UNSUPPORTED, "%s: more than 65535 K blocks", fn);
    FP8_TRY(check_device());
    return launched(launch_blockwise_quant(w, rows, cols, ldw, (int)fmt, 1, q, ldq, scale_records, ld_scale,
                                           (hipStream_t)stream),
                    fn);
}

}  // extern "C"
