// api_sanitize_driver.cpp - the C ABI's host code (csrc/api.cpp: argument
// validation, the device-properties cache, dispatch) under the address and
// undefined-behaviour sanitizers, without a GPU. The kernel launchers and the
// few HIP runtime calls api.cpp makes are replaced by stubs that report one
// gfx950 device and record which launcher ran; every entry point is called
// with valid arguments (fake device pointers, never dereferenced: the stub
// launchers take the place of the kernels) and with each class of invalid
// argument, and the host arrays of the batched calls are exactly count
// entries long, so a read past them is reported. Exit status 0 when every
// check holds.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../include/fp8amax.h"
#include "../fp8_scaled_gemm_amax_amd/csrc/kernels.hpp"

static std::string g_last;   // name of the last launcher the dispatch reached
static int g_fail = 0;

#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);      \
            ++g_fail;                                                            \
        }                                                                        \
    } while (0)

// ---------------------------------------------------------------- HIP stubs --
extern "C" {
hipError_t hipGetDevice(int* d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetDeviceCount(int* n) {
    *n = 1;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600* p, int dev) {
    if (dev != 0) return hipErrorInvalidDevice;
    std::memset(p, 0, sizeof *p);
    std::strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
    p->multiProcessorCount = 256;
    p->sharedMemPerBlock = 163840;
    p->totalGlobalMem = (size_t)288 << 30;
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "stub"; }
}

// ----------------------------------------------------------- launcher stubs --
namespace fp8amax {
#define STUB(name, ...)                 \
    hipError_t name(__VA_ARGS__) {      \
        g_last = #name;                 \
        return hipSuccess;              \
    }
STUB(launch_fill, float*, int64_t, float, hipStream_t)
STUB(launch_amax, const uint16_t*, int64_t, int64_t, int64_t, int, float*, hipStream_t)
STUB(launch_quant_row, const uint16_t*, int64_t, int64_t, int64_t, int, int, uint8_t*, int64_t, float*, float*, bool,
     hipStream_t)
STUB(launch_quant_row_batch, int, const uint16_t* const*, const int64_t*, int64_t, const int64_t*, int, int,
     uint8_t* const*, const int64_t*, float* const*, float* const*, float* const*, const int64_t* const*,
     const int32_t*, hipStream_t)
STUB(launch_quant_col, const uint16_t*, int64_t, int64_t, int64_t, int, int, int, uint8_t*, int64_t, float*,
     const float*, hipStream_t)
STUB(launch_quant_tensor, const uint16_t*, int64_t, int64_t, int64_t, int, int, const float*, uint8_t*, int64_t, float*,
     float*, hipStream_t)
STUB(launch_quant_rowcol, const uint16_t*, int64_t, int64_t, int64_t, int, int, uint8_t*, int64_t, float*, float*,
     uint8_t*, int64_t, float*, float*, hipStream_t)
STUB(launch_quant_tensor_batch, int, const uint16_t* const*, const int64_t*, int64_t, const int64_t*, int,
     const float* const*, uint8_t* const*, const int64_t*, float* const*, float* const*, hipStream_t)
STUB(launch_delayed_update, float*, float*, int32_t*, int64_t, int32_t, int, int, int, float*, float*, hipStream_t)
STUB(launch_gemm, const uint8_t*, int, int64_t, const uint8_t*, int, int64_t, int64_t, int64_t, int64_t, const float*,
     int, const float*, int, void*, int, int64_t, hipStream_t)
STUB(launch_grouped_gemm, const uint8_t*, int, int64_t, const uint8_t*, int, int64_t, int64_t, const int64_t*, int,
     int64_t, int64_t, int64_t, const float*, const float*, void*, int, int64_t, hipStream_t)
STUB(launch_gemm_compat, const uint8_t*, int, int64_t, const uint8_t*, int, int64_t, int64_t, int64_t, int64_t,
     const float*, int, const float*, int, void*, int, int64_t, hipStream_t)
STUB(launch_grouped_gemm_compat, const uint8_t*, int, int64_t, const uint8_t*, int, int64_t, int64_t, const int64_t*,
     int, int64_t, int64_t, int64_t, const float*, const float*, void*, int, int64_t, hipStream_t)
STUB(launch_grouped_quant_col, const uint16_t*, int64_t, int64_t, int64_t, int, int, const int64_t*, int, uint8_t*,
     int64_t, float*, float*, int, hipStream_t)
STUB(launch_grouped_gemm_ragged_k, const uint8_t*, int, int64_t, const uint8_t*, int, int64_t, const int64_t*, int,
     int64_t, int64_t, int64_t, const float*, const float*, void*, int, int64_t, int64_t, hipStream_t)
STUB(launch_mx_quant_row, const uint16_t*, int64_t, int64_t, int64_t, int, uint8_t*, int64_t, uint8_t*, int64_t,
     hipStream_t)
STUB(launch_blockwise_quant, const uint16_t*, int64_t, int64_t, int64_t, int, int, uint8_t*, int64_t, uint8_t*, int64_t,
     hipStream_t)
STUB(launch_gemm_mx, const uint8_t*, int, int64_t, const uint8_t*, int64_t, const uint8_t*, int, int64_t,
     const uint8_t*, int64_t, int64_t, int64_t, int64_t, void*, int, int64_t, hipStream_t)
STUB(launch_grouped_gemm_mx, const uint8_t*, int, int64_t, const uint8_t*, int64_t, const uint8_t*, int, int64_t,
     int64_t, const uint8_t*, int64_t, int64_t, const int64_t*, int, int64_t, int64_t, int64_t, void*, int, int64_t,
     hipStream_t)
STUB(launch_moe_route, const int32_t*, int64_t, int, int, int64_t*, int32_t*, hipStream_t)
STUB(launch_moe_permute_quant_row, const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, int, int64_t, int, int,
     uint8_t*, int64_t, float*, hipStream_t)
STUB(launch_swiglu_quant_row, const uint16_t*, int64_t, int64_t, int64_t, int, int, uint8_t*, int64_t, float*,
     hipStream_t)
STUB(launch_moe_unpermute_combine, const uint16_t*, int64_t, int64_t, int64_t, const int32_t*, const float*, int64_t,
     int, uint16_t*, int64_t, hipStream_t)
#undef STUB
}  // namespace fp8amax

// Fake device pointers: 256-byte aligned, never dereferenced.
static void* dev(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + i * 0x100000ull); }
#define U16(i) static_cast<const uint16_t*>(dev(i))
#define U8(i) static_cast<uint8_t*>(dev(i))
#define F32(i) static_cast<float*>(dev(i))
#define I64(i) static_cast<int64_t*>(dev(i))
#define I32(i) static_cast<int32_t*>(dev(i))

static void expect(fp8_status_t st, fp8_status_t want, const char* launcher, int line) {
    if (st != want) {
        std::fprintf(stderr, "FAILED line %d: status %s (%s), expected %s\n", line, fp8_status_string(st),
                     fp8_last_error(), fp8_status_string(want));
        ++g_fail;
    }
    if (want == FP8_OK && launcher && g_last != launcher) {
        std::fprintf(stderr, "FAILED line %d: dispatched to %s, expected %s\n", line, g_last.c_str(), launcher);
        ++g_fail;
    }
    if (want != FP8_OK && std::strlen(fp8_last_error()) == 0) {
        std::fprintf(stderr, "FAILED line %d: no error message\n", line);
        ++g_fail;
    }
}
#define OK(call, launcher)                  \
    do {                                    \
        g_last.clear();                     \
        expect((call), FP8_OK, launcher, __LINE__); \
    } while (0)
#define ERR(call, want)                     \
    do {                                    \
        g_last.clear();                     \
        expect((call), want, nullptr, __LINE__); \
        CHECK(g_last.empty());              \
    } while (0)

int main() {
    const auto IA = FP8_ERR_INVALID_ARG, AL = FP8_ERR_ALIGNMENT, UN = FP8_ERR_UNSUPPORTED;
    fp8_device_info_t info;
    OK(fp8_query_device(0, &info), nullptr);
    CHECK(info.is_gfx950 == 1 && info.native_e4m3 == FP8_E4M3 && info.compute_units == 256);
    ERR(fp8_query_device(1, &info), IA);
    ERR(fp8_query_device(0, nullptr), IA);
    for (int s = 0; s <= 5; ++s) CHECK(fp8_status_string((fp8_status_t)s) != nullptr);

    // amax
    OK(fp8_amax(U16(1), 64, 128, 128, FP8_AXIS_ROW, F32(2), nullptr), "launch_amax");
    ERR(fp8_amax(U16(1), 64, 128, 100, FP8_AXIS_ROW, F32(2), nullptr), IA);
    ERR(fp8_amax(U16(1), 64, 128, 128, (fp8_axis_t)7, F32(2), nullptr), IA);
    ERR(fp8_amax(U16(1), 64, 128, 128, FP8_AXIS_COL, nullptr, nullptr), IA);
    ERR(fp8_amax(reinterpret_cast<const uint16_t*>((char*)dev(1) + 1), 4, 8, 8, FP8_AXIS_TENSOR, F32(2), nullptr), AL);
    OK(fp8_amax(nullptr, 0, 0, 1, FP8_AXIS_TENSOR, F32(2), nullptr), "launch_amax");

    // tensorwise
    OK(fp8_quantize_tensor(U16(1), 64, 128, 128, FP8_E4M3, 0, F32(3), U8(4), 128, F32(5), F32(6), nullptr),
       "launch_quant_tensor");
    ERR(fp8_quantize_tensor(U16(1), 64, 128, 128, FP8_E4M3, 33, nullptr, U8(4), 128, F32(5), F32(6), nullptr), IA);
    ERR(fp8_quantize_tensor(U16(1), 64, 128, 128, FP8_E4M3, 0, nullptr, U8(4), 128, nullptr, F32(6), nullptr), IA);
    ERR(fp8_quantize_tensor(U16(1), 64, 128, 128, (fp8_format_t)4, 0, nullptr, U8(4), 128, F32(5), F32(6), nullptr),
        IA);

    // rowwise, with and without the column-amax side output
    OK(fp8_quantize_row(U16(1), 64, 128, 128, FP8_E5M2, 1, U8(4), 128, F32(5), nullptr, nullptr, nullptr),
       "launch_quant_row");
    OK(fp8_quantize_row(U16(1), 64, 128, 128, FP8_E5M2, 1, U8(4), 128, F32(5), F32(6), F32(7), nullptr),
       "launch_quant_row_batch");
    ERR(fp8_quantize_row(U16(1), 64, 128, 128, FP8_E5M2, 1, U8(4), 100, F32(5), nullptr, nullptr, nullptr), IA);
    ERR(fp8_quantize_row(U16(1), 64, 128, 128, FP8_E5M2, -1, U8(4), 128, F32(5), nullptr, nullptr, nullptr), IA);
    ERR(fp8_quantize_row(U16(1), 64, 128, 128, FP8_E5M2, 0, U8(4), 128, nullptr, nullptr, nullptr, nullptr), IA);
    ERR(fp8_quantize_row(U16(1), 64, 128, 128, FP8_E5M2, 0, U8(4), 128, F32(5), nullptr,
                         reinterpret_cast<float*>((char*)dev(7) + 2), nullptr),
        AL);

    // batched rowwise: host arrays of exactly `count` entries (heap, so an
    // overread is reported), and every count from 1 to the maximum
    for (int count = 1; count <= FP8_MAX_ROW_BATCH; ++count) {
        std::vector<const uint16_t*> x(count);
        std::vector<int64_t> rows(count), ld(count);
        std::vector<uint8_t*> q(count);
        std::vector<float*> si(count), am(count), ca(count);
        for (int j = 0; j < count; ++j) {
            x[j] = U16(10 + j);
            rows[j] = 3 * j;
            ld[j] = 256;
            q[j] = U8(20 + j);
            si[j] = F32(30 + j);
            am[j] = j % 2 ? nullptr : F32(40 + j);
            ca[j] = j % 3 ? F32(50 + j) : nullptr;
        }
        OK(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                  si.data(), am.data(), ca.data(), nullptr, nullptr, nullptr),
           "launch_quant_row_batch");
        OK(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                  si.data(), nullptr, nullptr, nullptr, nullptr, nullptr),
           "launch_quant_row_batch");
        std::vector<const float*> sc(count);
        for (int j = 0; j < count; ++j) {
            sc[j] = F32(60 + j);
            am[j] = F32(70 + j);
        }
        OK(fp8_quantize_tensor_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, sc.data(), q.data(),
                                     ld.data(), si.data(), am.data(), nullptr),
           "launch_quant_tensor_batch");
        if (count > 1) {
            ld[count - 1] = 100;                                     // the last tensor's row stride is too small
            ERR(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                       si.data(), nullptr, nullptr, nullptr, nullptr, nullptr),
                IA);
        }
        // grouped column amax: group counts and offsets (host arrays of count entries)
        std::vector<const int64_t*> go(count);
        std::vector<int32_t> gn(count);
        for (int j = 0; j < count; ++j) {
            ld[j] = 256;
            ca[j] = F32(50 + j);
            go[j] = j % 2 ? nullptr : reinterpret_cast<const int64_t*>(dev(80 + j));
            gn[j] = j % 2 ? 0 : 3 + j;
        }
        OK(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                  si.data(), nullptr, ca.data(), go.data(), gn.data(), nullptr),
           "launch_quant_row_batch");
        gn[0] = 4097;
        ERR(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                   si.data(), nullptr, ca.data(), go.data(), gn.data(), nullptr),
            IA);
        gn[0] = 2;
        go[0] = nullptr;                                             // groups without offsets
        ERR(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                   si.data(), nullptr, ca.data(), go.data(), gn.data(), nullptr),
            IA);
        go[0] = reinterpret_cast<const int64_t*>((char*)dev(80) + 4);   // misaligned offsets
        ERR(fp8_quantize_row_batch(count, x.data(), rows.data(), 256, ld.data(), FP8_E4M3, 0, q.data(), ld.data(),
                                   si.data(), nullptr, ca.data(), go.data(), gn.data(), nullptr),
            AL);
    }
    {
        const uint16_t* x[1] = {U16(1)};
        int64_t rows[1] = {4}, ld[1] = {16};
        uint8_t* q[1] = {U8(2)};
        float* si[1] = {F32(3)};
        ERR(fp8_quantize_row_batch(0, x, rows, 16, ld, FP8_E4M3, 0, q, ld, si, nullptr, nullptr, nullptr, nullptr,
                                   nullptr),
            IA);
        ERR(fp8_quantize_row_batch(FP8_MAX_ROW_BATCH + 1, x, rows, 16, ld, FP8_E4M3, 0, q, ld, si, nullptr, nullptr,
                                   nullptr, nullptr, nullptr),
            IA);
        ERR(fp8_quantize_row_batch(1, nullptr, rows, 16, ld, FP8_E4M3, 0, q, ld, si, nullptr, nullptr, nullptr,
                                   nullptr, nullptr),
            IA);
        // grouped column amax with a layout the single-pass kernel does not take
        float* ca[1] = {F32(4)};
        const int64_t* go[1] = {reinterpret_cast<const int64_t*>(dev(5))};
        int32_t gn[1] = {2};
        int64_t ld12[1] = {12};
        ERR(fp8_quantize_row_batch(1, x, rows, 12, ld12, FP8_E4M3, 0, q, ld12, si, nullptr, ca, go, gn, nullptr), AL);
        ERR(fp8_quantize_row_batch(1, x, rows, 16, ld, FP8_E4M3, 0, q, ld, si, nullptr, nullptr, go, gn, nullptr), IA);
    }

    // colwise, transposed and not
    OK(fp8_quantize_col(U16(1), 64, 128, 128, FP8_E4M3, 0, 1, U8(2), 64, F32(3), F32(4), 0, nullptr),
       "launch_quant_col");
    OK(fp8_quantize_col(U16(1), 64, 128, 128, FP8_E4M3, 0, 0, U8(2), 128, F32(3), F32(4), 1, nullptr),
       "launch_quant_col");
    ERR(fp8_quantize_col(U16(1), 64, 128, 128, FP8_E4M3, 0, 1, U8(2), 32, F32(3), F32(4), 0, nullptr), IA);
    ERR(fp8_quantize_col(U16(1), 64, 128, 128, FP8_E4M3, 0, 0, U8(2), 64, F32(3), F32(4), 0, nullptr), IA);
    ERR(fp8_quantize_col(U16(1), 64, 128, 128, FP8_E4M3, 0, 2, U8(2), 64, F32(3), F32(4), 0, nullptr), IA);
    ERR(fp8_quantize_col(U16(1), 64, 128, 128, FP8_E4M3, 0, 1, U8(2), 64, F32(3), F32(4), 3, nullptr), IA);

    // dual cast
    OK(fp8_quantize_rowcol(U16(1), 64, 128, 128, FP8_E5M2, 0, U8(2), 128, F32(3), F32(4), U8(5), 64, F32(6), F32(7),
                           nullptr),
       "launch_quant_rowcol");
    ERR(fp8_quantize_rowcol(U16(1), 64, 128, 128, FP8_E5M2, 0, U8(2), 128, F32(3), nullptr, U8(5), 64, F32(6), F32(7),
                            nullptr),
        IA);
    ERR(fp8_quantize_rowcol(U16(1), 64, 128, 128, FP8_E5M2, 0, U8(2), 128, F32(3), F32(4), U8(5), 32, F32(6), F32(7),
                            nullptr),
        IA);
    ERR(fp8_quantize_rowcol(U16(1), 64, 120, 120, FP8_E5M2, 0, nullptr, 128, F32(3), F32(4), U8(5), 64, F32(6),
                            F32(7), nullptr),
        IA);
    ERR(fp8_quantize_rowcol(U16(1), 64, 124, 124, FP8_E5M2, 0, U8(2), 128, F32(3), F32(4), U8(5), 64, F32(6), F32(7),
                            nullptr),
        AL);

    // delayed update
    OK(fp8_delayed_scale_update(F32(1), F32(2), I32(3), 4, 1024, FP8_AMAX_MAX, 0, FP8_E4M3, F32(4), F32(5), nullptr),
       "launch_delayed_update");
    ERR(fp8_delayed_scale_update(F32(1), F32(2), I32(3), 4, 0, FP8_AMAX_MAX, 0, FP8_E4M3, F32(4), F32(5), nullptr), IA);
    ERR(fp8_delayed_scale_update(F32(1), F32(2), nullptr, 4, 8, FP8_AMAX_MAX, 0, FP8_E4M3, F32(4), F32(5), nullptr), IA);
    ERR(fp8_delayed_scale_update(F32(1), F32(2), I32(3), 4, 8, (fp8_amax_algo_t)2, 0, FP8_E4M3, F32(4), F32(5), nullptr),
        IA);

    // GEMMs
    OK(fp8_gemm_scaled(U8(1), FP8_E4M3, 4096, U8(2), FP8_E5M2, 4096, 512, 512, 4096, F32(3), FP8_SCALE_VECTOR, F32(4),
                       FP8_SCALE_TENSOR, dev(5), FP8_OUT_BF16, 512, nullptr),
       "launch_gemm");
    ERR(fp8_gemm_scaled(U8(1), FP8_E4M3, 4096, U8(2), FP8_E4M3, 4096, 512, 512, 4088, F32(3), FP8_SCALE_VECTOR, F32(4),
                        FP8_SCALE_VECTOR, dev(5), FP8_OUT_BF16, 512, nullptr),
        IA);
    OK(fp8_gemm_scaled(U8(1), FP8_E4M3_FNUZ, 4096, U8(2), FP8_E4M3, 4096, 512, 512, 4096, F32(3), FP8_SCALE_VECTOR,
                       F32(4), FP8_SCALE_VECTOR, dev(5), FP8_OUT_BF16, 512, nullptr),
       "launch_gemm_compat");
    OK(fp8_grouped_gemm_scaled(U8(1), FP8_E5M2_FNUZ, 7168, U8(2), FP8_E4M3_FNUZ, 7168, 2048 * 7168, I64(3), 32, 16384,
                               2048, 7168, F32(4), F32(5), dev(6), FP8_OUT_F32, 2048, nullptr),
       "launch_grouped_gemm_compat");
    ERR(fp8_gemm_scaled(U8(1), FP8_E4M3, 4100, U8(2), FP8_E4M3, 4096, 512, 512, 4096, F32(3), FP8_SCALE_VECTOR, F32(4),
                        FP8_SCALE_VECTOR, dev(5), FP8_OUT_BF16, 512, nullptr),
        AL);
    OK(fp8_grouped_gemm_scaled(U8(1), FP8_E4M3, 7168, U8(2), FP8_E4M3, 7168, 2048 * 7168, I64(3), 32, 16384, 2048, 7168,
                               F32(4), F32(5), dev(6), FP8_OUT_BF16, 2048, nullptr),
       "launch_grouped_gemm");
    ERR(fp8_grouped_gemm_scaled(U8(1), FP8_E4M3, 7168, U8(2), FP8_E4M3, 7168, 8, I64(3), 32, 16384, 2048, 7168, F32(4),
                                F32(5), dev(6), FP8_OUT_BF16, 2048, nullptr),
        AL);
    ERR(fp8_grouped_gemm_scaled(U8(1), FP8_E4M3, 7168, U8(2), FP8_E4M3, 7168, 0, I64(3), 0, 16384, 2048, 7168, F32(4),
                                F32(5), dev(6), FP8_OUT_BF16, 2048, nullptr),
        IA);

    // MoE backward
    OK(fp8_grouped_quantize_col(U16(1), 1000, 256, 256, FP8_E5M2, 0, I64(2), 4, U8(3), 2048, F32(4), F32(5), 0,
                                nullptr),
       "launch_grouped_quant_col");
    ERR(fp8_grouped_quantize_col(U16(1), 1000, 256, 256, FP8_E5M2, 0, I64(2), 4, U8(3), 2040, F32(4), F32(5), 0,
                                 nullptr),
        AL);
    OK(fp8_grouped_gemm_ragged_k(U8(1), FP8_E5M2, 2048, U8(2), FP8_E4M3, 2048, I64(3), 4, 1000, 256, 512, F32(4),
                                 F32(5), dev(6), FP8_OUT_BF16, 512, 256 * 512, nullptr),
       "launch_grouped_gemm_ragged_k");
    ERR(fp8_grouped_gemm_ragged_k(U8(1), FP8_E5M2, 992, U8(2), FP8_E4M3, 2048, I64(3), 4, 1000, 256, 512, F32(4),
                                  F32(5), dev(6), FP8_OUT_BF16, 512, 256 * 512, nullptr),
        IA);
    ERR(fp8_grouped_gemm_ragged_k(U8(1), FP8_E5M2_FNUZ, 2048, U8(2), FP8_E4M3, 2048, I64(3), 4, 1000, 256, 512,
                                  F32(4), F32(5), dev(6), FP8_OUT_BF16, 512, 256 * 512, nullptr),
        UN);
    ERR(fp8_grouped_gemm_ragged_k(U8(1), FP8_E5M2, 2048, U8(2), FP8_E4M3, 2048, I64(3), 4, 1000, 256, 512, F32(4),
                                  F32(5), dev(6), FP8_OUT_BF16, 512, 100, nullptr),
        IA);

    // MX and blockwise
    OK(fp8_mx_quantize_row(U16(1), 64, 256, 256, FP8_E4M3, U8(2), 256, U8(3), 64, nullptr), "launch_mx_quant_row");
    ERR(fp8_mx_quantize_row(U16(1), 64, 250, 256, FP8_E4M3, U8(2), 256, U8(3), 64, nullptr), IA);
    ERR(fp8_mx_quantize_row(U16(1), 64, 256, 256, FP8_E4M3_FNUZ, U8(2), 256, U8(3), 64, nullptr), IA);
    OK(fp8_gemm_mx(U8(1), FP8_E4M3, 4096, U8(2), 512, U8(3), FP8_E4M3, 4096, U8(4), 512, 512, 512, 4096, dev(5),
                   FP8_OUT_BF16, 512, nullptr),
       "launch_gemm_mx");
    ERR(fp8_gemm_mx(U8(1), FP8_E4M3, 4096, U8(2), 512, U8(3), FP8_E4M3, 4096, U8(4), 512, 512, 512, 4224, dev(5),
                    FP8_OUT_BF16, 512, nullptr),
        IA);
    ERR(fp8_gemm_mx(U8(1), FP8_E4M3, 4096, U8(2), 512, U8(3), FP8_E4M3, 4096, U8(4), 512, 512, 512, 4000, dev(5),
                    FP8_OUT_BF16, 512, nullptr),
        UN);
    OK(fp8_grouped_gemm_mx(U8(1), FP8_E4M3, 7168, U8(2), 16384, U8(3), FP8_E4M3, 7168, 2048 * 7168, U8(4), 65536,
                           8192, I64(5), 32, 16384, 2048, 7168, dev(6), FP8_OUT_BF16, 2048, nullptr),
       "launch_grouped_gemm_mx");
    OK(fp8_blockwise_quantize_act(U16(1), 64, 256, 256, FP8_E4M3, U8(2), 256, U8(3), 64, nullptr),
       "launch_blockwise_quant");
    OK(fp8_blockwise_quantize_weight(U16(1), 64, 256, 256, FP8_E4M3, U8(2), 256, U8(3), 64, nullptr),
       "launch_blockwise_quant");
    ERR(fp8_blockwise_quantize_weight(U16(1), 64, 200, 256, FP8_E4M3, U8(2), 256, U8(3), 64, nullptr), IA);

    // MoE layer forward
    OK(fp8_moe_route(I32(1), 2048, 8, 32, I64(2), I32(3), nullptr), "launch_moe_route");
    ERR(fp8_moe_route(I32(1), 2048, 65, 32, I64(2), I32(3), nullptr), IA);
    ERR(fp8_moe_route(I32(1), 2048, 8, 0, I64(2), I32(3), nullptr), IA);
    OK(fp8_moe_permute_quantize_row(U16(1), 2048, 7168, 7168, I32(2), 8, 16384, FP8_E4M3, 0, U8(3), 7168, F32(4),
                                    nullptr),
       "launch_moe_permute_quant_row");
    ERR(fp8_moe_permute_quantize_row(U16(1), 2048, 20000, 20000, I32(2), 8, 16384, FP8_E4M3, 0, U8(3), 20000, F32(4),
                                     nullptr),
        UN);
    OK(fp8_swiglu_quantize_row(U16(1), 16384, 2048, 4096, FP8_E4M3, 0, U8(2), 2048, F32(3), nullptr),
       "launch_swiglu_quant_row");
    ERR(fp8_swiglu_quantize_row(U16(1), 16384, 8192, 16384, FP8_E4M3, 0, U8(2), 8192, F32(3), nullptr), UN);
    OK(fp8_moe_unpermute_combine(reinterpret_cast<const uint16_t*>(dev(1)), 16384, 7168, 7168, I32(2), F32(3), 2048, 8,
                                 reinterpret_cast<uint16_t*>(dev(4)), 7168, nullptr),
       "launch_moe_unpermute_combine");
    ERR(fp8_moe_unpermute_combine(reinterpret_cast<const uint16_t*>(dev(1)), 16384, 7168, 7168, I32(2), F32(3), 2048, 0,
                                  reinterpret_cast<uint16_t*>(dev(4)), 7168, nullptr),
        IA);

    if (g_fail) {
        std::fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    std::printf("api host code: every check passed under the sanitizers\n");
    return 0;
}
