// kernels.hpp - host-side launchers of the device kernels (internal to the
// library; the public interface is include/fp8amax.h). Each launcher assumes
// its arguments were validated by the C ABI layer and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8amax {

struct DeviceProps {
    int cus;
};
const DeviceProps& current_device_props();

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st);

hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis, float* out,
                       hipStream_t st);

// reread: x is read again right after (the column amax pass), so it is loaded
// through the caches; otherwise as streamed input (nontemporal loads).
hipError_t launch_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                            uint8_t* q, int64_t ldq, float* scale_inv, float* amax_out, bool reread, hipStream_t st);

// Rowwise casts of count tensors sharing cols (host arrays of count entries;
// amax_out and col_amax, or any of their entries, may be NULL): one launch
// when all take the register kernel (after a clearing launch when a column
// amax is asked for: it is then a side output of the same pass).
hipError_t launch_quant_row_batch(int count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                  const int64_t* ldx, int fmt, int margin, uint8_t* const* q, const int64_t* ldq,
                                  float* const* scale_inv, float* const* amax_out, float* const* col_amax,
                                  const int64_t* const* col_groups, const int32_t* ngroups, hipStream_t st);

// transpose: codes written transposed (qt [cols x rows]) or in x's layout (q [rows x cols]).
hipError_t launch_quant_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                            int transpose, uint8_t* qt, int64_t ldqt, float* scale_inv, const float* col_amax,
                            hipStream_t st);

// Dual cast (vector layout: x 16-byte aligned, ldx and cols multiples of 8; q
// 8-byte aligned, ldq % 8 == 0): row amax and column amax in one pass, then
// one pass writing the rowwise codes q and the colwise codes qt (transposed).
hipError_t launch_quant_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                               uint8_t* q, int64_t ldq, float* row_scale_inv, float* row_amax, uint8_t* qt,
                               int64_t ldqt, float* col_scale_inv, float* col_amax, hipStream_t st);

hipError_t launch_quant_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                               const float* scale, uint8_t* q, int64_t ldq, float* scale_inv, float* amax,
                               hipStream_t st);

// Delayed tensorwise casts of count tensors sharing cols (host arrays of
// count entries, every scale[j] set): one launch when all take the register kernel.
hipError_t launch_quant_tensor_batch(int count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                     const int64_t* ldx, int fmt, const float* const* scale, uint8_t* const* q,
                                     const int64_t* ldq, float* const* scale_inv, float* const* amax,
                                     hipStream_t st);

hipError_t launch_delayed_update(float* cur_amax, float* history, int32_t* head, int64_t n, int32_t L, int algo,
                                 int margin, int fmt, float* scale, float* scale_inv, hipStream_t st);

hipError_t launch_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t m,
                       int64_t n, int64_t k, const float* sa, int sa_vec, const float* sb, int sb_vec, void* d,
                       int out_f32, int64_t ldd, hipStream_t st);

hipError_t launch_grouped_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                               int64_t b_group_stride, const int64_t* offsets, int g, int64_t total_m, int64_t n,
                               int64_t k, const float* sa, const float* sb, void* d, int out_f32, int64_t ldd,
                               hipStream_t st);

// Products with fnuz operands (any of the four encodings on either side): the
// operands decoded to bf16 in registers and multiplied on the bf16 matrix cores.
hipError_t launch_gemm_compat(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t m,
                              int64_t n, int64_t k, const float* sa, int sa_vec, const float* sb, int sb_vec, void* d,
                              int out_f32, int64_t ldd, hipStream_t st);

hipError_t launch_grouped_gemm_compat(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                                      int64_t b_group_stride, const int64_t* offsets, int g, int64_t total_m,
                                      int64_t n, int64_t k, const float* sa, const float* sb, void* d, int out_f32,
                                      int64_t ldd, hipStream_t st);

// MoE backward: per-group colwise quantization into the grouped transposed
// layout, and the grouped product over ragged contraction ranges.
constexpr int64_t kGroupKAlign = 256;

hipError_t launch_grouped_quant_col(const uint16_t* x, int64_t total_m, int64_t cols, int64_t ldx, int fmt,
                                    int margin, const int64_t* offsets, int g, uint8_t* qt, int64_t ldqt,
                                    float* scale_inv, float* col_amax, int col_amax_ready, hipStream_t st);

hipError_t launch_grouped_gemm_ragged_k(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                                        const int64_t* offsets, int g, int64_t total_m, int64_t m, int64_t n,
                                        const float* sa, const float* sb, void* d, int out_f32, int64_t ldd,
                                        int64_t d_group_stride, hipStream_t st);

// MXFP8: rowwise block-32 quantization with E8M0 scales, and the products
// whose operands carry such scales along K (dense, and grouped over rows).
hipError_t launch_mx_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                               int64_t ldq, uint8_t* scale, int64_t ld_scale, hipStream_t st);

// Blockwise casts (1 x 128 activation blocks, or 128 x 128 weight tiles when
// weight != 0) with power-of-two scales, into MX scale records.
hipError_t launch_blockwise_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int weight,
                                  uint8_t* q, int64_t ldq, uint8_t* scale, int64_t ld_scale, hipStream_t st);

hipError_t launch_gemm_mx(const uint8_t* a, int fa, int64_t lda, const uint8_t* xa, int64_t ld_xa, const uint8_t* b,
                          int fb, int64_t ldb, const uint8_t* xb, int64_t ld_xb, int64_t m, int64_t n, int64_t k,
                          void* d, int out_f32, int64_t ldd, hipStream_t st);

hipError_t launch_grouped_gemm_mx(const uint8_t* a, int fa, int64_t lda, const uint8_t* xa, int64_t ld_xa,
                                  const uint8_t* b, int fb, int64_t ldb, int64_t b_group_stride, const uint8_t* xb,
                                  int64_t ld_xb, int64_t xb_group_stride, const int64_t* offsets, int g,
                                  int64_t total_m, int64_t n, int64_t k, void* d, int out_f32, int64_t ldd,
                                  hipStream_t st);

// MoE layer forward: routing, permutation fused with the rowwise cast, SwiGLU
// fused with the rowwise cast, weighted combine.
constexpr int kMoeMaxExperts = 1024;
constexpr int kMoeMaxTopk = 64;
constexpr int kSwigluMaxChunks = 8;                  // 16-byte chunks per lane: intermediate size <= 4096

hipError_t launch_moe_route(const int32_t* idx, int64_t tokens, int topk, int num_experts, int64_t* offsets,
                            int32_t* dest, hipStream_t st);

hipError_t launch_moe_permute_quant_row(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ldx,
                                        const int32_t* dest, int topk, int64_t rows_out, int fmt, int margin,
                                        uint8_t* q, int64_t ldq, float* scale_inv, hipStream_t st);

hipError_t launch_swiglu_quant_row(const uint16_t* h, int64_t rows, int64_t inter, int64_t ldh, int fmt, int margin,
                                   uint8_t* q, int64_t ldq, float* scale_inv, hipStream_t st);

hipError_t launch_moe_unpermute_combine(const uint16_t* y, int64_t rows, int64_t cols, int64_t ldy,
                                        const int32_t* dest, const float* wts, int64_t tokens, int topk,
                                        uint16_t* out, int64_t ldo, hipStream_t st);

}  // namespace fp8amax
