/*
 * fp8amax.h - C ABI of the MI355X (gfx950) FP8 linear-layer library.
 *
 * The operations are the hot path of the FP8 linear layer of FP8 training:
 * amax reduction, scale computation (current and delayed), a saturating
 * round-to-nearest-even cast to FP8, and the FP8 GEMM with fp32 accumulation and
 * a scale-applying epilogue, dense and grouped over MoE experts. Sources:
 *   [Flux]  "FP8 training for Flux models" (ROCm Primus docs): section
 *           "Configuration" (fp8 e4m3/hybrid, recipes delayed/tensorwise,
 *           fp8_margin, fp8_amax_history_len, fp8_amax_compute_algo, fp8_wgrad),
 *           section "Troubleshooting / NaN or inf in losses", section "Testing /
 *           Numerical verification status" (fused delayed-scale update).
 *   [MI300] "FP8 Training on MI300X": section on the AMD FP8 dtype difference
 *           (e4m3fn/e5m2 with e4m3 max 448 vs e4m3fnuz/e5m2fnuz with max 240 and
 *           unsigned zero; e4m3 forward, e5m2 backward).
 *   [Titan] "FP8 Training on AMD GPUs with TorchTitan and TorchAO": summary
 *           (rowwise FP8, fused quantization kernels, colwise scales, grouped
 *           GEMM for MoE) and its answers on the wrong-max corruption and on
 *           the non-coalesced colwise-scale writes.
 *   [Kimbodo] "How PyTorch FP8 Optimizations on AMD GPUs Reduce LLM Cost and
 *           Scale Training Past 1,000 GPUs": What Happened (per-MoE-layer
 *           latency).
 *
 * Conventions common to every entry point
 *  - Pointers named x, q, qt, amax*, scale*, history, head, a, b, d and
 *    group_offsets are DEVICE pointers owned by the caller. The library
 *    allocates nothing and keeps no state between calls except a per-device
 *    properties cache.
 *  - Matrices are row-major with an explicit leading dimension counted in
 *    elements (ldx for bf16 inputs, ldq/lda/ldb for FP8 codes, ldd for the
 *    output). A bf16 tensor is passed as its 16-bit patterns.
 *  - stream is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on it and returns; there is no host synchronisation and
 *    no device-to-host copy.
 *  - Errors: arguments are checked on the host before anything is launched;
 *    on error nothing is enqueued and the call returns a non-zero status.
 *    fp8_last_error() then describes it (thread-local). No exception crosses
 *    the ABI.
 *  - The cast, for every encoding (readings of [Flux]/[MI300]/[Titan], which
 *    do not spell out the arithmetic): with s the scale, p = fl32(x * s), then
 *    p is clamped to +-fmax (Inf saturates), rounded to the nearest FP8 value
 *    with ties to even, NaN -> NaN code (sign|0x7F for OCP, 0x80 for fnuz);
 *    a zero result keeps its sign in OCP and is 0x00 in fnuz.
 *  - Current scaling: s = fl32(fmax / amax) * 2^-margin (fmax / amax rounded
 *    once to fp32, FLT_MAX if it overflows); s = 1 if amax is 0 or not finite.
 *    Quantizers store scale_inv = fl32(1 / s), the factor that dequantises.
 *  - amax is max |x| over the reduction domain, returned in fp32; a NaN in the
 *    domain makes it NaN.
 */
#ifndef FP8AMAX_H
#define FP8AMAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 encodings [MI300]. OCP: e4m3 (max 448, no Inf, NaN = S.1111.111, signed
 * zero), e5m2 (max 57344, Inf and NaN in the top exponent, signed zero).
 * fnuz: e4m3 (bias 8, max 240) and e5m2 (bias 16, max 57344), no Inf, a single
 * zero, NaN = 0x80. gfx950's matrix cores consume the OCP encodings. */
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1, FP8_E4M3_FNUZ = 2, FP8_E5M2_FNUZ = 3 } fp8_format_t;

typedef enum { FP8_AXIS_TENSOR = 0, FP8_AXIS_ROW = 1, FP8_AXIS_COL = 2 } fp8_axis_t;

/* fp8_amax_compute_algo of [Flux] "Configuration". */
typedef enum { FP8_AMAX_MOST_RECENT = 0, FP8_AMAX_MAX = 1 } fp8_amax_algo_t;

/* A GEMM operand's dequantisation factor: one value, or one per row of the operand. */
typedef enum { FP8_SCALE_TENSOR = 0, FP8_SCALE_VECTOR = 1 } fp8_scale_mode_t;

typedef enum { FP8_OUT_BF16 = 0, FP8_OUT_F32 = 1 } fp8_out_t;

typedef enum {
    FP8_OK = 0,
    FP8_ERR_INVALID_ARG = 1,  /* null pointer, negative size, ld < width, bad enum, margin out of range */
    FP8_ERR_ALIGNMENT = 2,    /* a pointer or leading dimension breaks a stated alignment */
    FP8_ERR_UNSUPPORTED = 3,  /* valid request this build does not run (device not gfx950, fnuz MX / ragged-K operands) */
    FP8_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} fp8_status_t;

typedef struct {
    char arch[64];                /* gcnArchName, e.g. "gfx950:sramecc+:xnack-" */
    int32_t is_gfx950;            /* 1 if this library's kernels run on the device */
    int32_t native_e4m3;          /* encoding the matrix cores consume: FP8_E4M3 on gfx950, FP8_E4M3_FNUZ on gfx942 */
    int32_t native_e5m2;
    int32_t compute_units;
    int32_t lds_bytes_per_block;  /* sharedMemPerBlock */
    int64_t global_mem_bytes;
} fp8_device_info_t;

/* Availability probe (the role of [Flux]'s is_fp8_available check): fills
 * *info for HIP device `device`. Returns FP8_ERR_INVALID_ARG for a bad index
 * or NULL info, FP8_ERR_HIP if the runtime fails. Host-synchronous. */
fp8_status_t fp8_query_device(int device, fp8_device_info_t* info);

/* Static string naming a status code. */
const char* fp8_status_string(fp8_status_t status);

/* Message of the last error returned on the calling thread ("" if none). */
const char* fp8_last_error(void);

/* amax reduction ([Titan] rowwise and colwise scales; [Flux] tensorwise/delayed).
 * x: bf16 [rows x cols], row stride ldx >= cols. axis selects the domain:
 *   FP8_AXIS_TENSOR -> amax_out[0]; FP8_AXIS_ROW -> amax_out[rows];
 *   FP8_AXIS_COL -> amax_out[cols]. amax_out (fp32) is overwritten.
 * Alignment: x 2-byte aligned; 16-byte aligned x with ldx % 8 == 0 takes the
 * vector path. Empty domains give 0. */
fp8_status_t fp8_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_axis_t axis,
                      float* amax_out, void* stream);

/* Tensorwise quantization ([Flux] recipes "delayed" and "tensorwise").
 * x: bf16 [rows x cols] (ldx); q: codes [rows x cols] (ldq >= cols).
 *  - scale != NULL (delayed scaling): *scale (device fp32) is the scale to
 *    use; writes scale_inv_out[0] = fl32(1 / *scale) (the factor actually
 *    used, so it cannot disagree with a later state update), and FOLDS the
 *    tensor's amax into amax_out[0] (amax_out[0] = max(amax_out[0], amax(x))):
 *    amax_out is the delayed state's cur_amax, cleared by
 *    fp8_delayed_scale_update. margin is ignored (the state applies it).
 *  - scale == NULL (current scaling): amax_out[0] is overwritten with amax(x),
 *    s is computed from it with `margin`, scale_inv_out[0] = fl32(1 / s).
 * margin: 0..32. amax_out and scale_inv_out are required. */
fp8_status_t fp8_quantize_tensor(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                                 int32_t margin, const float* scale, uint8_t* q, int64_t ldq,
                                 float* scale_inv_out, float* amax_out, void* stream);

/* Rowwise quantization ([Titan] rowwise FP8: one scale per row, e.g. per token
 * of an activation or per output row of a weight). One pass over x: row amax,
 * scale, cast. x: bf16 [rows x cols] (ldx); q: codes [rows x cols] (ldq).
 * scale_inv_out[rows] (required); amax_out[rows] (optional, NULL to skip);
 * col_amax_out[cols] (optional): if given, it is overwritten with the
 * per-column amax of x, a side output for a later colwise quantization of the
 * same tensor (fp8_quantize_col with col_amax_ready = 1). On the vector path
 * with cols <= 16384 the column amax comes from the same single pass over x
 * (after a launch that clears col_amax_out); longer rows or other layouts
 * take a second pass over x for it.
 * margin: 0..32. Vector path when x, q are 16/8-byte aligned and ldx, ldq,
 * cols are multiples of 8; any other layout takes a scalar path. */
fp8_status_t fp8_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                              int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out, float* amax_out,
                              float* col_amax_out, void* stream);

/* Rowwise quantization of several tensors that share cols in one launch
 * ([Titan]: fused quantization kernels cut the launches and HBM round trips
 * of the FP8 path; a linear layer's activation [m x k] and weight [n x k]
 * share k). Tensor j (j < count) is x[j] (bf16 [rows[j] x cols], ldx[j]) with
 * codes q[j] (ldq[j]), scale_inv_out[j] [rows[j]] (required when rows[j] > 0)
 * amax_out[j] [rows[j]] and col_amax_out[j] [cols] (amax_out and col_amax_out
 * themselves, or any of their entries, may be NULL); every result equals what
 * fp8_quantize_row gives for that tensor alone, the column amax of a tensor
 * included (e.g. a linear layer's X and W, whose column amax the backward's
 * colwise casts of X^T and W^T then take as ready). x, rows, ldx, q, ldq,
 * scale_inv_out, amax_out, col_amax_out are HOST arrays of count entries (read
 * during the call); the pointers in them are device memory. count:
 * 1..FP8_MAX_ROW_BATCH. All tensors share fmt and margin. One launch (two
 * with column amax: the outputs are cleared first) when every tensor has the
 * vector layout (x 16-byte and q 8-byte aligned, ldx, ldq, cols multiples of
 * 8) and cols <= 16384; otherwise one launch per tensor, and a second pass
 * over each tensor whose column amax is asked for.
 * Grouped column amax (the per-group amax that fp8_grouped_quantize_col then
 * takes with col_amax_ready = 1, e.g. for the MoE backward's casts of X^T,
 * W^T and dY^T, whose groups are an expert's tokens or its weight rows):
 * col_groups (HOST int32 [count], or NULL for none) gives tensor j's group
 * count G_j, 0..4096 (0: one amax per column over all rows, as above);
 * with G_j > 0, col_group_offsets[j] (HOST array of count DEVICE pointers;
 * entry j: int64 [G_j + 1], non-decreasing, as for fp8_grouped_quantize_col)
 * is required and col_amax_out[j] [G_j x cols] receives, for each group g and
 * column c, the amax of column c over rows offsets[g] .. offsets[g+1]-1
 * (0 for an empty group; rows outside [offsets[0], offsets[G_j]) count in no
 * group). Still one pass over x, needing for every tensor of the call the
 * vector layout and cols <= 16384 (else FP8_ERR_ALIGNMENT /
 * FP8_ERR_UNSUPPORTED). Errors: any tensor's argument error (as
 * fp8_quantize_row) fails the whole call before anything is enqueued. */
#define FP8_MAX_ROW_BATCH 8
fp8_status_t fp8_quantize_row_batch(int32_t count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                    const int64_t* ldx, fp8_format_t fmt, int32_t margin, uint8_t* const* q,
                                    const int64_t* ldq, float* const* scale_inv_out, float* const* amax_out,
                                    float* const* col_amax_out, const int64_t* const* col_group_offsets,
                                    const int32_t* col_groups, void* stream);

/* Delayed tensorwise quantization of several tensors that share cols in one
 * launch ([Flux] delayed recipe; a linear layer's X and W, each with its own
 * delayed state). Tensor j is cast exactly as fp8_quantize_tensor with
 * scale = scale[j] (device fp32, required) would: scale_inv_out[j][0] =
 * fl32(1 / *scale[j]) and the tensor's amax is folded into amax_out[j][0] (the
 * state's cur_amax, cleared by fp8_delayed_scale_update). x, rows, ldx, scale,
 * q, ldq, scale_inv_out, amax_out are HOST arrays of count entries (all
 * required); the pointers in them are device memory. count: 1..FP8_MAX_ROW_BATCH.
 * One launch when every tensor has rows > 0 and the vector layout (x 16-byte,
 * q 8-byte aligned; ldx, ldq, cols multiples of 8) and cols <= 16384; otherwise
 * one launch per tensor. Errors as fp8_quantize_tensor, for any tensor, before
 * anything is enqueued. */
fp8_status_t fp8_quantize_tensor_batch(int32_t count, const uint16_t* const* x, const int64_t* rows, int64_t cols,
                                       const int64_t* ldx, fp8_format_t fmt, const float* const* scale,
                                       uint8_t* const* q, const int64_t* ldq, float* const* scale_inv_out,
                                       float* const* amax_out, void* stream);

/* Colwise quantization ([Titan] colwise scales, whose non-coalesced writes
 * the post singles out). One scale per column of x (reduction over the rows,
 * e.g. over tokens).
 *  - transpose_out = 1: the codes are written transposed so that the next
 *    GEMM's contraction dimension is contiguous: q[j * ldq + i] =
 *    cast(x[i * ldx + j] * s_j), q is [cols x rows], ldq >= rows (the layout
 *    every GEMM operand of this library takes). The transpose goes through
 *    LDS in tiles, so reads and writes are both coalesced.
 *  - transpose_out = 0: the codes keep x's layout, q[i * ldq + j] =
 *    cast(x[i * ldx + j] * s_j), q is [rows x cols], ldq >= cols.
 * col_amax[cols]: if col_amax_ready == 0 it is overwritten with the column
 * amax (computed by a first pass over x); if 1 it is read as already holding
 * it (from fp8_amax(FP8_AXIS_COL) or fp8_quantize_row's side output).
 * scale_inv_out[cols] (required). margin: 0..32; transpose_out: 0 or 1. */
fp8_status_t fp8_quantize_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                              int32_t margin, int32_t transpose_out, uint8_t* q, int64_t ldq, float* scale_inv_out,
                              float* col_amax, int32_t col_amax_ready, void* stream);

/* Dual cast of one tensor: rowwise codes and colwise-transposed codes ([Flux]
 * "Configuration": fp8 hybrid and fp8_wgrad, where the output gradient dY
 * feeds the dgrad rowwise and the wgrad colwise; [Titan] colwise scales and
 * fused quantization kernels). Gives exactly what fp8_quantize_row (q,
 * scale_inv_out, amax_out) and fp8_quantize_col with transpose_out = 1 (qt,
 * col_scale_inv_out, col_amax_out) give, in two passes over x instead of
 * three: the row and column amax together, then one pass writing both code
 * tensors. x: bf16 [rows x cols] (ldx); q: codes [rows x cols] (ldq >= cols);
 * qt: codes [cols x rows] (ldqt >= rows). scale_inv_out[rows], amax_out[rows],
 * col_scale_inv_out[cols] and col_amax_out[cols] are all required (the amax
 * outputs hold the first pass's results). Requirements: x 16-byte aligned,
 * ldx and cols multiples of 8; q 8-byte aligned, ldq % 8 == 0 (else
 * FP8_ERR_ALIGNMENT). margin: 0..32. */
fp8_status_t fp8_quantize_rowcol(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                                 int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out, float* amax_out,
                                 uint8_t* qt, int64_t ldqt, float* col_scale_inv_out, float* col_amax_out,
                                 void* stream);

/* Fused end-of-step update of n delayed-scaling states ([Flux] "Configuration":
 * fp8_amax_history_len, fp8_amax_compute_algo, fp8_margin; [Flux] "Testing":
 * the fused delayed-scale update). State layout, all device memory:
 *   cur_amax[n]   amax recorded this step (fp8_quantize_tensor folds into it);
 *   history[n*L]  ring of the last L recorded amaxes per tensor (row i at i*L);
 *   head[1]       int32 next ring slot, shared by the n tensors, in [0, L);
 *   scale[n], scale_inv[n].
 * For each tensor: history[i*L + head] = cur_amax[i]; amax_eff = cur_amax[i]
 * (MOST_RECENT) or the max over the L slots (MAX); if amax_eff is finite and
 * > 0: scale[i] = fl32(fmax / amax_eff) * 2^-margin (FLT_MAX on overflow),
 * scale_inv[i] = fl32(1 / scale[i]); otherwise both are kept. cur_amax[i] = 0.
 * Then head = (head + 1) % L. Initial state: history 0, head 0, scale 1,
 * scale_inv 1, cur_amax 0. L: 1..65536; margin 0..32. */
fp8_status_t fp8_delayed_scale_update(float* cur_amax, float* history, int32_t* head, int64_t n, int32_t L,
                                      fp8_amax_algo_t algo, int32_t margin, fp8_format_t fmt, float* scale,
                                      float* scale_inv, void* stream);

/* Scaled FP8 GEMM ([Titan] FP8 linear layers; [Flux] FP8 wgrad):
 *   d[i, j] = out( fp32acc( sum_k dec(a[i, k]) * dec(b[j, k]) ) * sa_i * sb_j )
 * a: codes [m x k] (lda), b: codes [n x k] (ldb): both K-contiguous, d = a * b^T
 * (for y = x * w^T, a = x and b = w). sa_i = a_scale_inv[i] (VECTOR, [m]) or
 * a_scale_inv[0] (TENSOR); likewise sb_j with b_scale_inv ([n]). The scales
 * are the quantizers' scale_inv outputs (device fp32). out: bf16
 * (round-to-nearest-even) or fp32, d [m x n] with row stride ldd >= n.
 * Formats: fa, fb any of the four encodings, mixed allowed ([Flux] "hybrid":
 * e4m3 activations and weights, e5m2 gradients). OCP pairs run on the FP8
 * matrix cores. A pair with a fnuz operand ([MI300]: the encodings of MI300
 * parts, which gfx950's FP8 matrix cores do not consume and no fixed
 * re-encoding maps onto OCP) takes a compatibility path: both operands are
 * decoded to bf16 (exact for every FP8 value) and multiplied on the bf16
 * matrix cores with fp32 accumulation, the same arithmetic at a lower rate.
 * Requirements: k % 16 == 0; a, b 16-byte aligned; lda, ldb multiples of 16;
 * d 4-byte aligned. m, n >= 0 arbitrary (ragged tiles are masked); k == 0
 * writes zeros times the scales. */
fp8_status_t fp8_gemm_scaled(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* b, fp8_format_t fb,
                             int64_t ldb, int64_t m, int64_t n, int64_t k, const float* a_scale_inv,
                             fp8_scale_mode_t a_mode, const float* b_scale_inv, fp8_scale_mode_t b_mode, void* d,
                             fp8_out_t d_type, int64_t ldd, void* stream);

/* Grouped (MoE) scaled FP8 GEMM ([Titan]: FP8 grouped GEMM for mixture-of-experts
 * layers). Rows of a are sorted by expert: rows group_offsets[g] ..
 * group_offsets[g+1]-1 belong to expert g, whose weight is
 * b_g = b + g * b_group_stride (codes [n x k], row stride ldb). For those rows:
 *   d[i, j] = out( fp32acc( sum_k dec(a[i, k]) * dec(b_g[j, k]) ) * a_scale_inv[i] * b_scale_inv[g*n + j] ).
 * group_offsets: DEVICE int64 [g+1], non-decreasing, offsets[0] = 0,
 * offsets[g] = total_m (the library cannot read it without a host sync, so
 * it is not checked; rows outside [0, total_m) are never touched). Empty groups
 * produce nothing. a: [total_m x k]; a_scale_inv [total_m]; b_scale_inv [g x n];
 * d [total_m x n]. b_group_stride >= 0, a multiple of 16; the groups' weights may
 * interleave (e.g. b_group_stride = k with ldb = g * k: the experts' columns of
 * one grouped transposed matrix, see below). Formats and alignment as
 * fp8_gemm_scaled; g: 1..4096. */
fp8_status_t fp8_grouped_gemm_scaled(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* b,
                                     fp8_format_t fb, int64_t ldb, int64_t b_group_stride,
                                     const int64_t* group_offsets, int32_t g, int64_t total_m, int64_t n, int64_t k,
                                     const float* a_scale_inv, const float* b_scale_inv, void* d, fp8_out_t d_type,
                                     int64_t ldd, void* stream);

/* ------------------------------------------------------------ MoE backward --
 * The backward of an MoE layer ([Titan]: FP8 grouped GEMM for MoE, the colwise
 * scales of the MoE layer, the MoE model's backward-pass speedup). For expert g
 * with tokens offsets[g] .. offsets[g+1]-1 (m_g rows), forward y_g = x_g w_g^T:
 *   dgrad dx_g = dy_g w_g: fp8_quantize_row(dy) times w_g quantized per column
 *     over its rows (fp8_grouped_quantize_col on the stacked weights, groups of
 *     n rows), with fp8_grouped_gemm_scaled;
 *   wgrad dw_g = dy_g^T x_g: a contraction over the group's own tokens, so dy
 *     and x are quantized per column over each group's tokens
 *     (fp8_grouped_quantize_col) and multiplied by fp8_grouped_gemm_ragged_k.
 * Grouped transposed layout (a reading: the pages name no layout): the codes
 * of group g sit at columns P_g .. P_g + m_g - 1 of one matrix, where
 * P_g = sum over h < g of roundup(m_h, FP8_GROUP_K_ALIGN), and columns
 * P_g + m_g .. P_{g+1} - 1 hold zero codes. P_G <= total_m + g * (FP8_GROUP_K_ALIGN - 1). */
#define FP8_GROUP_K_ALIGN 256

/* Grouped colwise quantization. x: bf16 [total_m x cols] (ldx), rows sorted by
 * group per group_offsets (DEVICE int64 [g+1], non-decreasing, offsets[0] = 0,
 * offsets[g] = total_m; not checked, rows outside [0, total_m) are never
 * touched). Per group g and column j: s_{g,j} from the amax of column j over
 * the group's rows only, and
 *   qt[j * ldqt + P_g + (i - offsets[g])] = cast(x[i * ldx + j] * s_{g,j}),
 * zero codes in the group's padding. qt: [cols x ldqt]; columns >= ldqt are
 * never written, so ldqt >= P_G is needed for the whole result
 * (total_m + g * (FP8_GROUP_K_ALIGN - 1) always suffices; ldqt >= total_m is
 * checked). col_amax [g x cols]: overwritten when col_amax_ready == 0, read as
 * already holding the per-group column amax when 1. scale_inv_out [g x cols]
 * (required). An empty group has amax 0 and scale 1. Requirements: x 16-byte
 * aligned, ldx and cols multiples of 8; qt 16-byte aligned, ldqt % 16 == 0;
 * g: 1..4096; margin: 0..32. */
fp8_status_t fp8_grouped_quantize_col(const uint16_t* x, int64_t total_m, int64_t cols, int64_t ldx,
                                      fp8_format_t fmt, int32_t margin, const int64_t* group_offsets, int32_t g,
                                      uint8_t* qt, int64_t ldqt, float* scale_inv_out, float* col_amax,
                                      int32_t col_amax_ready, void* stream);

/* Grouped GEMM over ragged contraction ranges (the MoE weight gradient):
 *   d_g[i, j] = out( fp32acc( sum_{t < m_g} dec(a[i * lda + P_g + t]) * dec(b[j * ldb + P_g + t]) )
 *                    * a_scale_inv[g * m + i] * b_scale_inv[g * n + j] )
 * for g = 0..G-1, m_g and P_g from group_offsets as above (offsets[g] =
 * total_m). a: codes [m x lda] and b: codes [n x ldb] in the grouped
 * transposed layout, whose zero padding lets the contraction run over
 * roundup(m_g, FP8_GROUP_K_ALIGN) columns (the padding must hold zero codes,
 * as fp8_grouped_quantize_col writes it). d_g = d + g * d_group_stride
 * (elements), [m x n] with row stride ldd; d_group_stride >= m * ldd. An
 * empty group writes 0 * sa * sb. Columns at or past min(lda, ldb) are never
 * read: lda, ldb >= P_G is needed (total_m + g * (FP8_GROUP_K_ALIGN - 1)
 * always suffices), and since P_G depends on the device offsets it is not
 * checked on the host; a group whose padded range P_g + roundup(m_g,
 * FP8_GROUP_K_ALIGN) runs past min(lda, ldb) writes NaN to its whole output
 * instead of a sum that silently misses columns. Checked: lda, ldb >= total_m;
 * lda, ldb < 2^24 (else FP8_ERR_UNSUPPORTED). Alignment as fp8_gemm_scaled;
 * formats OCP e4m3 / e5m2 only (fnuz: FP8_ERR_UNSUPPORTED); g: 1..4096. */
fp8_status_t fp8_grouped_gemm_ragged_k(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* b,
                                       fp8_format_t fb, int64_t ldb, const int64_t* group_offsets, int32_t g,
                                       int64_t total_m, int64_t m, int64_t n, const float* a_scale_inv,
                                       const float* b_scale_inv, void* d, fp8_out_t d_type, int64_t ldd,
                                       int64_t d_group_stride, void* stream);

/* ------------------------------------------------------------------- MXFP8 --
 * Block-scaled FP8 ([Flux] section "Configuration": mxfp8 among the recipes;
 * [Titan] summary and next steps: MXFP8 grouped GEMM for MI355X). The pages
 * name the recipe without defining it; this follows the OCP microscaling
 * (MX) format, a reading: along K (the row of x, a and b), every block of
 * FP8_MX_BLOCK consecutive elements shares one scale X = 2^e stored as the
 * E8M0 byte e + 127 (255 = NaN). For a block with amax = max |x| over its
 * elements:
 *   e = floor(log2 amax) - emax (emax 8 for e4m3, 15 for e5m2), clamped to
 *       -127..127; a zero block has e = -127;
 *   element code = cast(x * 2^-e) with the saturating RNE cast above;
 *   a block holding a NaN or an Inf gets the byte 255 and its elements are
 *   cast with scale 1.
 * Only the OCP encodings (e4m3, e5m2) carry MX data. */
#define FP8_MX_BLOCK 32

/* Scale layout of the MX entry points (K-step major, a layout of this
 * library): the scales of blocks 4j .. 4j+3 of row r (elements 128j ..
 * 128j + 127) are the four bytes, in block order, of the 4-byte record at
 * scale + 4 * (j * ld_scale + r); ld_scale >= rows counts records. A matrix
 * with cols columns has ceil(cols / 128) record rows, (ceil(cols / 128) - 1)
 * * ld_scale + rows records in all. The 256 rows of a GEMM tile then bring
 * one K step's scales in as one contiguous 1 KB run per operand. */

/* MX rowwise quantization. x: bf16 [rows x cols] (ldx); q: codes [rows x cols]
 * (ldq); scale_e8m0: the rows' block scales as records (above; bytes of
 * blocks past cols / 32 in the last record are written as 0). Requirements:
 * cols % 32 == 0; x 16-byte aligned, ldx % 8 == 0; q 8-byte aligned,
 * ldq % 8 == 0; scale_e8m0 4-byte aligned, ld_scale >= rows; rows < 2^26
 * (else FP8_ERR_UNSUPPORTED); fmt e4m3 or e5m2. */
fp8_status_t fp8_mx_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, fp8_format_t fmt,
                                 uint8_t* q, int64_t ldq, uint8_t* scale_e8m0, int64_t ld_scale, void* stream);

/* MX GEMM:
 *   d[i, j] = out( sum over blocks c < k/32 of
 *                  2^(sa(i, c) - 127) * 2^(sb(j, c) - 127)
 *                  * sum_{t in block c} dec(a[i * lda + t]) * dec(b[j * ldb + t]) )
 * accumulated in fp32 (a NaN scale byte makes the sums it enters NaN), where
 * sa(i, c) is block c's scale of row i of a in the records of a_scale (record
 * stride ld_as >= m), sb(j, c) likewise in b_scale (ld_bs >= n). a: codes
 * [m x k], b: codes [n x k] (K-contiguous rows, b is W as stored).
 * Requirements: k % 256 == 0 (else FP8_ERR_UNSUPPORTED); the scales 4-byte
 * aligned; lda, ldb < 2^24 (else FP8_ERR_UNSUPPORTED); fewer than 2^24 tiles
 * of 256 x 256; output type, formats (OCP only) and operand alignment as
 * fp8_gemm_scaled. */
fp8_status_t fp8_gemm_mx(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* a_scale, int64_t ld_as,
                         const uint8_t* b, fp8_format_t fb, int64_t ldb, const uint8_t* b_scale, int64_t ld_bs,
                         int64_t m, int64_t n, int64_t k, void* d, fp8_out_t d_type, int64_t ldd, void* stream);

/* Grouped MX GEMM (MoE experts): rows offsets[g] .. offsets[g+1]-1 of a
 * (scale records of a_scale, ld_as >= total_m) and of d belong to group g,
 * whose weights are the codes b + g * b_group_stride [n x k] (ldb) with the
 * scale records at b_scale + g * b_scale_group_stride (bytes; ld_bs >= n);
 * each group's rows as fp8_gemm_mx. group_offsets as fp8_grouped_gemm_scaled
 * (device int64 [g+1], clamped to [0, total_m]). b_group_stride % 16 == 0,
 * b_scale_group_stride % 4 == 0, g: 1..4096; otherwise as fp8_gemm_mx. */
fp8_status_t fp8_grouped_gemm_mx(const uint8_t* a, fp8_format_t fa, int64_t lda, const uint8_t* a_scale,
                                 int64_t ld_as, const uint8_t* b, fp8_format_t fb, int64_t ldb, int64_t b_group_stride,
                                 const uint8_t* b_scale, int64_t ld_bs, int64_t b_scale_group_stride,
                                 const int64_t* group_offsets, int32_t g, int64_t total_m, int64_t n, int64_t k,
                                 void* d, fp8_out_t d_type, int64_t ldd, void* stream);

/* ---------------------------------------------------------------- blockwise --
 * Blockwise recipe ([Flux] section "Configuration": blockwise among the
 * recipes; no block shapes or scale rule on the pages). Reading: activations
 * and gradients take one scale per 1 x 128 block along K (per row), weights
 * one per 128 x 128 tile; the scale s is the current-scaling scale fmax / amax
 * of the block (1 for a zero or non-finite amax, FLT_MAX at most) rounded down
 * to a power of two, so no element saturates; codes are cast(x * s). s is
 * stored as the E8M0 byte of 1 / s in the MX scale records (above), all four
 * bytes of a record equal (a 128-deep K step is one block), so blockwise
 * operands multiply with fp8_gemm_mx / fp8_grouped_gemm_mx. Requirements of
 * both: cols % 128 == 0; x 16-byte aligned, ldx % 8 == 0; q 8-byte aligned,
 * ldq % 8 == 0; records 4-byte aligned, ld_scale >= rows; rows < 2^26 (else
 * FP8_ERR_UNSUPPORTED); fmt e4m3 or e5m2. */

/* 1 x 128 blocks of x bf16 [rows x cols] (ldx). */
fp8_status_t fp8_blockwise_quantize_act(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx,
                                        fp8_format_t fmt, uint8_t* q, int64_t ldq, uint8_t* scale_records,
                                        int64_t ld_scale, void* stream);

/* 128 x 128 tiles of w bf16 [rows x cols] (ldw; the last row tile may be
 * shorter); every row of a tile gets the tile's record. */
fp8_status_t fp8_blockwise_quantize_weight(const uint16_t* w, int64_t rows, int64_t cols, int64_t ldw,
                                           fp8_format_t fmt, uint8_t* q, int64_t ldq, uint8_t* scale_records,
                                           int64_t ld_scale, void* stream);

/* -------------------------------------------------------- MoE layer forward --
 * The MoE layer around its two grouped GEMMs ([Kimbodo] What Happened: the
 * per-MoE-layer latency; [Titan] fused quantization kernels, FP8 grouped GEMM
 * for MoE). The pages do not define the layer; the reading is the plain top-k
 * MoE feed-forward layer: token t goes to the experts expert_idx[t, 0..k-1];
 * expert e applies y = down( silu(x gate_e^T) * (x up_e^T) ); the k results are
 * summed with the router's weights. The forward, all on the device:
 *   fp8_moe_route                  -> expert offsets and each entry's row
 *   fp8_moe_permute_quantize_row   -> tokens cast rowwise into expert order
 *   fp8_grouped_gemm_scaled        -> h = [gate | up] per expert (bf16)
 *   fp8_swiglu_quantize_row        -> silu(gate) * up cast rowwise
 *   fp8_grouped_gemm_scaled        -> expert outputs in expert order (bf16)
 *   fp8_moe_unpermute_combine      -> weighted sum back in token order
 * An "entry" is a (token, slot) pair, numbered t * topk + j. */

/* Routing: expert_idx int32 [tokens x topk] (device). A stable counting sort of
 * the entries by expert: offsets_out int64 [num_experts + 1] (expert e owns
 * rows offsets[e] .. offsets[e+1]-1), dest_out int32 [tokens x topk] = the row
 * of each entry, entries of one expert in entry order (deterministic). An
 * index outside [0, num_experts) drops its entry: dest = -1, not counted.
 * Limits: topk 1..64, num_experts 1..1024, tokens * topk < 2^31. One
 * workgroup: meant for the per-GPU token counts of a layer (tens of thousands
 * of entries). */
fp8_status_t fp8_moe_route(const int32_t* expert_idx, int64_t tokens, int32_t topk, int32_t num_experts,
                           int64_t* offsets_out, int32_t* dest_out, void* stream);

/* Permutation fused with the rowwise cast: token t of x bf16 [tokens x cols]
 * (ldx) is quantized once (as fp8_quantize_row) and its codes and scale_inv
 * written to rows dest[t * topk + j] (j < topk) of q [rows_out x cols] (ldq)
 * and scale_inv_out [rows_out]. Destinations outside [0, rows_out) are
 * skipped. Requirements: x 16-byte aligned, ldx and cols multiples of 8,
 * cols <= 16384 (else FP8_ERR_UNSUPPORTED); q 8-byte aligned, ldq % 8 == 0;
 * margin 0..32. */
fp8_status_t fp8_moe_permute_quantize_row(const uint16_t* x, int64_t tokens, int64_t cols, int64_t ldx,
                                          const int32_t* dest, int32_t topk, int64_t rows_out, fp8_format_t fmt,
                                          int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out,
                                          void* stream);

/* SwiGLU fused with the rowwise cast: row r of h bf16 [rows x 2 inter] (ldh)
 * holds gate (columns 0 .. inter-1) and up (inter .. 2 inter-1);
 * a = silu(gate) * up = gate / (1 + exp(-gate)) * up in fp32, then per row
 * s from max |a| (the current-scaling rule), q[r] = cast(a * s),
 * scale_inv_out[r] = 1 / s. q: codes [rows x inter] (ldq). Requirements: h
 * 16-byte aligned, ldh and inter multiples of 8, inter <= 4096 (else
 * FP8_ERR_UNSUPPORTED); q 8-byte aligned, ldq % 8 == 0. */
fp8_status_t fp8_swiglu_quantize_row(const uint16_t* h, int64_t rows, int64_t inter, int64_t ldh, fp8_format_t fmt,
                                     int32_t margin, uint8_t* q, int64_t ldq, float* scale_inv_out, void* stream);

/* Weighted combine back to token order:
 *   out[t] = bf16( sum over j = 0 .. topk-1, in that order, of
 *                  weights[t * topk + j] * y[dest[t * topk + j]] )
 * with fp32 accumulation; y bf16 [rows x cols] (ldy) in expert order, out bf16
 * [tokens x cols] (ldo); slots whose destination is outside [0, rows) add
 * nothing. Requirements: y and out 16-byte aligned, ldy, ldo and cols
 * multiples of 8. */
fp8_status_t fp8_moe_unpermute_combine(const uint16_t* y, int64_t rows, int64_t cols, int64_t ldy,
                                       const int32_t* dest, const float* weights, int64_t tokens, int32_t topk,
                                       uint16_t* out, int64_t ldo, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8AMAX_H */
