/*
 * fp8_oracle.c - plain CPU oracle for the FP8 linear layer of FP8 training.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark load this library. The HIP library never
 * links, loads or calls it; the two share no source, header, table or generator.
 *
 * What it computes, and where the pages fix it (pages cited by title and section):
 *  - The FP8 encodings. "FP8 Training on MI300X", section "DISCOVERED AMD FP8 DTYPE
 *    DIFFERENCE": e4m3fn/e5m2 (max 448) versus the fnuz variants with unsigned
 *    zero (e4m3 max 240). The bit layouts beyond those maxima are the standard
 *    OCP FP8 and fnuz definitions (sign, exponent with bias, mantissa).
 *  - Scale from amax with a power-of-two margin; delayed scaling over an amax
 *    history window with "most_recent" or "max". "FP8 training for Flux models",
 *    section "Configuration" (key FP8 parameters fp8_margin, fp8_amax_history_len,
 *    fp8_amax_compute_algo) and section "Troubleshooting / NaN or inf in losses".
 *  - Per-row / per-column ("colwise scales") / per-tensor scaling.
 *    "FP8 Training on AMD GPUs with TorchTitan and TorchAO" (rowwise FP8, the
 *    colwise-scales kernel) and "FP8 training for Flux models" (tensorwise/delayed).
 *  - The scaled FP8 GEMM, dense and grouped over MoE experts: the same two pages.
 *  - MX (block-32, power-of-two scaled) quantization and product: the MXFP8
 *    grouped GEMM the TorchTitan/TorchAO page names as next; the format is a
 *    reading, stated at the MX block section below.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - cast: saturate to +-fmax, then round to nearest, ties to even; NaN stays NaN;
 *    OCP keeps the sign of a zero result, fnuz has a single (unsigned) zero.
 *  - scale s = fl32(fmax / amax) * 2^-margin; amax 0 or non-finite -> s = 1
 *    (current scaling) or the previous s (delayed); fmax/amax overflowing fp32
 *    -> FLT_MAX. The dequantisation factor stored is fl32(1 / s).
 *  - element cast: p = fl32(x * s) first, then p is encoded (two roundings).
 *  - delayed: the window holds the last L recorded amaxes including the current
 *    one; the scale used at step t was computed at the end of step t-1; initial
 *    s = 1, history all zeros.
 *  - GEMM: Y = (sum_k dec(A_ik) dec(B_jk)) * sa_i * sb_j evaluated in fp64.
 *
 * Arithmetic is fp64 wherever a value is not fixed by a stated fp32 rounding.
 * Every loop is the definition written out; OpenMP only splits independent rows.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORC_E4M3 0
#define ORC_E5M2 1
#define ORC_E4M3_FNUZ 2
#define ORC_E5M2_FNUZ 3

#define ORC_ALGO_MOST_RECENT 0
#define ORC_ALGO_MAX 1

/* ---------------------------------------------------------------- formats -- */

typedef struct {
    int ebits, mbits, bias, fnuz;
    double fmax;
} orc_fmt;

static int fmt_get(int fmt, orc_fmt* f) {
    switch (fmt) {
        case ORC_E4M3:      f->ebits = 4; f->mbits = 3; f->bias = 7;  f->fnuz = 0; break;
        case ORC_E5M2:      f->ebits = 5; f->mbits = 2; f->bias = 15; f->fnuz = 0; break;
        case ORC_E4M3_FNUZ: f->ebits = 4; f->mbits = 3; f->bias = 8;  f->fnuz = 1; break;
        case ORC_E5M2_FNUZ: f->ebits = 5; f->mbits = 2; f->bias = 16; f->fnuz = 1; break;
        default: return -1;
    }
    /* Largest finite value. OCP e4m3 gives up the all-ones code to NaN, so its
     * largest mantissa at the top exponent is 110b; OCP e5m2 reserves the whole
     * top exponent for Inf/NaN; fnuz uses every code except 0x80. */
    int emax_field = (1 << f->ebits) - 1;
    int mmax = (1 << f->mbits) - 1;
    if (fmt == ORC_E4M3) mmax -= 1;
    if (fmt == ORC_E5M2) emax_field -= 1;
    f->fmax = ldexp((double)((1 << f->mbits) + mmax), emax_field - f->bias - f->mbits);
    return 0;
}

int orc_fmt_info(int fmt, double* fmax, int* ebits, int* mbits, int* bias) {
    orc_fmt f;
    if (fmt_get(fmt, &f)) return -1;
    *fmax = f.fmax; *ebits = f.ebits; *mbits = f.mbits; *bias = f.bias;
    return 0;
}

/* Value of one FP8 code: (-1)^s 2^(E-bias) (1 + M/2^m) for E > 0,
 * (-1)^s 2^(1-bias) M/2^m for E = 0, with the special codes of each encoding. */
double orc_decode(int fmt, uint8_t code) {
    orc_fmt f;
    if (fmt_get(fmt, &f)) return NAN;
    int s = code >> 7;
    int E = (code >> f.mbits) & ((1 << f.ebits) - 1);
    int M = code & ((1 << f.mbits) - 1);
    if (f.fnuz && code == 0x80) return NAN;
    if (fmt == ORC_E4M3 && E == 15 && M == 7) return NAN;
    if (fmt == ORC_E5M2 && E == 31) return M == 0 ? (s ? -INFINITY : INFINITY) : NAN;
    double mag = (E == 0) ? ldexp((double)M, 1 - f.bias - f.mbits)
                          : ldexp((double)((1 << f.mbits) + M), E - f.bias - f.mbits);
    return s ? -mag : mag;
}

/* Saturating round-to-nearest-even cast of one fp32 value. */
uint8_t orc_encode(int fmt, float p) {
    orc_fmt f;
    if (fmt_get(fmt, &f)) return 0;
    if (isnan(p)) return f.fnuz ? 0x80 : (signbit(p) ? 0xFF : 0x7F);
    int sign = signbit(p) ? 1 : 0;
    double a = fabs((double)p);
    if (a > f.fmax) a = f.fmax;                       /* saturate (Inf included) */
    int code;
    double min_normal = ldexp(1.0, 1 - f.bias);
    if (a < min_normal) {
        /* subnormal grid: multiples of 2^(1-bias-m); n = 2^m lands on min normal */
        double n = nearbyint(a / ldexp(1.0, 1 - f.bias - f.mbits));
        code = (int)n;
    } else {
        int e = ilogb(a);                             /* a in [2^e, 2^(e+1)) */
        double n = nearbyint(a / ldexp(1.0, e - f.mbits)); /* in [2^m, 2^(m+1)] */
        if (n == (double)(2 << f.mbits)) { e += 1; n = (double)(1 << f.mbits); }
        code = ((e + f.bias) << f.mbits) | ((int)n - (1 << f.mbits));
    }
    if (code == 0) return (f.fnuz || !sign) ? 0x00 : 0x80;
    return (uint8_t)(code | (sign << 7));
}

void orc_encode_array(int fmt, const float* p, int64_t n, uint8_t* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = orc_encode(fmt, p[i]);
}

void orc_decode_array(int fmt, const uint8_t* c, int64_t n, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(fmt, c[i]);
}

/* ------------------------------------------------------------------ scales -- */

static float bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float v;
    memcpy(&v, &u, 4);
    return v;
}

/* Order used for every amax: magnitudes compare as numbers, and NaN is larger
 * than everything (a NaN anywhere in the domain makes the amax NaN). */
static float amax_combine(float acc, float v) {
    if (isnan(acc)) return acc;
    if (isnan(v)) return fabsf(v);
    float a = fabsf(v);
    return a > acc ? a : acc;
}

/* s = fl32(fmax/amax) * 2^-margin. fp64 division rounded once to fp32 equals the
 * correctly rounded fp32 quotient (53 >= 2*24+2). Overflow of the quotient gives
 * FLT_MAX. Returns 0 when amax is 0 or not finite: the caller picks the fallback. */
static int scale_from_amax(int fmt, float amax, int margin, float* s_out) {
    orc_fmt f;
    fmt_get(fmt, &f);
    if (!(amax > 0.0f) || !isfinite(amax)) return 0;
    float s = (float)(f.fmax / (double)amax);
    if (isinf(s)) s = FLT_MAX;
    s = (float)((double)s * ldexp(1.0, -margin));
    *s_out = s;
    return 1;
}

float orc_scale_current(int fmt, float amax, int margin) {
    float s;
    return scale_from_amax(fmt, amax, margin, &s) ? s : 1.0f;
}

float orc_reciprocal(float s) { return (float)(1.0 / (double)s); }

/* One element: p = fl32(x*s) (the fp64 product of a bf16 and an fp32 is exact),
 * then the saturating RNE cast of p. */
uint8_t orc_quantize_value(int fmt, uint16_t x_bf16, float s) {
    float p = (float)((double)bf16_value(x_bf16) * (double)s);
    return orc_encode(fmt, p);
}

/* ------------------------------------------------------------------- amax -- */

/* axis 0: whole tensor -> out[0]; axis 1: per row -> out[rows]; axis 2: per column -> out[cols] */
void orc_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis, float* out) {
    if (axis == 0) {
        /* the tensor's amax is the amax of its row amaxes */
        float acc = 0.0f;
        #pragma omp parallel
        {
            float part = 0.0f;
            #pragma omp for schedule(static)
            for (int64_t i = 0; i < rows; ++i)
                for (int64_t j = 0; j < cols; ++j) part = amax_combine(part, bf16_value(x[i * ldx + j]));
            #pragma omp critical
            acc = amax_combine(acc, part);
        }
        out[0] = acc;
    } else if (axis == 1) {
        #pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            float acc = 0.0f;
            for (int64_t j = 0; j < cols; ++j) acc = amax_combine(acc, bf16_value(x[i * ldx + j]));
            out[i] = acc;
        }
    } else {
        #pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < cols; ++j) {
            float acc = 0.0f;
            for (int64_t i = 0; i < rows; ++i) acc = amax_combine(acc, bf16_value(x[i * ldx + j]));
            out[j] = acc;
        }
    }
}

/* ------------------------------------------------------------- quantizers -- */

/* Per-row current scaling: one scale per row over its cols elements. */
void orc_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                      uint8_t* q, int64_t ldq, float* scale_inv, float* amax) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        float a = 0.0f;
        for (int64_t j = 0; j < cols; ++j) a = amax_combine(a, bf16_value(x[i * ldx + j]));
        float s = orc_scale_current(fmt, a, margin);
        for (int64_t j = 0; j < cols; ++j) q[i * ldq + j] = orc_quantize_value(fmt, x[i * ldx + j], s);
        scale_inv[i] = orc_reciprocal(s);
        if (amax) amax[i] = a;
    }
}

/* Per-column current scaling (one scale per column over the rows), written
 * transposed: qt[j*ldqt + i] holds element (i, j). */
void orc_quantize_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                      uint8_t* qt, int64_t ldqt, float* scale_inv, float* amax) {
    #pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < cols; ++j) {
        float a = 0.0f;
        for (int64_t i = 0; i < rows; ++i) a = amax_combine(a, bf16_value(x[i * ldx + j]));
        float s = orc_scale_current(fmt, a, margin);
        for (int64_t i = 0; i < rows; ++i) qt[j * ldqt + i] = orc_quantize_value(fmt, x[i * ldx + j], s);
        scale_inv[j] = orc_reciprocal(s);
        if (amax) amax[j] = a;
    }
}

/* Tensorwise cast with a given scale s (delayed scaling: s comes from the state).
 * Writes the dequantisation factor that was used and folds this tensor's amax
 * into *amax_acc (max with what it already holds). */
void orc_quantize_tensor_scaled(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt,
                                float s, uint8_t* q, int64_t ldq, float* scale_inv_used, float* amax_acc) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) q[i * ldq + j] = orc_quantize_value(fmt, x[i * ldx + j], s);
    float a;
    orc_amax(x, rows, cols, ldx, 0, &a);
    *amax_acc = amax_combine(*amax_acc, a);
    *scale_inv_used = orc_reciprocal(s);
}

/* Tensorwise current scaling: amax over the whole tensor, then one scale. */
void orc_quantize_tensor_current(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                                 uint8_t* q, int64_t ldq, float* scale_inv, float* amax) {
    float a;
    orc_amax(x, rows, cols, ldx, 0, &a);
    float s = orc_scale_current(fmt, a, margin);
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) q[i * ldq + j] = orc_quantize_value(fmt, x[i * ldx + j], s);
    *scale_inv = orc_reciprocal(s);
    *amax = a;
}

/* --------------------------------------------------------- delayed scaling -- */

/* End-of-step update of n delayed-scaling states. history is [n x L], a ring
 * whose next slot is *head (shared by the n tensors). For each tensor: record
 * cur_amax in the ring; the effective amax is the one just recorded
 * ("most_recent") or the max over all L slots ("max"); if it is finite and
 * positive the scale becomes fl32(fmax/amax_eff) * 2^-margin, else the scale is
 * kept; cur_amax is cleared for the next step. Then the head advances. */
void orc_delayed_update(float* cur_amax, float* history, int32_t* head, int64_t n, int L, int algo, int margin,
                        int fmt, float* scale, float* scale_inv) {
    int h = *head;
    for (int64_t i = 0; i < n; ++i) {
        float* hist = history + i * (int64_t)L;
        hist[h] = cur_amax[i];
        float eff;
        if (algo == ORC_ALGO_MOST_RECENT) {
            eff = cur_amax[i];
        } else {
            eff = 0.0f;
            for (int t = 0; t < L; ++t) eff = amax_combine(eff, hist[t]);
        }
        float s;
        if (scale_from_amax(fmt, eff, margin, &s)) {
            scale[i] = s;
            scale_inv[i] = orc_reciprocal(s);
        }
        cur_amax[i] = 0.0f;
    }
    *head = (h + 1) % L;
}

/* ------------------------------------------------------------------- GEMM -- */

/* Y[i, j] = (sum_k dec(A[i, k]) * dec(B[j, k])) * sa * sb in fp64, with
 * sa = a_scale[i] (a_vec) or a_scale[0], likewise sb. A is [m x k] (row stride
 * lda), B is [n x k] (row stride ldb): Y = A * B^T. bound (if not NULL) gets
 * |sa * sb| * sum_k |dec(A[i, k]) * dec(B[j, k])|. */
static double dot_row(const double* ar, const double* br, int64_t k, double* abs_sum) {
    double s = 0.0, t = 0.0;
    for (int64_t kk = 0; kk < k; ++kk) {
        double p = ar[kk] * br[kk];
        s += p;
        t += fabs(p);
    }
    *abs_sum = t;
    return s;
}

static void decode_rows(const uint8_t* src, int64_t rows, int64_t k, int64_t ld, int fmt, double* dst) {
    double lut[256];
    for (int c = 0; c < 256; ++c) lut[c] = orc_decode(fmt, (uint8_t)c);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t kk = 0; kk < k; ++kk) dst[r * k + kk] = lut[src[r * ld + kk]];
}

/* Dense product over all outputs. ad/bd are caller scratch of m*k and n*k doubles. */
void orc_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
              int64_t m, int64_t n, int64_t k, const float* a_scale, int a_vec, const float* b_scale, int b_vec,
              double* ad, double* bd, double* y, int64_t ldy, double* bound) {
    decode_rows(a, m, k, lda, fa, ad);
    decode_rows(b, n, k, ldb, fb, bd);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        double sa = a_scale[a_vec ? i : 0];
        for (int64_t j = 0; j < n; ++j) {
            double sb = b_scale[b_vec ? j : 0];
            double t;
            double s = dot_row(ad + i * k, bd + j * k, k, &t);
            y[i * ldy + j] = s * sa * sb;
            if (bound) bound[i * ldy + j] = fabs(sa * sb) * t;
        }
    }
}

/* Selected outputs only: Y[ii[e], jj[e]] for e < count (for shapes too large to
 * evaluate whole). Decodes each needed operand row on the fly. */
void orc_gemm_entries(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t k,
                      const float* a_scale, int a_vec, const float* b_scale, int b_vec,
                      const int64_t* ii, const int64_t* jj, int64_t count, double* y, double* bound) {
    double la[256], lb[256];
    for (int c = 0; c < 256; ++c) { la[c] = orc_decode(fa, (uint8_t)c); lb[c] = orc_decode(fb, (uint8_t)c); }
    #pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        const uint8_t* ar = a + ii[e] * lda;
        const uint8_t* br = b + jj[e] * ldb;
        double s = 0.0, t = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double p = la[ar[kk]] * lb[br[kk]];
            s += p;
            t += fabs(p);
        }
        double sa = a_scale[a_vec ? ii[e] : 0], sb = b_scale[b_vec ? jj[e] : 0];
        y[e] = s * sa * sb;
        if (bound) bound[e] = fabs(sa * sb) * t;
    }
}

/* Grouped (MoE) product: rows offsets[g]..offsets[g+1]-1 of A belong to expert
 * g, whose weight is B_g = b + g*b_group_stride ([n x k], row stride ldb) with
 * per-output scales b_scale[g*n + j]. a_scale has one entry per row of A.
 * Each group is the dense product above; empty groups produce nothing. */
void orc_grouped_gemm_entries(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                              int64_t b_group_stride, const int64_t* offsets, int g, int64_t n, int64_t k,
                              const float* a_scale, const float* b_scale,
                              const int64_t* ii, const int64_t* jj, int64_t count, double* y, double* bound) {
    double la[256], lb[256];
    for (int c = 0; c < 256; ++c) { la[c] = orc_decode(fa, (uint8_t)c); lb[c] = orc_decode(fb, (uint8_t)c); }
    #pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        int64_t i = ii[e], j = jj[e];
        int grp = -1;
        for (int gg = 0; gg < g; ++gg)
            if (offsets[gg] <= i && i < offsets[gg + 1]) { grp = gg; break; }
        if (grp < 0) { y[e] = NAN; if (bound) bound[e] = NAN; continue; }
        const uint8_t* ar = a + i * lda;
        const uint8_t* br = b + grp * b_group_stride + j * ldb;
        double s = 0.0, t = 0.0;
        for (int64_t kk = 0; kk < k; ++kk) {
            double p = la[ar[kk]] * lb[br[kk]];
            s += p;
            t += fabs(p);
        }
        double sa = a_scale[i], sb = b_scale[(int64_t)grp * n + j];
        y[e] = s * sa * sb;
        if (bound) bound[e] = fabs(sa * sb) * t;
    }
}

/* --------------------------------------------------------------- MX blocks -- */
/* MXFP8: the pages name an MXFP8 grouped GEMM for MI355X as the next step of
 * the MoE work ("FP8 Training on AMD GPUs with TorchTitan and TorchAO",
 * summary) without defining the block format. Reading used here, the plainest
 * microscaling one: each row is cut into blocks of 32 consecutive elements
 * along K; a block shares a power-of-two scale X = 2^e stored as the biased
 * exponent e + 127 (E8M0, 0xFF = NaN) with e = floor(log2(amax)) - emax, emax
 * the exponent of the element format's largest normal (8 for e4m3, 15 for
 * e5m2), clamped to [-127, 127]; an all-zero block gets e = -127; a block with
 * a NaN or Inf gets 0xFF and its elements are cast with scale 1. An element is
 * the saturating RNE cast of x * 2^-e (exact in fp32): values of the top binade
 * above fmax saturate. Dequantised value: dec(code) * X. OCP encodings only. */
#define ORC_MX_BLOCK 32

static int mx_emax(int fmt) { return fmt == ORC_E4M3 ? 8 : 15; }

/* Biased scale exponent of a block whose amax (max |x|, NaN dominating) is a. */
uint8_t orc_mx_scale(int fmt, float amax) {
    if (!isfinite(amax)) return 0xFF;
    if (!(amax > 0.0f)) return 0;
    int e = ilogbf(amax) - mx_emax(fmt);                  /* floor(log2(amax)) - emax */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (uint8_t)(e + 127);
}

double orc_mx_scale_value(uint8_t s) { return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127); }

/* Rowwise MX quantization: x [rows x cols] (cols % 32 == 0) -> codes q
 * [rows x cols] and scales [rows x cols/32] (row stride lds). */
void orc_mx_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                         int64_t ldq, uint8_t* scale, int64_t lds) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b0 = 0; b0 < cols; b0 += ORC_MX_BLOCK) {
            float amax = 0.0f;
            for (int64_t c = b0; c < b0 + ORC_MX_BLOCK; ++c) amax = amax_combine(amax, bf16_value(x[r * ldx + c]));
            uint8_t s = orc_mx_scale(fmt, amax);
            scale[r * lds + b0 / ORC_MX_BLOCK] = s;
            double mul = (s == 0xFF) ? 1.0 : ldexp(1.0, 127 - (int)s);
            for (int64_t c = b0; c < b0 + ORC_MX_BLOCK; ++c)
                q[r * ldq + c] = orc_encode(fmt, (float)((double)bf16_value(x[r * ldx + c]) * mul));
        }
    }
}

/* MX product Y = A * B^T in fp64: Y[i, j] = sum over blocks b of X_a[i, b] *
 * X_b[j, b] * sum_{k in b} dec(A[i, k]) * dec(B[j, k]); bound (if not NULL)
 * gets the same with |.| of every term. A [m x k] with scales sa [m x k/32]
 * (row stride ldsa), B [n x k] with sb [n x k/32]. ad/bd: caller scratch of
 * m*k and n*k doubles. */
void orc_mx_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* sa, int64_t ldsa, const uint8_t* b, int fb,
                 int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t m, int64_t n, int64_t k, double* ad,
                 double* bd, double* y, int64_t ldy, double* bound) {
    decode_rows(a, m, k, lda, fa, ad);
    decode_rows(b, n, k, ldb, fb, bd);
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0, t = 0.0;
            for (int64_t b0 = 0; b0 < k; b0 += ORC_MX_BLOCK) {
                double x = orc_mx_scale_value(sa[i * ldsa + b0 / ORC_MX_BLOCK]) *
                           orc_mx_scale_value(sb[j * ldsb + b0 / ORC_MX_BLOCK]);
                double bt;
                double bs = dot_row(ad + i * k + b0, bd + j * k + b0, ORC_MX_BLOCK, &bt);
                s += x * bs;
                t += fabs(x) * bt;
            }
            y[i * ldy + j] = s;
            if (bound) bound[i * ldy + j] = t;
        }
    }
}
