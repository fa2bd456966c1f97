/* Drives every C entry point of the CPU oracle (oracle/fp8_oracle.c) on small
 * ragged shapes and special values, for a build with the address and
 * undefined-behaviour sanitizers (tests/test_oracle_sanitize.py). Exits 0 when
 * the few consistency checks below hold; the sanitizers abort on any invalid
 * access or undefined operation. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_fmt_info(int fmt, double* fmax, int* ebits, int* mbits, int* bias);
double orc_decode(int fmt, uint8_t code);
uint8_t orc_encode(int fmt, float p);
void orc_encode_array(int fmt, const float* p, int64_t n, uint8_t* out);
void orc_decode_array(int fmt, const uint8_t* c, int64_t n, double* out);
float orc_scale_current(int fmt, float amax, int margin);
float orc_reciprocal(float s);
uint8_t orc_quantize_value(int fmt, uint16_t x_bf16, float s);
void orc_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int axis, float* out);
void orc_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin, uint8_t* q,
                      int64_t ldq, float* scale_inv, float* amax);
void orc_quantize_col(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin, uint8_t* qt,
                      int64_t ldqt, float* scale_inv, float* amax);
void orc_quantize_tensor_scaled(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, float s,
                                uint8_t* q, int64_t ldq, float* scale_inv_used, float* amax_acc);
void orc_quantize_tensor_current(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, int margin,
                                 uint8_t* q, int64_t ldq, float* scale_inv, float* amax);
void orc_delayed_update(float* cur_amax, float* history, int32_t* head, int64_t n, int L, int algo, int margin,
                        int fmt, float* scale, float* scale_inv);
void orc_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t m, int64_t n,
              int64_t k, const float* a_scale, int a_vec, const float* b_scale, int b_vec, double* ad, double* bd,
              double* y, int64_t ldy, double* bound);
void orc_gemm_entries(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb, int64_t k,
                      const float* a_scale, int a_vec, const float* b_scale, int b_vec, const int64_t* ii,
                      const int64_t* jj, int64_t count, double* y, double* bound);
void orc_grouped_gemm_entries(const uint8_t* a, int fa, int64_t lda, const uint8_t* b, int fb, int64_t ldb,
                              int64_t b_group_stride, const int64_t* offsets, int g, int64_t n, int64_t k,
                              const float* a_scale, const float* b_scale, const int64_t* ii, const int64_t* jj,
                              int64_t count, double* y, double* bound);
uint8_t orc_mx_scale(int fmt, float amax);
double orc_mx_scale_value(uint8_t s);
void orc_mx_quantize_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                         int64_t ldq, uint8_t* scale, int64_t lds);
void orc_mx_gemm(const uint8_t* a, int fa, int64_t lda, const uint8_t* sa, int64_t ldsa, const uint8_t* b, int fb,
                 int64_t ldb, const uint8_t* sb, int64_t ldsb, int64_t m, int64_t n, int64_t k, double* ad,
                 double* bd, double* y, int64_t ldy, double* bound);

static uint32_t rng_state = 12345u;
static uint32_t rnd(void) {   /* xorshift32: inputs only */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}
static uint16_t bf16_of(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
/* bf16 matrix with mixed magnitudes and, every 37th element, a special value */
static uint16_t* make_x(int64_t rows, int64_t ld) {
    uint16_t* x = malloc((size_t)(rows * ld) * sizeof *x);
    const float special[] = {0.0f, -0.0f, NAN, INFINITY, -INFINITY, 1e-40f, 3e38f, 448.0f, 57344.0f};
    for (int64_t i = 0; i < rows * ld; ++i) {
        float v = ((float)(rnd() % 20001) - 10000.0f) / 977.0f * ldexpf(1.0f, (int)(rnd() % 17) - 8);
        if (i % 37 == 5) v = special[(i / 37) % 9];
        x[i] = bf16_of(v);
    }
    return x;
}
static uint8_t* make_codes(int64_t n, int fmt) {
    uint8_t* c = malloc((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        uint8_t v = (uint8_t)(rnd() & 0xFF);
        while (isnan(orc_decode(fmt, v)) || isinf(orc_decode(fmt, v))) v = (uint8_t)(rnd() & 0xFF);
        c[i] = v;
    }
    return c;
}

int main(void) {
    int bad = 0;
    for (int fmt = 0; fmt < 4; ++fmt) {
        double fmax;
        int e, mb, bias;
        if (orc_fmt_info(fmt, &fmax, &e, &mb, &bias) != 0) bad |= 1;
        for (int c = 0; c < 256; ++c) {   /* finite codes round-trip (fnuz: no -0) */
            double v = orc_decode(fmt, (uint8_t)c);
            if (isfinite(v) && !(v == 0.0 && c != 0) && orc_encode(fmt, (float)v) != c) bad |= 2;
        }
        float p[64];
        uint8_t q[64];
        double d[64];
        for (int i = 0; i < 64; ++i) p[i] = ((float)i - 32.0f) * 7.3f;
        orc_encode_array(fmt, p, 64, q);
        orc_decode_array(fmt, q, 64, d);
        (void)orc_quantize_value(fmt, 0x3F81, orc_scale_current(fmt, 3.0f, 1));
        (void)orc_reciprocal(orc_scale_current(fmt, 0.0f, 0));

        const int64_t rows = 37, cols = 45, ld = 48;
        uint16_t* x = make_x(rows, ld);
        uint8_t* qr = malloc(rows * ld);
        uint8_t* qt = malloc(cols * (rows + 3));
        float* si = malloc(sizeof(float) * 64);
        float* am = malloc(sizeof(float) * 64);
        for (int axis = 0; axis < 3; ++axis) orc_amax(x, rows, cols, ld, axis, am);
        orc_quantize_row(x, rows, cols, ld, fmt, 2, qr, ld, si, am);
        orc_quantize_col(x, rows, cols, ld, fmt, 0, qt, rows + 3, si, am);
        float used, acc = 0.5f;
        orc_quantize_tensor_scaled(x, rows, cols, ld, fmt, 0.75f, qr, ld, &used, &acc);
        orc_quantize_tensor_current(x, rows, cols, ld, fmt, 1, qr, ld, &used, &acc);
        orc_quantize_row(x, 0, cols, ld, fmt, 0, qr, ld, si, am);    /* empty */

        /* delayed state: 3 tensors, L = 4, 10 steps with zero / NaN / Inf amax */
        float cur[3], hist[12] = {0}, sc[3] = {1, 1, 1}, sci[3] = {1, 1, 1};
        int32_t head = 0;
        const float seq[10] = {8.0f, 1.0f, 0.0f, NAN, INFINITY, 2.0f, 1e-30f, 500.0f, 1.0f, 1.0f};
        for (int t = 0; t < 10; ++t) {
            for (int j = 0; j < 3; ++j) cur[j] = seq[(t + 3 * j) % 10];
            orc_delayed_update(cur, hist, &head, 3, 4, t & 1, t % 3, fmt, sc, sci);
        }

        /* dense product, sampled entries (k above the 256 of one table), grouped */
        const int64_t m = 5, n = 7, k = 320;
        uint8_t* a = make_codes(m * k, fmt);
        uint8_t* b = make_codes(n * k, 3 - fmt);
        float sa[5] = {1, 2, 0.5f, 3, 0.25f}, sb[7] = {1, 1, 2, 2, 4, 4, 0.125f};
        double *ad = malloc(sizeof(double) * m * k), *bd = malloc(sizeof(double) * n * k);
        double y[35], bound[35];
        orc_gemm(a, fmt, k, b, 3 - fmt, k, m, n, k, sa, 1, sb, 1, ad, bd, y, n, bound);
        int64_t ii[6] = {0, 4, 2, 3, 1, 4}, jj[6] = {6, 0, 3, 5, 2, 6};
        double ye[6], be[6];
        orc_gemm_entries(a, fmt, k, b, 3 - fmt, k, k, sa, 1, sb, 1, ii, jj, 6, ye, be);
        for (int i = 0; i < 6; ++i)
            if (fabs(ye[i] - y[ii[i] * n + jj[i]]) > 1e-9 * (1.0 + fabs(ye[i]))) bad |= 4;
        const int64_t offsets[4] = {0, 2, 2, 5};    /* an empty group */
        float sbg[21];
        for (int i = 0; i < 21; ++i) sbg[i] = 0.5f + (float)i;
        orc_grouped_gemm_entries(a, fmt, k, b, 3 - fmt, k, 0, offsets, 3, n, k, sa, sbg, ii, jj, 6, ye, be);

        if (fmt < 2) {   /* MX: OCP formats, k % 32 == 0 */
            const int64_t mk = 64;
            uint16_t* xm = make_x(rows, mk);
            uint8_t* qm = malloc(rows * mk);
            uint8_t* sm = malloc(rows * (mk / 32));
            orc_mx_quantize_row(xm, rows, mk, mk, fmt, qm, mk, sm, mk / 32);
            (void)orc_mx_scale_value(orc_mx_scale(fmt, 3.0f));
            uint8_t* am2 = make_codes(m * mk, fmt);
            uint8_t* bm2 = make_codes(n * mk, fmt);
            uint8_t sam[10], sbm[14];
            for (int i = 0; i < 10; ++i) sam[i] = (uint8_t)(120 + i);
            for (int i = 0; i < 14; ++i) sbm[i] = (uint8_t)(130 - i);
            double *amd = malloc(sizeof(double) * m * mk), *bmd = malloc(sizeof(double) * n * mk);
            orc_mx_gemm(am2, fmt, mk, sam, 2, bm2, fmt, mk, sbm, 2, m, n, mk, amd, bmd, y, n, bound);
            free(xm); free(qm); free(sm); free(am2); free(bm2); free(amd); free(bmd);
        }
        free(x); free(qr); free(qt); free(si); free(am); free(a); free(b); free(ad); free(bd);
    }
    if (bad) fprintf(stderr, "oracle consistency checks failed: %d\n", bad);
    return bad ? 1 : 0;
}
