/*
 * Host sanitizer driver for the CPU oracle (test infrastructure).
 *
 * Built by tests/test_oracle_sanitizers.py together with
 * oracle/convrot_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer
 * (no recovery), without OpenMP.  It calls every exported oracle function on
 * small inputs, ragged where the function allows it, with zero rows, signed
 * zeros, infinities, NaNs and extreme magnitudes, so that any out-of-bounds
 * access, use of freed memory, signed overflow, bad shift or invalid
 * conversion in the oracle aborts the run.  A few cheap invariants are
 * checked as well; the numerical pins live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_set_threads(int n);
int orc_get_threads(void);
float orc_bf16_to_f32_one(uint16_t h);
uint16_t orc_f32_to_bf16_one(float f);
void orc_bf16_to_f32(const uint16_t* in, float* out, int64_t n);
void orc_f32_to_bf16(const float* in, uint16_t* out, int64_t n);
void orc_fwht256(float* v);
void orc_rotate_row(float* row, int64_t k);
void orc_rotate_rows(float* rows, int64_t nrows, int64_t k);
void orc_quantize_row(const float* v, int64_t k, int8_t* q, float* s_out);
void orc_quantize_rows(const float* v, int64_t nrows, int64_t k, int8_t* q, float* s);
int orc_quantize_weight(const float* w, int64_t n, int64_t k, int8_t* q, float* s);
int orc_rotate_quant_act_rows(const uint16_t* x, int64_t k, const int64_t* rows, int64_t nrows, int8_t* q,
                              float* s);
int orc_rotate_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* q, float* s);
void orc_gemm_s32(const int8_t* qx, int64_t nrows, const int8_t* qw, int64_t n, int64_t k, int32_t* acc);
float orc_dequant_one(int32_t acc, float s_x, float s_w);
void orc_dequant_bf16(const int32_t* acc, int64_t nrows, int64_t n, const float* s_x, const float* s_w,
                      uint16_t* y);
float orc_exp(float x);
float orc_silu(float g);
void orc_swiglu_bf16(const int32_t* acc, int64_t nrows, int64_t i_width, const float* s_x, const float* s_w,
                     uint16_t* y);
void orc_swiglu_ref(const int32_t* acc, int64_t nrows, int64_t i_width, const float* s_x, const float* s_w,
                    double* ref, double* mag);
void orc_swiglu_pairs_bf16(const uint16_t* gu, int64_t nrows, int64_t i_width, uint16_t* h);
int orc_swiglu_rotate_quant_rows(const uint16_t* gu, int64_t i_width, const int64_t* rows, int64_t nrows,
                                 int8_t* q, float* s);
void orc_dequantize_weight(const int8_t* q, const float* s, int64_t n, int64_t k, float* w);
void orc_lora_add(float* w, int64_t n, int64_t k, const float* b, const float* a, int64_t rank, float scale);
void orc_attention_rows(const int8_t* qc, const float* sq, int64_t nq, const int8_t* kc, const float* sk,
                        const double* v, int64_t s, int64_t d, double* out, double* absw);
void orc_mx_quantize_rows(const float* v, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales);
void orc_mx_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, double* out);
void orc_mx_gemm(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* bc, const uint8_t* bs,
                 int64_t n, int64_t k, double* y, double* absacc);

static int failures = 0;
#define CHECK(cond, what)                                          \
    do {                                                           \
        if (!(cond)) {                                             \
            fprintf(stderr, "invariant failed: %s\n", what);      \
            ++failures;                                            \
        }                                                          \
    } while (0)

/* xorshift64*: a small deterministic source of test values */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static float uniform(float lo, float hi) {
    return lo + (hi - lo) * (float)((next_u64() >> 40) * (1.0 / 16777216.0));
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

/* rows of fp32 values with the special cases the oracle must survive */
static void fill_rows(float* v, int64_t rows, int64_t k) {
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t i = 0; i < k; ++i) {
            float x;
            switch (r % 6) {
                case 0: x = 0.0f; break;                                   /* all-zero row */
                case 1: x = (i & 1) ? -0.0f : 0.0f; break;                 /* signed zeros */
                case 2: x = uniform(-3.0f, 3.0f) * 1e-40f; break;          /* denormals */
                case 3: x = uniform(-1.0f, 1.0f) * ((i % 97) ? 1.0f : 3e38f); break;   /* huge outliers */
                default: x = uniform(-4.0f, 4.0f); break;
            }
            v[r * k + i] = x;
        }
    }
}

static void test_bf16(void) {
    uint16_t h[4096];
    float f[4096];
    for (int i = 0; i < 4096; ++i) h[i] = (uint16_t)(i * 16 + (i >> 8));   /* spans every exponent, NaN, inf */
    orc_bf16_to_f32(h, f, 4096);
    uint16_t back[4096];
    orc_f32_to_bf16(f, back, 4096);
    for (int i = 0; i < 4096; ++i) {
        if (isnan(f[i])) continue;
        CHECK(back[i] == h[i], "bf16 -> fp32 -> bf16 round trip");
        CHECK(orc_f32_to_bf16_one(orc_bf16_to_f32_one(h[i])) == h[i], "one-value round trip");
    }
    const float specials[] = {NAN, -NAN, INFINITY, -INFINITY, 3.4028235e38f, -3.4028235e38f, 1e-45f, -0.0f};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i) (void)orc_f32_to_bf16_one(specials[i]);
}

static void test_rotate_and_quantize(void) {
    const int64_t ks[] = {256, 512, 768};
    for (size_t t = 0; t < 3; ++t) {
        const int64_t k = ks[t], rows = 7;
        float* v = xmalloc(sizeof(float) * rows * k);
        fill_rows(v, rows, k);
        float* w = xmalloc(sizeof(float) * rows * k);
        memcpy(w, v, sizeof(float) * rows * k);
        orc_rotate_rows(w, rows, k);
        orc_rotate_row(w, k);
        orc_fwht256(w + k);
        int8_t* q = xmalloc((size_t)(rows * k));
        float* s = xmalloc(sizeof(float) * rows);
        orc_quantize_rows(v, rows, k, q, s);
        for (int64_t i = 0; i < rows * k; ++i) CHECK(q[i] >= -127 && q[i] <= 127, "code range");
        orc_quantize_row(v, k, q, s);
        CHECK(orc_quantize_weight(v, rows, k, q, s) == 0, "quantize_weight status");
        CHECK(orc_quantize_weight(v, rows, k - 1, q, s) != 0, "quantize_weight rejects a ragged k");

        uint16_t* x = xmalloc(sizeof(uint16_t) * rows * k);
        orc_f32_to_bf16(v, x, rows * k);
        CHECK(orc_rotate_quant_act(x, rows, k, q, s) == 0, "rotate_quant_act status");
        const int64_t pick[] = {6, 0, 3};
        CHECK(orc_rotate_quant_act_rows(x, k, pick, 3, q, s) == 0, "row selection status");
        CHECK(orc_rotate_quant_act_rows(x, k + 1, pick, 3, q, s) != 0, "rotate_quant rejects a ragged k");
        CHECK(orc_rotate_quant_act(x, 0, k, q, s) == 0, "zero rows");
        free(v); free(w); free(q); free(s); free(x);
    }
}

static void test_gemm_and_epilogues(void) {
    const int64_t m = 5, n = 6, k = 512, iw = 3;
    int8_t* qx = xmalloc((size_t)(m * k));
    int8_t* qw = xmalloc((size_t)(n * k));
    for (int64_t i = 0; i < m * k; ++i) qx[i] = (int8_t)((i % 5 == 0) ? 127 : (int)(next_u64() % 255) - 127);
    for (int64_t i = 0; i < n * k; ++i) qw[i] = (int8_t)((i % 7 == 0) ? -127 : (int)(next_u64() % 255) - 127);
    int32_t* acc = xmalloc(sizeof(int32_t) * m * n);
    orc_gemm_s32(qx, m, qw, n, k, acc);
    for (int64_t j = 0; j < m; ++j)
        for (int64_t c = 0; c < n; ++c) {
            int64_t ref = 0;
            for (int64_t i = 0; i < k; ++i) ref += (int64_t)qx[j * k + i] * qw[c * k + i];
            CHECK(acc[j * n + c] == (int32_t)ref, "int32 contraction");
        }
    /* the int32 extreme at the largest k the contraction supports */
    {
        const int64_t kmax = 133120;
        int8_t* a = xmalloc((size_t)kmax);
        memset(a, 127, (size_t)kmax);
        int32_t e;
        orc_gemm_s32(a, 1, a, 1, kmax, &e);
        CHECK(e == (int32_t)(16129 * kmax), "int32 extreme");
        free(a);
    }
    float sx[5] = {1e-3f, 0.0f, 3e38f, 1e-40f, 0.5f};
    float sw[6] = {2e-3f, 1.0f, 0.0f, 3e38f, 1e-39f, -0.0f};
    uint16_t* y = xmalloc(sizeof(uint16_t) * m * n);
    orc_dequant_bf16(acc, m, n, sx, sw, y);
    (void)orc_dequant_one(2147483647, 3e38f, 3e38f);
    (void)orc_dequant_one(-2147483647 - 1, 1e-45f, -1e-45f);
    uint16_t* ys = xmalloc(sizeof(uint16_t) * m * iw);
    orc_swiglu_bf16(acc, m, iw, sx, sw, ys);
    double* ref = xmalloc(sizeof(double) * m * iw);
    double* mag = xmalloc(sizeof(double) * m * iw);
    orc_swiglu_ref(acc, m, iw, sx, sw, ref, mag);
    free(ref); free(mag);
    const float xs[] = {-1e30f, -200.0f, -88.0f, -86.0f, -1.0f, -0.0f, 0.0f, 1.0f, 80.0f, 88.72f, 89.0f,
                        1e30f, INFINITY, -INFINITY, NAN};
    for (size_t i = 0; i < sizeof xs / sizeof xs[0]; ++i) {
        (void)orc_exp(xs[i]);
        (void)orc_silu(xs[i]);
    }
    CHECK(orc_exp(0.0f) == 1.0f, "exp(0)");
    CHECK(orc_silu(0.0f) == 0.0f, "silu(0)");
    free(qx); free(qw); free(acc); free(y); free(ys);
}

static void test_swiglu_side_and_weights(void) {
    const int64_t rows = 4, iw = 512;
    float* g = xmalloc(sizeof(float) * rows * 2 * iw);
    fill_rows(g, rows, 2 * iw);
    uint16_t* gu = xmalloc(sizeof(uint16_t) * rows * 2 * iw);
    orc_f32_to_bf16(g, gu, rows * 2 * iw);
    uint16_t* h = xmalloc(sizeof(uint16_t) * rows * iw);
    orc_swiglu_pairs_bf16(gu, rows, iw, h);
    int8_t* q = xmalloc((size_t)(rows * iw));
    float* s = xmalloc(sizeof(float) * rows);
    const int64_t pick[] = {3, 1};
    CHECK(orc_swiglu_rotate_quant_rows(gu, iw, pick, 2, q, s) == 0, "output-side swiglu status");
    CHECK(orc_swiglu_rotate_quant_rows(gu, iw, NULL, rows, q, s) == 0, "output-side swiglu, all rows");
    CHECK(orc_swiglu_rotate_quant_rows(gu, iw - 128, NULL, rows, q, s) != 0, "rejects a ragged width");

    const int64_t n = 3, k = 512;
    int8_t* qw = xmalloc((size_t)(n * k));
    for (int64_t i = 0; i < n * k; ++i) qw[i] = (int8_t)((int)(next_u64() % 255) - 127);
    float sw[3] = {1e-3f, 0.0f, 3e38f};
    float* w = xmalloc(sizeof(float) * n * k);
    orc_dequantize_weight(qw, sw, n, k, w);
    const int64_t rank = 3;
    float* b = xmalloc(sizeof(float) * n * rank);
    float* a = xmalloc(sizeof(float) * rank * k);
    for (int64_t i = 0; i < n * rank; ++i) b[i] = uniform(-1.0f, 1.0f);
    for (int64_t i = 0; i < rank * k; ++i) a[i] = uniform(-1.0f, 1.0f);
    orc_lora_add(w, n, k, b, a, rank, 0.5f);
    orc_lora_add(w, n, k, b, a, 0, 1.0f);
    free(g); free(gu); free(h); free(q); free(s); free(qw); free(w); free(b); free(a);
}

static void test_attention(void) {
    const int64_t d = 128;
    const int64_t sizes[] = {0, 1, 5, 67};
    for (size_t t = 0; t < 4; ++t) {
        const int64_t s = sizes[t], nq = 3;
        int8_t* qc = xmalloc((size_t)(nq * d));
        int8_t* kc = xmalloc((size_t)((s ? s : 1) * d));
        float sq[3] = {1e-2f, 0.0f, 3.0f};
        float* sk = xmalloc(sizeof(float) * (s ? s : 1));
        double* v = xmalloc(sizeof(double) * (s ? s : 1) * d);
        for (int64_t i = 0; i < nq * d; ++i) qc[i] = (int8_t)((int)(next_u64() % 255) - 127);
        for (int64_t i = 0; i < s * d; ++i) kc[i] = (int8_t)((int)(next_u64() % 255) - 127);
        for (int64_t j = 0; j < s; ++j) sk[j] = j % 3 ? 1e-2f : 0.0f;
        for (int64_t i = 0; i < s * d; ++i) v[i] = uniform(-2.0f, 2.0f);
        double* out = xmalloc(sizeof(double) * nq * d);
        double* absw = xmalloc(sizeof(double) * nq * d);
        orc_attention_rows(qc, sq, nq, kc, sk, v, s, d, out, absw);
        if (s > 0)
            for (int64_t i = 0; i < nq * d; ++i) CHECK(fabs(out[i]) <= absw[i] * (1 + 1e-12), "|O| <= sum p|v|");
        free(qc); free(kc); free(sk); free(v); free(out); free(absw);
    }
}

static void test_mx(void) {
    const int64_t rows = 7, ks[] = {32, 128, 384};
    for (size_t t = 0; t < 3; ++t) {
        const int64_t k = ks[t];
        float* v = xmalloc(sizeof(float) * rows * k);
        fill_rows(v, rows, k);
        uint8_t* codes = xmalloc((size_t)(rows * k / 2));
        uint8_t* scales = xmalloc((size_t)(rows * k / 32));
        orc_mx_quantize_rows(v, rows, k, codes, scales);
        double* dec = xmalloc(sizeof(double) * rows * k);
        orc_mx_decode(codes, scales, rows, k, dec);
        for (int64_t i = 0; i < rows * k; ++i) CHECK(isfinite(dec[i]), "decoded values are finite");
        double* y = xmalloc(sizeof(double) * rows * rows);
        double* absacc = xmalloc(sizeof(double) * rows * rows);
        orc_mx_gemm(codes, scales, rows, codes, scales, rows, k, y, absacc);
        for (int64_t i = 0; i < rows * rows; ++i) CHECK(fabs(y[i]) <= absacc[i], "|y| <= sum |ab|");
        free(v); free(codes); free(scales); free(dec); free(y); free(absacc);
    }
}

int main(void) {
    orc_set_threads(1);
    CHECK(orc_get_threads() >= 1, "thread count");
    test_bf16();
    test_rotate_and_quantize();
    test_gemm_and_epilogues();
    test_swiglu_side_and_weights();
    test_attention();
    test_mx();
    if (failures) {
        fprintf(stderr, "%d invariant(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
