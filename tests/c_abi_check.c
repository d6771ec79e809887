/*
 * The C ABI used from C (test infrastructure): no Python, no torch.
 *
 * Built by tests/c_abi_build.py with gcc as C11 against include/convrot.h,
 * rotation_quantized_dit_amd/libconvrot.so, the HIP runtime and the CPU
 * oracle (oracle/convrot_oracle.c, linked in as plain C).  It drives the
 * ConvRot linear through its entry points on a HIP stream of its own, with
 * device memory from hipMalloc, and checks the results against the oracle:
 * weight and activation codes and scales, int32 accumulators and the bf16
 * dequant output bit for bit, the fused SwiGLU output within one bf16 ulp of
 * the oracle's exact value.  Then it checks that argument errors come back as
 * status codes, before anything is enqueued.  Exit status 0 when all hold.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "convrot.h"

/* the oracle (oracle/convrot_oracle.c) */
void orc_f32_to_bf16(const float* in, uint16_t* out, int64_t n);
int orc_quantize_weight(const float* w, int64_t n, int64_t k, int8_t* q, float* s);
int orc_rotate_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* q, float* s);
void orc_gemm_s32(const int8_t* qx, int64_t nrows, const int8_t* qw, int64_t n, int64_t k, int32_t* acc);
void orc_dequant_bf16(const int32_t* acc, int64_t nrows, int64_t n, const float* s_x, const float* s_w,
                      uint16_t* y);
void orc_swiglu_ref(const int32_t* acc, int64_t nrows, int64_t i_width, const float* s_x, const float* s_w,
                    double* ref, double* mag);

#define HIP_CHECK(call)                                                                 \
    do {                                                                                \
        hipError_t e_ = (call);                                                         \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));           \
            exit(2);                                                                    \
        }                                                                               \
    } while (0)

static int failures = 0;
static void expect(int cond, const char* what) {
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}
static void expect_status(int got, int want, const char* what) {
    if (got != want) {
        fprintf(stderr, "FAILED: %s: status %d (%s), expected %d\n", what, got, convrot_status_string(got), want);
        ++failures;
    }
}

/* xorshift64* and a Box-Muller normal: the test's own seeded inputs */
static uint64_t rng = 0x2545F4914F6CDD1Dull;
static double unif(void) {
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return ((rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normal(void) {
    const double u = unif() + 1e-300, v = unif();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}

static void* host(size_t n) {
    void* p = calloc(n ? n : 1, 1);
    if (!p) exit(2);
    return p;
}
static void* dev(size_t n) {
    void* p = NULL;
    HIP_CHECK(hipMalloc(&p, n ? n : 16));
    return p;
}

static double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int main(void) {
    /* 67 tokens (a ragged tile), k = 768 (three Hadamard groups), 96 weight rows
     * (48 gate + 48 up for the fused SwiGLU) */
    const int64_t m = 67, k = 768, n = 96, i = n / 2;
    float* x32 = host(sizeof(float) * m * k);
    float* w = host(sizeof(float) * n * k);
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < k; ++c) x32[r * k + c] = normal() * ((c % 101 == 7) ? 50.0f : 1.0f);
    for (int64_t e = 0; e < n * k; ++e) w[e] = 0.02f * normal();
    uint16_t* x = host(sizeof(uint16_t) * m * k);
    orc_f32_to_bf16(x32, x, m * k);

    hipStream_t st;
    HIP_CHECK(hipStreamCreate(&st));
    uint16_t* dx = dev(sizeof(uint16_t) * m * k);
    float* dw = dev(sizeof(float) * n * k);
    int8_t* dqw = dev((size_t)(n * k));
    float* dsw = dev(sizeof(float) * n);
    int8_t* dqx = dev((size_t)(m * k));
    float* dsx = dev(sizeof(float) * m);
    int32_t* dacc = dev(sizeof(int32_t) * m * n);
    uint16_t* dy = dev(sizeof(uint16_t) * m * n);
    uint16_t* dysw = dev(sizeof(uint16_t) * m * i);
    const size_t ws_bytes = convrot_workspace_bytes(m, k);
    expect(ws_bytes == (size_t)(m * k + 4 * m), "convrot_workspace_bytes = m k + 4 m");
    void* ws = dev(ws_bytes);
    HIP_CHECK(hipMemcpyAsync(dx, x, sizeof(uint16_t) * m * k, hipMemcpyHostToDevice, st));
    HIP_CHECK(hipMemcpyAsync(dw, w, sizeof(float) * n * k, hipMemcpyHostToDevice, st));

    expect_status(convrot_quantize_weight(dw, n, k, dqw, dsw, st), CONVROT_OK, "convrot_quantize_weight");
    expect_status(convrot_rotate_quant_act(dx, m, k, dqx, dsx, st), CONVROT_OK, "convrot_rotate_quant_act");
    expect_status(convrot_gemm_s32(dqx, dqw, m, n, k, dacc, st), CONVROT_OK, "convrot_gemm_s32");
    expect_status(convrot_linear(dx, m, k, dqw, dsw, n, dy, ws, ws_bytes, st), CONVROT_OK, "convrot_linear");
    expect_status(convrot_linear_swiglu(dx, m, k, dqw, dsw, i, dysw, ws, ws_bytes, st), CONVROT_OK,
                  "convrot_linear_swiglu");

    int8_t* gqw = host((size_t)(n * k));
    float* gsw = host(sizeof(float) * n);
    int8_t* gqx = host((size_t)(m * k));
    float* gsx = host(sizeof(float) * m);
    int32_t* gacc = host(sizeof(int32_t) * m * n);
    uint16_t* gy = host(sizeof(uint16_t) * m * n);
    uint16_t* gysw = host(sizeof(uint16_t) * m * i);
    HIP_CHECK(hipMemcpyAsync(gqw, dqw, (size_t)(n * k), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(gsw, dsw, sizeof(float) * n, hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(gqx, dqx, (size_t)(m * k), hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(gsx, dsx, sizeof(float) * m, hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(gacc, dacc, sizeof(int32_t) * m * n, hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(gy, dy, sizeof(uint16_t) * m * n, hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipMemcpyAsync(gysw, dysw, sizeof(uint16_t) * m * i, hipMemcpyDeviceToHost, st));
    HIP_CHECK(hipStreamSynchronize(st));

    int8_t* oqw = host((size_t)(n * k));
    float* osw = host(sizeof(float) * n);
    int8_t* oqx = host((size_t)(m * k));
    float* osx = host(sizeof(float) * m);
    int32_t* oacc = host(sizeof(int32_t) * m * n);
    uint16_t* oy = host(sizeof(uint16_t) * m * n);
    double* ref = host(sizeof(double) * m * i);
    double* mag = host(sizeof(double) * m * i);
    expect(orc_quantize_weight(w, n, k, oqw, osw) == 0, "oracle quantize_weight");
    expect(orc_rotate_quant_act(x, m, k, oqx, osx) == 0, "oracle rotate_quant_act");
    orc_gemm_s32(oqx, m, oqw, n, k, oacc);
    orc_dequant_bf16(oacc, m, n, osx, osw, oy);
    orc_swiglu_ref(oacc, m, i, osx, osw, ref, mag);

    expect(memcmp(gqw, oqw, (size_t)(n * k)) == 0, "weight codes bit-exact");
    expect(memcmp(gsw, osw, sizeof(float) * n) == 0, "weight scales bit-exact");
    expect(memcmp(gqx, oqx, (size_t)(m * k)) == 0, "activation codes bit-exact");
    expect(memcmp(gsx, osx, sizeof(float) * m) == 0, "activation scales bit-exact");
    expect(memcmp(gacc, oacc, sizeof(int32_t) * m * n) == 0, "int32 accumulators exact");
    expect(memcmp(gy, oy, sizeof(uint16_t) * m * n) == 0, "bf16 dequant output bit-exact");
    int64_t outside = 0;
    for (int64_t e = 0; e < m * i; ++e) {
        const double err = fabs(bf16_value(gysw[e]) - ref[e]);
        if (!(err <= ldexp(fabs(ref[e]), -8) + ldexp(1.0 + mag[e], -120))) ++outside;
    }
    expect(outside == 0, "fused SwiGLU output within one bf16 ulp of the exact value");

    /* argument errors: a status, and nothing enqueued */
    expect_status(convrot_linear(dx, m, 300, dqw, dsw, n, dy, ws, ws_bytes, st), CONVROT_ERR_SHAPE,
                  "k not a multiple of 256");
    expect_status(convrot_linear(dx, m, CONVROT_MAX_K + 256, dqw, dsw, n, dy, ws, ws_bytes, st),
                  CONVROT_ERR_SHAPE, "k above the int32 bound");
    expect_status(convrot_linear(dx, -1, k, dqw, dsw, n, dy, ws, ws_bytes, st), CONVROT_ERR_SHAPE,
                  "negative m");
    expect_status(convrot_linear(NULL, m, k, dqw, dsw, n, dy, ws, ws_bytes, st), CONVROT_ERR_NULL, "NULL x");
    expect_status(convrot_linear((const uint16_t*)((const char*)dx + 2), m, k, dqw, dsw, n, dy, ws, ws_bytes, st),
                  CONVROT_ERR_ALIGN, "x not 16-byte aligned");
    expect_status(convrot_linear(dx, m, k, dqw, dsw, n, dy, ws, ws_bytes - 1, st), CONVROT_ERR_WORKSPACE,
                  "workspace one byte short");
    expect_status(convrot_linear(dx, 0, k, NULL, NULL, n, NULL, NULL, 0, st), CONVROT_OK, "m = 0 is a no-op");
    expect_status(convrot_linear_swiglu(dx, m, k, dqw, dsw, -2, dysw, ws, ws_bytes, st), CONVROT_ERR_SHAPE,
                  "negative i");
    for (int s = CONVROT_OK; s <= CONVROT_ERR_LAUNCH; ++s)
        expect(convrot_status_string(s) != NULL && strcmp(convrot_status_string(s), "unknown status") != 0,
               "every status has a string");
    expect(strcmp(convrot_status_string(99), "unknown status") == 0, "unknown status string");
    HIP_CHECK(hipStreamSynchronize(st));
    HIP_CHECK(hipGetLastError());

    HIP_CHECK(hipStreamDestroy(st));
    hipFree(dx); hipFree(dw); hipFree(dqw); hipFree(dsw); hipFree(dqx); hipFree(dsx);
    hipFree(dacc); hipFree(dy); hipFree(dysw); hipFree(ws);
    free(x32); free(w); free(x); free(gqw); free(gsw); free(gqx); free(gsx); free(gacc); free(gy);
    free(gysw); free(oqw); free(osw); free(oqx); free(osx); free(oacc); free(oy); free(ref); free(mag);
    if (failures) {
        fprintf(stderr, "c abi check: %d failure(s)\n", failures);
        return 1;
    }
    printf("c abi check: ok (%lld x %lld x %lld linear and SwiGLU through the C ABI on a HIP stream)\n",
           (long long)m, (long long)k, (long long)n);
    return 0;
}
