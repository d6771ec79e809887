/*
 * CPU oracle for the ConvRot int8 quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  It is used by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark, and by nothing else.  It shares no source
 * with the HIP path: the two meet only at the seeded input generator.
 *
 * It is deliberately plain: scalar loops, one IEEE fp32 operation per C
 * operator (build with -O2 -ffp-contract=off -fno-fast-math on x86-64, where
 * float arithmetic is SSE and has no excess precision), the textbook stage
 * order for the Walsh-Hadamard butterfly, and an int32 triple loop for the
 * contraction.  The only parallelism is an OpenMP loop over independent rows
 * (each row's arithmetic is identical whatever the thread count).
 *
 * Sources of what is computed (the pages):
 *   - cloud-worker docs/RESEARCH.md, "Weight families": the int8_convrot
 *     weight family; what this file computes for it is a block-diagonal
 *     orthonormal Hadamard-256 transform along K, applied before per-row
 *     symmetric int8 quantization of both operands.
 *   - h3-rs README, model file table: the DiT weights are "int8 per-row +
 *     ConvRot (Hadamard-256)", i.e. one scale per output row, Hadamard groups of
 *     256 along the contraction dimension.
 *   - h3-rs README, "Speed": the fused int8 GEMM quantizes activations per row
 *     (one scale per token), the Hadamard rotation runs inside that quantizer,
 *     the GEMM writes bf16 directly, and fc1's gate/up rows are paired so that
 *     SwiGLU is applied in the GEMM epilogue.
 *   - h3-rs README, "Speed": the DiT's attention multiplies int8 Q by int8 K^T
 *     and fp16 P by fp16 V (see orc_attention_rows for the readings).
 * Every step the pages leave open is a stated reading (see the comment at each
 * function): Sylvester ordering, orthonormal scaling 1/16, contiguous groups,
 * symmetric absmax/127 scales, round-half-even, (acc*s_x)*s_w dequant order,
 * gate rows first in the fused fc1 weight, and one fixed fp32 exponential.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GROUP 256

/* ---------------------------------------------------------------- threads */

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------ bf16 <-> f32 */

/* bf16 -> fp32 widening: the 16 bf16 bits are the upper half of the fp32
 * pattern, so this is exact. */
float orc_bf16_to_f32_one(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest with ties to even on the 16 discarded bits.
 * NaN stays NaN (forced quiet); infinities and overflow to infinity follow
 * from the same rounding. */
uint16_t orc_f32_to_bf16_one(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

void orc_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32_one(in[i]);
}

void orc_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16_one(in[i]);
}

/* --------------------------------------------------------------- rotation */

/* 256-point fast Walsh-Hadamard transform, in place, in fp32, followed by the
 * orthonormal scaling 1/16 (exact: a power of two).
 *
 * Reading of "Hadamard-256" (h3-rs README, model file table): the Sylvester
 * matrix H[i][j] = (-1)^popcount(i & j), which is what the in-place butterfly
 * computes; scaled by 1/16 so that H/16 is orthogonal and involutive (the
 * "rotation" of RESEARCH.md, "Weight families").  Stage order is fixed as the
 * textbook one, span h = 1, 2, 4, ..., 128; at every stage the pair (a, b) at
 * (i, i+h) with bit h of i clear becomes (a + b, a - b).  Each sum is one RNE
 * fp32 operation, so the result is a fixed function of the input bits. */
void orc_fwht256(float* v) {
    for (int h = 1; h < ORC_GROUP; h <<= 1) {
        for (int i = 0; i < ORC_GROUP; ++i) {
            if (i & h) continue;
            float a = v[i];
            float b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    for (int i = 0; i < ORC_GROUP; ++i) v[i] = v[i] * 0.0625f;
}

/* Group-wise rotation of one row of length k (k a multiple of 256): the
 * convolution with kernel = stride = 256 of RESEARCH.md, "Weight families",
 * i.e. the block-diagonal product row * blockdiag(H/16).  Groups are the
 * contiguous, non-overlapping 256-element blocks of the row. */
void orc_rotate_row(float* row, int64_t k) {
    for (int64_t g = 0; g + ORC_GROUP <= k; g += ORC_GROUP) orc_fwht256(row + g);
}

void orc_rotate_rows(float* rows, int64_t nrows, int64_t k) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) orc_rotate_row(rows + r * k, k);
}

/* ------------------------------------------------------------ quantizer */

/* Symmetric per-row int8 quantization of one (already rotated) fp32 row.
 *
 * One scale for the whole row ("per row" in h3-rs README, "Speed" for tokens,
 * and "int8 per-row" in its model file table for weights).  Reading: no zero
 * point, s = max_k |v_k| / 127 (one correctly rounded fp32 division), code =
 * rint(v_k / s) (correctly rounded division, then round half to even),
 * clamped to [-127, 127].  An all-zero row gets s = 0 and all-zero codes. */
void orc_quantize_row(const float* v, int64_t k, int8_t* q, float* s_out) {
    float amax = 0.0f;
    for (int64_t i = 0; i < k; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float s = amax / 127.0f;
    *s_out = s;
    if (s == 0.0f) {
        for (int64_t i = 0; i < k; ++i) q[i] = 0;
        return;
    }
    for (int64_t i = 0; i < k; ++i) {
        float t = rintf(v[i] / s);
        if (t > 127.0f) t = 127.0f;
        if (t < -127.0f) t = -127.0f;
        q[i] = (int8_t)(int)t;
    }
}

/* Quantize rows that are already in the wanted basis (no rotation).  The
 * unrotated per-token int8 baseline is this function applied to raw rows. */
void orc_quantize_rows(const float* v, int64_t nrows, int64_t k, int8_t* q, float* s) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < nrows; ++r) orc_quantize_row(v + r * k, k, q + r * k, s + r);
}

/* Load-time weight preparation: rotate every row of the fp32 weight [n, k]
 * along k, then per-row int8 (h3-rs README: weights are "int8 per-row +
 * ConvRot (Hadamard-256)" and stay quantized in memory).  Returns 0, or -1
 * when k is not a positive multiple of 256 or memory runs out. */
int orc_quantize_weight(const float* w, int64_t n, int64_t k, int8_t* q, float* s) {
    if (k <= 0 || k % ORC_GROUP) return -1;
    int fail = 0;
    int64_t r;
#pragma omp parallel for schedule(static) reduction(| : fail)
    for (r = 0; r < n; ++r) {
        float* row = (float*)malloc((size_t)k * sizeof(float));
        if (!row) { fail |= 1; continue; }
        memcpy(row, w + r * k, (size_t)k * sizeof(float));
        orc_rotate_row(row, k);
        orc_quantize_row(row, k, q + r * k, s + r);
        free(row);
    }
    return fail ? -1 : 0;
}

/* Per-token activation preparation: widen bf16 to fp32 (exact), rotate along
 * k, quantize with one scale per token (h3-rs README, "Speed").  The optional
 * row list selects which rows of x to process (NULL: rows 0..m-1); output row
 * j belongs to input row rows[j]. */
int orc_rotate_quant_act_rows(const uint16_t* x, int64_t k, const int64_t* rows, int64_t nrows,
                              int8_t* q, float* s) {
    if (k <= 0 || k % ORC_GROUP) return -1;
    int fail = 0;
    int64_t j;
#pragma omp parallel for schedule(static) reduction(| : fail)
    for (j = 0; j < nrows; ++j) {
        int64_t r = rows ? rows[j] : j;
        float* row = (float*)malloc((size_t)k * sizeof(float));
        if (!row) { fail |= 1; continue; }
        orc_bf16_to_f32(x + r * k, row, k);
        orc_rotate_row(row, k);
        orc_quantize_row(row, k, q + j * k, s + j);
        free(row);
    }
    return fail ? -1 : 0;
}

int orc_rotate_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* q, float* s) {
    return orc_rotate_quant_act_rows(x, k, NULL, m, q, s);
}

/* ---------------------------------------------------------- contraction */

/* acc[j][c] = sum_k qx[j][k] * qw[c][k] in int32 (the int8 GEMM of h3-rs
 * README, "Speed").  Codes are in [-127, 127], so |acc| <= 16129 * k and the
 * sum cannot overflow for k <= 133120.  qx holds nrows rows of length k
 * (already selected), qw holds n rows of length k. */
void orc_gemm_s32(const int8_t* qx, int64_t nrows, const int8_t* qw, int64_t n, int64_t k,
                  int32_t* acc) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < nrows; ++j) {
        const int8_t* a = qx + j * k;
        for (int64_t c = 0; c < n; ++c) {
            const int8_t* b = qw + c * k;
            int32_t sum = 0;
            for (int64_t i = 0; i < k; ++i) sum += (int32_t)a[i] * (int32_t)b[i];
            acc[j * n + c] = sum;
        }
    }
}

/* ---------------------------------------------------------- epilogues */

/* Dual-scale dequantization straight to bf16 (h3-rs README, "Speed": the GEMM
 * "writes bf16 directly").  Reading of the operation order: convert the int32
 * accumulator to fp32 (RNE), multiply by the token's scale, then by the
 * weight row's scale (two RNE multiplies), then round to bf16. */
float orc_dequant_one(int32_t acc, float s_x, float s_w) {
    float f = (float)acc;
    f = f * s_x;
    f = f * s_w;
    return f;
}

void orc_dequant_bf16(const int32_t* acc, int64_t nrows, int64_t n, const float* s_x,
                      const float* s_w, uint16_t* y) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < nrows; ++j)
        for (int64_t c = 0; c < n; ++c)
            y[j * n + c] = orc_f32_to_bf16_one(orc_dequant_one(acc[j * n + c], s_x[j], s_w[c]));
}

/* Fixed fp32 exponential used by silu.
 *
 * The pages do not say how the SwiGLU epilogue evaluates exp; the layer's
 * definition here fixes one algorithm so that the fused epilogue is
 * reproducible bit for bit:
 *   Cody and Waite argument reduction (W. J. Cody, W. Waite, "Software Manual
 *   for the Elementary Functions", 1980): k = rint(x * log2(e)),
 *   r = x - k*ln2 with ln2 split into a 15-bit head (so k*head is exact) and
 *   an fp32 tail, each subtraction one fused multiply-add;
 *   then the degree-7 Taylor polynomial of e^r (coefficients RN_fp32(1/n!))
 *   in Horner form with fused multiply-adds, and finally the exact scaling
 *   by 2^k.
 * Constants (derived from the mathematics, all RN to fp32):
 *   log2(e) = 0x1.715476p+0; ln2 head = floor(ln2 * 2^16) / 2^16 = 0x1.62e4p-1;
 *   ln2 tail = RN(ln2 - head) = 0x1.7f7d1cp-20.
 * Range: x > 88.72 gives +inf (e^x overflows fp32); x < -86 gives 0 (below
 * 4.5e-38; silu only ever adds it to 1, where it vanishes).  Accuracy is a
 * few ulp against the exact exponential (pinned by the tests). */
float orc_exp(float x) {
    if (x > 88.72f) return INFINITY;
    if (x < -86.0f) return 0.0f;
    const float log2e = 0x1.715476p+0f;
    const float ln2_hi = 0x1.62e4p-1f;
    const float ln2_lo = 0x1.7f7d1cp-20f;
    float kf = rintf(x * log2e);
    float r = fmaf(-kf, ln2_hi, x);
    r = fmaf(-kf, ln2_lo, r);
    float p = 0x1.a01a02p-13f;             /* 1/7! */
    p = fmaf(p, r, 0x1.6c16c2p-10f);       /* 1/6! */
    p = fmaf(p, r, 0x1.111112p-7f);        /* 1/5! */
    p = fmaf(p, r, 0x1.555556p-5f);        /* 1/4! */
    p = fmaf(p, r, 0x1.555556p-3f);        /* 1/3! */
    p = fmaf(p, r, 0.5f);                  /* 1/2! */
    p = fmaf(p, r, 1.0f);                  /* 1/1! */
    p = fmaf(p, r, 1.0f);                  /* 1/0! */
    return ldexpf(p, (int)kf);
}

/* silu(g) = g / (1 + e^(-g)), one correctly rounded fp32 division. */
float orc_silu(float g) {
    return g / (1.0f + orc_exp(-g));
}

/* SwiGLU epilogue of the fused fc1 GEMM (h3-rs README, "Speed": gate/up rows
 * are paired so SwiGLU fuses into the epilogue).  Reading: the fc1 weight is
 * one [2i, k] matrix whose rows [0, i) are the gate and rows [i, 2i) the up
 * projection.  g and u are dequantized to fp32 as in orc_dequant_one and are
 * not rounded to bf16 before y = bf16(silu(g) * u).
 * acc has 2i columns per row; s_w has 2i entries. */
void orc_swiglu_bf16(const int32_t* acc, int64_t nrows, int64_t i_width, const float* s_x,
                     const float* s_w, uint16_t* y) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < nrows; ++j) {
        for (int64_t c = 0; c < i_width; ++c) {
            float g = orc_dequant_one(acc[j * 2 * i_width + c], s_x[j], s_w[c]);
            float u = orc_dequant_one(acc[j * 2 * i_width + i_width + c], s_x[j], s_w[i_width + c]);
            y[j * i_width + c] = orc_f32_to_bf16_one(orc_silu(g) * u);
        }
    }
}

/* The exact value the fused fc1 epilogue approximates (h3-rs README,
 * "Speed": SwiGLU fused into the GEMM epilogue; the layer's contract checks
 * its bf16 output against the exact result within a relative bound, and
 * requires bit equality only of codes, scales and integer accumulators).
 * g and u are the fp32 dequantized gate and up values exactly as in
 * orc_dequant_one (that step is part of the definition); then, in fp64 with
 * libm's exp, ref = g / (1 + e^(-g)) * u, with no rounding to bf16.  mag
 * receives |g * u|, the scale of an absolute floor where the quotient leaves
 * the fp32 normal range.  acc has 2i columns per row; s_w has 2i entries. */
void orc_swiglu_ref(const int32_t* acc, int64_t nrows, int64_t i_width, const float* s_x, const float* s_w,
                    double* ref, double* mag) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < nrows; ++j) {
        for (int64_t c = 0; c < i_width; ++c) {
            const double g = (double)orc_dequant_one(acc[j * 2 * i_width + c], s_x[j], s_w[c]);
            const double u =
                (double)orc_dequant_one(acc[j * 2 * i_width + i_width + c], s_x[j], s_w[i_width + c]);
            ref[j * i_width + c] = g / (1.0 + exp(-g)) * u;
            mag[j * i_width + c] = fabs(g * u);
        }
    }
}

/* --------------------------------------------- SwiGLU on fc1's output side */

/* SwiGLU placed on the output side of fc1 (hybrid model card, "Native NVFP4
 * projection benchmarks": an "FFN output + SwiGLU" projection, i.e. SwiGLU
 * applied to fc1's written output rather than inside its epilogue).  Reading:
 * fc1 writes its dequantized gate and up columns as bf16 in one [rows, 2i]
 * array, gate columns [0, i) and up columns [i, 2i); each is widened exactly
 * and h = bf16(silu(g) * u), silu as in orc_silu. */
static void swiglu_pairs_row(const uint16_t* gu, int64_t i_width, uint16_t* h) {
    for (int64_t c = 0; c < i_width; ++c) {
        float g = orc_bf16_to_f32_one(gu[c]);
        float u = orc_bf16_to_f32_one(gu[i_width + c]);
        h[c] = orc_f32_to_bf16_one(orc_silu(g) * u);
    }
}

void orc_swiglu_pairs_bf16(const uint16_t* gu, int64_t nrows, int64_t i_width, uint16_t* h) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < nrows; ++j) swiglu_pairs_row(gu + j * 2 * i_width, i_width, h + j * i_width);
}

/* The down projection's activation preparation with SwiGLU moved in front
 * of it: h of each selected row as in orc_swiglu_pairs_bf16, then the same
 * widening, rotation and per-token quantization as orc_rotate_quant_act_rows
 * (so the codes equal those of rotating and quantizing the bf16 SwiGLU
 * output).  Output row j belongs to input row rows[j] (rows NULL: 0..n-1). */
int orc_swiglu_rotate_quant_rows(const uint16_t* gu, int64_t i_width, const int64_t* rows,
                                 int64_t nrows, int8_t* q, float* s) {
    if (i_width <= 0 || i_width % ORC_GROUP) return -1;
    int fail = 0;
    int64_t j;
#pragma omp parallel for schedule(static) reduction(| : fail)
    for (j = 0; j < nrows; ++j) {
        int64_t r = rows ? rows[j] : j;
        uint16_t* h = (uint16_t*)malloc((size_t)i_width * sizeof(uint16_t));
        float* row = (float*)malloc((size_t)i_width * sizeof(float));
        if (!h || !row) { free(h); free(row); fail |= 1; continue; }
        swiglu_pairs_row(gu + r * 2 * i_width, i_width, h);
        orc_bf16_to_f32(h, row, i_width);
        orc_rotate_row(row, i_width);
        orc_quantize_row(row, i_width, q + j * i_width, s + j);
        free(h);
        free(row);
    }
    return fail ? -1 : 0;
}

/* ----------------------------------------- weight dequantize / LoRA merge */

/* Dequantize ConvRot weights back to the unrotated basis (h3-rs README, model
 * file table: quantized weights are dequantized per layer by kernels; "Speed":
 * LoRAs are merged at load by dequantizing, adding and requantizing).
 * Reading: W = (q . s) . H/16 per row; since H/16 is its own inverse this
 * undoes the rotation.  The codes are rotated first: with |q| <= 127 every
 * butterfly partial sum is an integer below 2^15, so orc_fwht256 (butterfly
 * then the exact 1/16) is exact, and the only rounding is the one multiply
 * w = RN((H q / 16) * s). */
void orc_dequantize_weight(const int8_t* q, const float* s, int64_t n, int64_t k, float* w) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        float* row = w + r * k;
        for (int64_t c = 0; c < k; ++c) row[c] = (float)q[r * k + c];
        orc_rotate_row(row, k);
        for (int64_t c = 0; c < k; ++c) row[c] = row[c] * s[r];
    }
}

/* Low-rank delta added in place: W[n][c] += scale * sum_j B[n][j] * A[j][c]
 * (h3-rs README: ComfyUI LoRA files, merged at load; B is the up factor
 * [n, rank], A the down factor [rank, k], scale the caller's strength times
 * alpha / rank).  Reading of the fp32 arithmetic: the sum runs over j in
 * increasing order as a chain of fused multiply-adds starting from 0, then
 * one multiply by scale and one add to W. */
void orc_lora_add(float* w, int64_t n, int64_t k, const float* b, const float* a, int64_t rank,
                  float scale) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            float acc = 0.0f;
            for (int64_t j = 0; j < rank; ++j) acc = fmaf(b[r * rank + j], a[j * k + c], acc);
            w[r * k + c] = w[r * k + c] + scale * acc;
        }
    }
}

/* ---------------------------------------------------- int8 Q.K^T / fp16 P.V
 *
 * The DiT's attention as h3-rs runs it (h3-rs README, "Speed": the logits come
 * from an int8 Q.K^T, the value product is an fp16 P.V), over the full
 * sequence with no mask (hybrid model card, "Notes and limitations": the
 * evaluated implementation uses full attention).
 *
 * Readings (the pages give only the operand types):
 *   - Q and K are quantized per token and per head: each head's d values of a
 *     token form one row for the per-row quantizer above, without rotation
 *     (the pages name no rotation for attention).
 *   - logit_ij = acc_ij * s_q[i] * s_k[j] / sqrt(d), acc_ij the exact integer
 *     dot product of the codes; softmax over all keys j.
 *   - V enters as fp16 values (the caller converts), the output is
 *     O_i = sum_j p_ij v_j / sum_j p_ij with p_ij = exp(logit_ij - max_j).
 * Everything after the integer dot product is evaluated in fp64, so this is
 * the definition itself; the kernel's fp32 logits, fp16 probabilities and
 * fp32 sums differ from it by rounding only.  absw receives
 * sum_j p_ij |v_jc| / sum_j p_ij, the scale of that rounding per output. */
void orc_attention_rows(const int8_t* qc, const float* sq, int64_t nq, const int8_t* kc,
                        const float* sk, const double* v, int64_t s, int64_t d, double* out,
                        double* absw) {
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    int64_t i;
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nq; ++i) {
        double* logit = (double*)malloc((size_t)(s > 0 ? s : 1) * sizeof(double));
        double mx = -INFINITY;
        for (int64_t j = 0; j < s; ++j) {
            int32_t acc = 0;
            for (int64_t c = 0; c < d; ++c) acc += (int32_t)qc[i * d + c] * (int32_t)kc[j * d + c];
            logit[j] = (double)acc * (double)sq[i] * (double)sk[j] * inv_sqrt_d;
            if (logit[j] > mx) mx = logit[j];
        }
        double z = 0.0;
        for (int64_t c = 0; c < d; ++c) {
            out[i * d + c] = 0.0;
            absw[i * d + c] = 0.0;
        }
        for (int64_t j = 0; j < s; ++j) {
            const double p = exp(logit[j] - mx);
            z += p;
            for (int64_t c = 0; c < d; ++c) {
                out[i * d + c] += p * v[j * d + c];
                absw[i * d + c] += p * fabs(v[j * d + c]);
            }
        }
        for (int64_t c = 0; c < d; ++c) {
            out[i * d + c] /= z;
            absw[i * d + c] /= z;
        }
        free(logit);
    }
}

/* ------------------------------------------------------- MXFP4 (NEXT row)
 *
 * The hybrid checkpoints of the Minimax_h3_hybrid model card ("Checkpoints")
 * run the QKV and FFN-input projections in a 4-bit block format (NVFP4) and
 * keep the output projections int8 ConvRot.  NVFP4 is a Blackwell format;
 * its analog on this hardware is the OCP Microscaling format MXFP4, which the
 * MI355X matrix cores take natively.  The readings (from the OCP MX format
 * definition, as this build reads it):
 *   - blocks of 32 consecutive elements along K share one scale 2^e stored as
 *     an 8-bit biased exponent (E8M0, code = e + 127);
 *   - e = floor(log2(max |v|)) - 2 (2 is the largest exponent of the element
 *     format), clamped to [-127, 127]; an all-zero block takes code 0;
 *   - each element is v / 2^e (exact: a power-of-two scaling) rounded to
 *     FP4 E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), to nearest, ties to
 *     the even mantissa bit, magnitudes above 6 saturated to 6; the sign bit
 *     is the sign of v (so -0 and small negatives that round to zero keep it);
 *   - element 2j of a row is the low nibble of byte j, element 2j + 1 the high
 *     nibble; no rotation (the hybrid's NVFP4 layers carry none). */

/* E2M1 magnitude of a 3-bit code (exponent bits 2..1, mantissa bit 0). */
static double e2m1_mag(int c) {
    const int e = (c >> 1) & 3, m = c & 1;
    return e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
}

/* Nearest E2M1 magnitude code of y >= 0: the candidates are taken in order;
 * at an exact midpoint the code with mantissa bit 0 wins; above 6 saturates. */
static int e2m1_round(double y) {
    if (y >= 6.0) return 7;
    int best = 0;
    double bd = y;                      /* distance to code 0 (magnitude 0) */
    for (int c = 1; c < 8; ++c) {
        const double d = fabs(y - e2m1_mag(c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    return best;
}

void orc_mx_quantize_rows(const float* v, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < k / 32; ++b) {
            const float* x = v + r * k + 32 * b;
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i)
                if (fabsf(x[i]) > amax) amax = fabsf(x[i]);
            int e = -127;
            if (amax > 0.0f) {
                int fe;
                frexpf(amax, &fe);     /* amax = f 2^fe, f in [0.5, 1): floor(log2) = fe - 1 */
                e = fe - 1 - 2;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            scales[r * (k / 32) + b] = (uint8_t)(e + 127);
            for (int i = 0; i < 32; ++i) {
                const double y = ldexp((double)x[i], -e);
                const int c = (signbit(x[i]) ? 8 : 0) | (amax > 0.0f ? e2m1_round(fabs(y)) : 0);
                uint8_t* byte = codes + r * (k / 2) + 16 * b + i / 2;
                if (i % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xf0) | c);
                else
                    *byte = (uint8_t)((*byte & 0x0f) | (c << 4));
            }
        }
    }
}

/* Value of element i of a quantized row. */
static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t i) {
    const int c = (i % 2 == 0) ? (codes[i / 2] & 15) : (codes[i / 2] >> 4);
    const double m = e2m1_mag(c & 7);
    return ldexp((c & 8) ? -m : m, (int)scales[i / 32] - 127);
}

void orc_mx_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, double* out) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r)
        for (int64_t i = 0; i < k; ++i)
            out[r * k + i] = mx_value(codes + r * (k / 2), scales + r * (k / 32), i);
}

/* y[m][n] = sum_k a[m][k] b[n][k] over the decoded values, in fp64 (exact for
 * these operands: every product is a short binary fraction); absacc receives
 * sum_k |a b| (the scale of the fp32 accumulation error of a kernel). */
void orc_mx_gemm(const uint8_t* ac, const uint8_t* as, int64_t m, const uint8_t* bc, const uint8_t* bs,
                 int64_t n, int64_t k, double* y, double* absacc) {
    int64_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < m; ++r) {
        double* arow = (double*)malloc((size_t)k * sizeof(double));
        for (int64_t i = 0; i < k; ++i) arow[i] = mx_value(ac + r * (k / 2), as + r * (k / 32), i);
        for (int64_t c = 0; c < n; ++c) {
            double s = 0.0, sa = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                const double p = arow[i] * mx_value(bc + c * (k / 2), bs + c * (k / 32), i);
                s += p;
                sa += fabs(p);
            }
            y[r * n + c] = s;
            absacc[r * n + c] = sa;
        }
        free(arow);
    }
}
