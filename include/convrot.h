/*
 * convrot.h -- C ABI of the ConvRot int8 quantized linear for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (MiniMax H3 DiT projections, hidden size 5376):
 *   1. rotate each activation row along K with the orthonormal Hadamard of
 *      size 256, group by group (cloud-worker docs/RESEARCH.md, "Weight
 *      families": ConvRot is a group-wise Hadamard rotation written as a
 *      convolution, which spreads activation outliers; h3-rs README, model
 *      file table: "Hadamard-256");
 *   2. quantize the rotated row to int8 with one symmetric scale per token
 *      (h3-rs README, "Speed": the fused GEMM quantizes activations per row and
 *      the rotation runs inside that quantizer);
 *   3. contract with int8 weights that were rotated the same way and quantized
 *      with one scale per output row, accumulating in int32 (h3-rs README,
 *      model file table: "int8 per-row"; quantized weights stay quantized in
 *      memory);
 *   4. rescale by both scales and write bf16 (h3-rs README, "Speed": the GEMM
 *      writes bf16 directly), optionally applying SwiGLU to paired gate/up rows
 *      in the same epilogue (h3-rs README, "Speed": fc1's gate/up rows are
 *      paired so SwiGLU fuses into the epilogue; Minimax_h3_hybrid model card,
 *      "Checkpoints": int8 ConvRot keeps the fused SwiGLU path).
 *
 * Exact definitions, as computed:
 *   rotation   v = x . blockdiag(H/16), H[i][j] = (-1)^popcount(i & j), over
 *              contiguous groups of 256; fp32 butterfly with spans 1, 2, ...,
 *              128 in that order, each step one RNE add or subtract, then * 1/16;
 *   scale      s = max_k |v_k| / 127 (correctly rounded fp32);
 *   codes      q_k = rint(v_k / s) with a correctly rounded quotient and round
 *              half to even; s == 0 gives all-zero codes;
 *   contract   acc[m][n] = sum_k q_x[m][k] * q_w[n][k] (exact int32);
 *   dequant    y = bf16_rne(((float)acc * s_x[m]) * s_w[n]);
 *   SwiGLU     g, u = the fp32 dequant of gate column j and up column i + j;
 *              y = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)), in the
 *              fused epilogue evaluated on the transcendental unit as
 *              (g * rcp(1 + exp2(-g * log2 e))) * u: y lies within 2^-8 |y|
 *              of the exact value (one bf16 rounding plus ~1.2e-5 relative
 *              from the fp32 evaluation), or within |g u| 2^-126 where
 *              1 + e^-g exceeds 2^126.
 *   fixed exp  the output-side SwiGLU pass (convrot_swiglu_rotate_quant_act),
 *              whose h decides int8 codes, uses one fixed fp32 exp instead
 *              (Cody-Waite reduction with ln2 split into 0x1.62e4p-1 +
 *              0x1.7f7d1cp-20, k = rint(x * 0x1.715476p+0), degree-7 Taylor
 *              polynomial in Horner form with fused multiply-adds, scaled by
 *              2^k; exp(x) = +inf for x > 88.72 and 0 for x < -86) and one IEEE
 *              division, so that its codes are reproducible bit for bit.
 * All results are deterministic: the same inputs give the same bytes on every
 * call, launch shape and device of this architecture; every result except
 * the fused SwiGLU output is the definition's rounding sequence bit for bit.
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers, owned by the caller.  The library
 *     never allocates, frees, synchronizes, or changes the current device.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream) on the current device.
 *   - Arrays are dense and row-major (leading dimension = last extent).
 *     bf16 travels as its raw 16-bit pattern (uint16_t).
 *   - Every pointer must be 16-byte aligned.
 *   - k must be a positive multiple of 256 and at most 133120 (so that
 *     127 * 127 * k < 2^31: the int32 accumulator cannot overflow).
 *   - m == 0 or n == 0 (i == 0) is success with no work enqueued; sizes are
 *     checked first, so an empty call may pass NULL pointers.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     leave all memory untouched.  A failed launch returns CONVROT_ERR_LAUNCH
 *     (this includes a device that is not gfx950).  Faults during execution
 *     surface at the caller's next synchronization.  Nothing aborts and no C++
 *     exception crosses the ABI.
 *   - Outputs must not overlap inputs.  Non-finite inputs give unspecified
 *     outputs.
 *   - The library keeps no state; calls are thread-safe and reentrant.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    CONVROT_OK = 0,
    CONVROT_ERR_NULL = 1,      /* a required pointer is NULL                      */
    CONVROT_ERR_SHAPE = 2,     /* negative size, k % 256 != 0, k > 133120, ...   */
    CONVROT_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned               */
    CONVROT_ERR_WORKSPACE = 4, /* workspace NULL or smaller than required        */
    CONVROT_ERR_LAUNCH = 5,    /* the kernel launch failed (see hipGetLastError) */
    CONVROT_ERR_SCRATCH = 6    /* too large for convrot_linear_noalloc's scratch  */
};

#define CONVROT_GROUP 256
#define CONVROT_MAX_K 133120

/* Load-time weight preparation (h3-rs README, model file table: int8 per-row +
 * ConvRot Hadamard-256; weights stay quantized in memory).
 *   w    [n, k] fp32 input weight (rows = output channels)
 *   q_w  [n, k] int8 output codes of the rotated rows
 *   s_w  [n]    fp32 output per-row scales                                  */
int convrot_quantize_weight(const float* w, int64_t n, int64_t k,
                            int8_t* q_w, float* s_w, void* stream);

/* Per-token activation rotation + quantization (h3-rs README, "Speed").
 *   x    [m, k] bf16 input activations
 *   q_x  [m, k] int8 output codes
 *   s_x  [m]    fp32 output per-token scales                                */
int convrot_rotate_quant_act(const uint16_t* x, int64_t m, int64_t k,
                             int8_t* q_x, float* s_x, void* stream);

/* The down projection's activation preparation with SwiGLU applied in front
 * of the rotation instead of in fc1's epilogue (Minimax_h3_hybrid model card,
 * "Native NVFP4 projection benchmarks": an "FFN output + SwiGLU" projection).
 * fc1 writes its dequantized gate and up columns as bf16 (convrot_linear with
 * n = 2i); this pass forms h = bf16(silu(g) * u), silu(g) = g / (1 + exp(-g))
 * with the fixed exponential and one IEEE division, widens h exactly,
 * and rotates and quantizes it per token as convrot_rotate_quant_act does.
 *   gu   [m, 2i] bf16: columns [0, i) gate, columns [i, 2i) up
 *   q_h  [m, i]  int8 output codes;  s_h [m] fp32 output per-token scales
 * i is the down projection's k: i % 256 == 0, i <= CONVROT_MAX_K.            */
int convrot_swiglu_rotate_quant_act(const uint16_t* gu, int64_t m, int64_t i,
                                    int8_t* q_h, float* s_h, void* stream);

/* Workspace that convrot_linear / convrot_linear_swiglu need for m tokens of
 * length k: q_x at offset 0 (m * k bytes), then s_x at offset m * k (4 * m
 * bytes; 256-byte aligned whenever the workspace is, since k % 256 == 0).
 * Returns 0 for invalid sizes.                                               */
size_t convrot_workspace_bytes(int64_t m, int64_t k);

/* The ConvRot int8 linear: y = dequant(rotate_quant(x) . q_w^T) (h3-rs
 * README, "Speed": fused int8 GEMM that quantizes activations per row and
 * writes bf16 directly).
 *   x          [m, k] bf16 activations
 *   q_w, s_w   [n, k] int8 / [n] fp32 from convrot_quantize_weight
 *   y          [m, n] bf16 output
 *   workspace  >= convrot_workspace_bytes(m, k) bytes of device memory; on
 *              return it holds this call's q_x and s_x (enqueued).          */
int convrot_linear(const uint16_t* x, int64_t m, int64_t k,
                   const int8_t* q_w, const float* s_w, int64_t n,
                   uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* The same linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * it takes no workspace and calls no allocator.  Its q_x / s_x (the
 * workspace of convrot_linear, m * k + 4 * m bytes) live in a fixed array of
 * CONVROT_NOALLOC_SCRATCH_BYTES in the library's device code, which every GPU
 * the library runs this call on holds until the process ends; the array's
 * device address is looked up once per device on the first call there.
 * Arguments, checks, results and errors are those of convrot_linear, except:
 *   - m * k + 4 * m > CONVROT_NOALLOC_SCRATCH_BYTES returns
 *     CONVROT_ERR_SCRATCH before anything is enqueued (use convrot_linear);
 *   - every call on one GPU uses that GPU's one array, so calls on one GPU
 *     whose executions overlap (different streams, no ordering between them)
 *     race on it and give unspecified outputs; calls on one stream are
 *     ordered and safe.  Nothing in the array needs to start at zero: each
 *     call writes q_x and s_x before it reads them.                          */
#define CONVROT_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int convrot_linear_noalloc(const uint16_t* x, int64_t m, int64_t k,
                           const int8_t* q_w, const float* s_w, int64_t n,
                           uint16_t* y, void* stream);

/* The fc1 ConvRot linear with SwiGLU fused into its epilogue (h3-rs README,
 * "Speed"; Minimax_h3_hybrid model card, "Checkpoints").
 *   q_w, s_w   [2i, k] int8 / [2i] fp32: rows [0, i) are the gate projection,
 *              rows [i, 2i) the up projection (quantize the whole [2i, k]
 *              weight with convrot_quantize_weight; scales are per row, so this
 *              equals quantizing the halves separately)
 *   y          [m, i] bf16 output silu(gate) * up, within 2^-8 |y| of the
 *              exact value (the SwiGLU line of the arithmetic above)          */
int convrot_linear_swiglu(const uint16_t* x, int64_t m, int64_t k,
                          const int8_t* q_w, const float* s_w, int64_t i,
                          uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* The contraction with its bf16 dequant epilogue on codes prepared by the
 * caller (the second half of convrot_linear).
 *   q_x, s_x   [m, k] int8 / [m] fp32;  q_w, s_w  [n, k] int8 / [n] fp32
 *   y          [m, n] bf16                                                   */
int convrot_gemm_dequant(const int8_t* q_x, const float* s_x, const int8_t* q_w,
                         const float* s_w, int64_t m, int64_t n, int64_t k,
                         uint16_t* y, void* stream);

/* The contraction with the SwiGLU epilogue on prepared codes (the second half
 * of convrot_linear_swiglu).  q_w, s_w have 2i rows; y is [m, i] bf16.       */
int convrot_gemm_swiglu(const int8_t* q_x, const float* s_x, const int8_t* q_w,
                        const float* s_w, int64_t m, int64_t i, int64_t k,
                        uint16_t* y, void* stream);

/* The raw int32 accumulators of the same contraction (same main loop), for
 * exact checks: acc [m, n] int32 = q_x . q_w^T.                              */
int convrot_gemm_s32(const int8_t* q_x, const int8_t* q_w, int64_t m, int64_t n, int64_t k,
                     int32_t* acc, void* stream);

/* ---- load-time weight operations: merging a LoRA into ConvRot weights ----
 * (h3-rs README, "Speed": LoRAs are merged into the int8 weights at load by
 * dequantizing, adding and requantizing, so they cost nothing per step;
 * model file table: quantized weights are dequantized per layer by kernels.) */

/* Dequantize ConvRot weights back to the unrotated basis:
 *   w[r][c] = RN((H q_r / 16)[c] * s_w[r]) per 256-group (H/16 is its own
 *   inverse; the code rotation is exact in fp32, the multiply is the only
 *   rounding).
 *   q_w [n, k] int8, s_w [n] fp32 (from convrot_quantize_weight); w [n, k] fp32
 *   output.  Sizes as convrot_quantize_weight.                              */
int convrot_dequantize_weight(const int8_t* q_w, const float* s_w, int64_t n, int64_t k,
                              float* w, void* stream);

/* Add a low-rank delta in place: w[r][c] += scale * sum_j b[r][j] * a[j][c],
 * the sum over j in increasing order as a chain of fp32 fused multiply-adds
 * from 0, then one multiply by scale and one add (each rounded to nearest).
 *   w [n, k] fp32 (in/out); b [n, rank] fp32 (the LoRA up factor); a [rank, k]
 *   fp32 (the down factor); scale = strength * alpha / rank, as the caller
 *   defines it.  rank >= 0; b and a may be NULL when rank == 0.              */
int convrot_lora_add(float* w, int64_t n, int64_t k, const float* lora_b, const float* lora_a,
                     int64_t rank, float scale, void* stream);

/* Workspace convrot_merge_lora needs: the fp32 weights, 4 * n * k bytes
 * (0 for invalid sizes).                                                     */
size_t convrot_merge_workspace_bytes(int64_t n, int64_t k);

/* Merge a LoRA into ConvRot weights: dequantize (as convrot_dequantize_weight)
 * into the workspace, add the delta there (as convrot_lora_add), and quantize
 * the result again (as convrot_quantize_weight) into q_out / s_out.  The three
 * steps run in order on the stream, so q_out / s_out may be q_w / s_w (an
 * in-place update).  On return the workspace holds the merged fp32 weights. */
int convrot_merge_lora(const int8_t* q_w, const float* s_w, int64_t n, int64_t k,
                       const float* lora_b, const float* lora_a, int64_t rank, float scale,
                       int8_t* q_out, float* s_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * int8 Q.K^T / fp16 P.V attention (h3-rs README, "Speed": the DiT's attention
 * is one flash kernel with an int8 Q.K^T and an fp16 P.V; Minimax_h3_hybrid
 * model card, "Notes and limitations": full attention, no mask).
 *
 * Q, K, V are [s, ld] bf16 row-major with head h at columns
 * [h * 128, h * 128 + 128) -- the thirds of the fused QKV projection's output
 * may be passed directly (ld = 3 * heads * 128).  Head dimension 128 only.
 *   quantize   per token and head, as the layer's per-row quantizer without
 *              rotation: s = max|x| / 127 over the head's 128 values
 *              (correctly rounded fp32), codes rint(x / s), half to even,
 *              s == 0 gives zero codes;
 *   logits     acc_ij * s_q[i] * s_k[j] / sqrt(128), acc_ij the exact int32
 *              dot product of the codes (evaluated in fp32, base 2);
 *   softmax    over all s keys, probabilities rounded to fp16;
 *   output     O_i = sum_j p_ij v_j / sum_j p_ij with V rounded to fp16 (RNE),
 *              fp32 sums, written as bf16 (RNE) to out [s, ld_out], head h at
 *              columns [h * 128, h * 128 + 128).
 * The codes and scales are bit-exact; the output agrees with the fp64
 * evaluation of the same definition to the rounding of the fp16 probabilities,
 * the fp32 sums and the bf16 store.
 *
 * Shapes: 0 <= s <= 2^24 - 64 (one head's fp16 V blocks must fit a 32-bit
 * byte range), heads >= 0, head_dim == 128; ld and ld_out are
 * multiples of 8 and at least heads * 128.  s == 0 or heads == 0 is success
 * with nothing enqueued.  V values beyond the fp16 range give unspecified
 * outputs.  The output must not overlap the inputs or the workspace.
 * ------------------------------------------------------------------------ */
#define CONVROT_ATTN_HEAD_DIM 128

/* Workspace of the attention of s tokens and `heads` heads; returns its size
 * in bytes (0 for invalid sizes).  If `offsets` is not NULL it receives the
 * byte offsets of the five regions (each 256-byte aligned), s_pad being s
 * rounded up to a multiple of 64:
 *   [0] Q codes   int8 [heads][s][128]
 *   [1] Q scales  fp32 [heads][s]
 *   [2] K codes   int8 [heads][s_pad][128]   (rows past s are zero)
 *   [3] K scales  fp32 [heads][s_pad]        (zero past s)
 *   [4] V         fp16 [heads][s_pad / 64][128][64]: per block of 64 keys,
 *                 row d holds head dimension d of the 64 keys, key j of each
 *                 32 at position j with bits 2 and 3 swapped (zero past s). */
size_t convrot_attention_workspace(int64_t s, int64_t heads, int64_t head_dim, size_t offsets[5]);

/* Step 1: quantize Q and K and lay out V in the workspace.                  */
int convrot_attention_prep(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld,
                           int64_t s, int64_t heads, int64_t head_dim, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Step 2: attention over a workspace filled by convrot_attention_prep with
 * the same s and heads.                                                      */
int convrot_attention_prepared(const void* workspace, size_t workspace_bytes, int64_t s,
                               int64_t heads, int64_t head_dim, uint16_t* out, int64_t ld_out,
                               void* stream);

/* Both steps in order on the stream.                                        */
int convrot_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld, int64_t s,
                      int64_t heads, int64_t head_dim, uint16_t* out, int64_t ld_out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MXFP4 projections: the analog, on MI355X's native microscaling format, of
 * the hybrid checkpoints that run the QKV and FFN-input projections in a
 * 4-bit block format while the output projections stay int8 ConvRot
 * (Minimax_h3_hybrid model card, "Checkpoints"; its 4-bit format, NVFP4, is
 * a different hardware's).  OCP MXFP4 as computed here:
 *   blocks     32 consecutive elements of a row along k share one scale 2^e,
 *              e = floor(log2(max |v|)) - 2 clamped to [-127, 127], stored as
 *              the byte e + 127 (E8M0); an all-zero block has byte 0;
 *   elements   v / 2^e (exact) rounded to FP4 E2M1 -- magnitudes 0, 0.5, 1,
 *              1.5, 2, 3, 4, 6 -- to nearest, ties to the even mantissa bit,
 *              saturating at 6; the sign bit is v's; element 2j is the low
 *              nibble of byte j of the row's codes;
 *   product    y[m][n] = bf16_rne(sum_k a[m][k] b[n][k]) over the decoded
 *              values, both block scales applied inside the MFMA, fp32
 *              accumulation (within 2^-8 |y| + (k/32) 2^-23 sum |a b| of the
 *              exact value);
 *   rotation   optional (rotate != 0): the rows are first rotated along k
 *              with the orthonormal Hadamard-256 exactly as the int8 ConvRot
 *              path rotates them (k a multiple of 256), which keeps the
 *              product of two rotated operands and spreads outlier channels
 *              across their group; rotate == 0 is the plain format, like the
 *              hybrid's 4-bit layers, which carry no rotation.
 * Layouts: codes [rows, k/2] bytes, row-major; scales chunk-major
 * [k/128][rows][4] bytes -- the scale of block b of row r is byte
 * (b / 4) * rows * 4 + r * 4 + b % 4 -- so that the four scales of one
 * 128-element chunk of consecutive rows are contiguous, as the product
 * streams them.
 * k must be a positive multiple of 128 (256 when rotating), at most 2^20.
 * Pointers 16-byte aligned; sizes checked first; rows == 0 is a no-op.
 * Both operands of a product must be quantized with the same rotate flag.
 * ------------------------------------------------------------------------ */
#define CONVROT_MX_MAX_K (1 << 20)

/* Quantize bf16 activation rows x [m, k] to MXFP4 (rotated if rotate).     */
int convrot_mx_quantize_act(const uint16_t* x, int64_t m, int64_t k, int rotate, uint8_t* codes,
                            uint8_t* scales, void* stream);

/* Quantize fp32 weight rows w [n, k] to MXFP4 (load time; rotated if rotate). */
int convrot_mx_quantize_weight(const float* w, int64_t n, int64_t k, int rotate, uint8_t* codes,
                               uint8_t* scales, void* stream);

/* out [m, n] bf16 = A . B^T of MXFP4 operands A [m, k] and B [n, k].        */
int convrot_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, uint16_t* out,
                    void* stream);

/* Workspace convrot_mx_linear needs for m rows of k: the activation codes
 * and scales (0 for invalid sizes).                                         */
size_t convrot_mx_workspace_bytes(int64_t m, int64_t k);

/* MXFP4 linear: quantize x [m, k] (bf16; rotated if rotate) into the
 * workspace, then the product with a weight prepared with the same rotate
 * flag (codes [n, k/2], scales [k/128][n][4]).                              */
int convrot_mx_linear(const uint16_t* x, int64_t m, int64_t k, int rotate, const uint8_t* w_codes,
                      const uint8_t* w_scales, int64_t n, uint16_t* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL).         */
const char* convrot_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
