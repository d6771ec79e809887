// Internal launchers shared by the C-ABI layer and the HIP kernels.
// Every launcher assumes its arguments were validated by convrot_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// K-ROT: group-wise Hadamard-256 rotation + per-row absmax int8 quantization.
hipError_t launch_rotate_quant_bf16(const uint16_t* x, int64_t rows, int64_t k, int8_t* q,
                                    float* s, hipStream_t stream);
hipError_t launch_rotate_quant_f32(const float* x, int64_t rows, int64_t k, int8_t* q,
                                   float* s, hipStream_t stream);
// The same pass on h = bf16(silu(g) * u) formed from fc1's bf16 output
// gu [rows, 2i] (gate columns [0, i), up columns [i, 2i)); q is [rows, i].
hipError_t launch_swiglu_rotate_quant(const uint16_t* gu, int64_t rows, int64_t i, int8_t* q,
                                      float* s, hipStream_t stream);

// Load-time weight operations: W = (q . s) . H/16 per row, and
// W += scale * (B . A) in place (b [n, rank], a [rank, k]).
hipError_t launch_dequantize_weight(const int8_t* q, const float* s, int64_t n, int64_t k,
                                    float* w, hipStream_t stream);
hipError_t launch_lora_add(float* w, int64_t n, int64_t k, const float* b, const float* a,
                           int64_t rank, float scale, hipStream_t stream);

// The ConvRot linear behind convrot_linear / convrot_linear_swiglu (in
// convrot_api.cpp): linear_args validates sizes and pointers exactly as those
// entry points do (CONVROT_OK also for an empty call); linear_common validates
// and then runs rotate+quantize into the workspace and the GEMM (n_rows_w is
// n, or 2n with swiglu).  Both return a CONVROT_* status.
int linear_args(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w, const float* s_w,
                int64_t n, int64_t n_rows_w, const uint16_t* y);
int linear_common(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w, const float* s_w,
                  int64_t n, int64_t n_rows_w, uint16_t* y, void* workspace, size_t workspace_bytes,
                  bool swiglu, void* stream);

// K-GEMM: int8 x int8 -> int32 on MFMA with one of three epilogues.
enum class Epilogue { S32, BF16, SWIGLU };

// For Epilogue::SWIGLU, n is the output width i and q_w / s_w hold 2i rows.
hipError_t launch_gemm(Epilogue ep, const int8_t* q_x, const float* s_x, const int8_t* q_w,
                       const float* s_w, int64_t m, int64_t n, int64_t k, void* out,
                       hipStream_t stream);

// K-ATTN: int8 Q.K^T / fp16 P.V attention, head dimension 128.  Keys are
// padded to attn_pad_keys(s) (a multiple of 64).  prep: q/k/v are [s, ld]
// bf16 with head h at columns [128 h, 128 h + 128); writes qc [heads][s][128],
// sq [heads][s], kc [heads][s_pad][128], sk [heads][s_pad] and V^T blocks
// vt [heads][s_pad / 64][128][64] (fp16).  flash: out [s, ld_out] bf16.
int64_t attn_pad_keys(int64_t s);
hipError_t launch_attn_prep(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld,
                            int64_t s, int64_t heads, int8_t* qc, float* sq, int8_t* kc, float* sk,
                            void* vt, hipStream_t stream);
hipError_t launch_attn_flash(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                             const void* vt, int64_t s, int64_t heads, uint16_t* out, int64_t ld_out,
                             hipStream_t stream);

// MXFP4: block-32 E8M0 scales + FP4 E2M1 codes (two per byte) of rows of k
// elements (k % 128 == 0; with rotate, k % 256 == 0 and the rows are first
// rotated by the Hadamard-256 of the int8 path): codes [rows, k/2], scales
// chunk-major [k/128][rows][4].
hipError_t launch_mx_quant_bf16(const uint16_t* x, int64_t rows, int64_t k, bool rotate, uint8_t* codes,
                                uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_quant_f32(const float* x, int64_t rows, int64_t k, bool rotate, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream);
// out [m, n] bf16 = A [m, k] . B [n, k]^T over the decoded MXFP4 values.
hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, uint16_t* out,
                          hipStream_t stream);

}  // namespace convrot
