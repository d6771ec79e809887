// C ABI of the ConvRot int8 quantized linear (declared in include/convrot.h).
//
// This layer only validates arguments and enqueues the HIP kernels: every
// step of the computation runs on the GPU.  Validation happens before any HIP
// call, so argument errors never touch memory or the device.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/convrot.h"
#include "kernels.h"

namespace {

using convrot::Epilogue;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// k: a positive multiple of the 256-element Hadamard group, small enough that
// 127 * 127 * k fits int32.  Row counts must fit the launch grid (int32).
inline int check_k(int64_t k) {
    if (k <= 0 || (k % CONVROT_GROUP) != 0 || k > CONVROT_MAX_K) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

inline int check_rows(int64_t r) {
    if (r < 0 || r > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

inline int launched(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_ERR_LAUNCH; }

inline size_t ws_bytes(int64_t m, int64_t k) { return (size_t)m * (size_t)k + 4u * (size_t)m; }

// Shape checks of the GEMM entry points.  n_rows_w is the number of weight
// rows (n, or 2i for SwiGLU).
int check_gemm_shape(int64_t m, int64_t n, int64_t n_rows_w, int64_t k) {
    int st;
    if ((st = check_rows(m)) || (st = check_rows(n)) || (st = check_rows(n_rows_w)) ||
        (st = check_k(k)))
        return st;
    // the tile grid (256 tokens x at least 128 columns per workgroup) must fit one launch
    if (((m + 255) / 256) * ((n + 127) / 128) > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

// Pointer checks of the GEMM entry points (after the shape checks and the
// zero-size early return, so empty calls may pass NULL).
int check_gemm_ptrs(const void* q_x, const void* s_x, bool need_sx, const void* q_w,
                    const void* s_w, bool need_sw, const void* out) {
    if (!q_x || !q_w || !out || (need_sx && !s_x) || (need_sw && !s_w)) return CONVROT_ERR_NULL;
    if (!aligned16(q_x) || !aligned16(q_w) || !aligned16(out) || (need_sx && !aligned16(s_x)) ||
        (need_sw && !aligned16(s_w)))
        return CONVROT_ERR_ALIGN;
    return CONVROT_OK;
}

}  // namespace

extern "C" {

const char* convrot_status_string(int status) {
    switch (status) {
        case CONVROT_OK: return "ok";
        case CONVROT_ERR_NULL: return "a required pointer is NULL";
        case CONVROT_ERR_SHAPE:
            return "invalid shape (negative size, k not a positive multiple of 256, or k > 133120)";
        case CONVROT_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case CONVROT_ERR_WORKSPACE: return "workspace is NULL or smaller than convrot_workspace_bytes(m, k)";
        case CONVROT_ERR_LAUNCH: return "kernel launch failed (is the device gfx950?)";
        case CONVROT_ERR_SCRATCH:
            return "m * k + 4 * m exceeds the built-in scratch of convrot_linear_noalloc "
                   "(CONVROT_NOALLOC_SCRATCH_BYTES); use convrot_linear with a workspace";
        default: return "unknown status";
    }
}

size_t convrot_workspace_bytes(int64_t m, int64_t k) {
    if (check_rows(m) || check_k(k)) return 0;
    return ws_bytes(m, k);
}

int convrot_quantize_weight(const float* w, int64_t n, int64_t k, int8_t* q_w, float* s_w,
                            void* stream) {
    int st;
    if ((st = check_rows(n)) || (st = check_k(k))) return st;
    if (n == 0) return CONVROT_OK;
    if (!w || !q_w || !s_w) return CONVROT_ERR_NULL;
    if (!aligned16(w) || !aligned16(q_w) || !aligned16(s_w)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_rotate_quant_f32(w, n, k, q_w, s_w, (hipStream_t)stream));
}

int convrot_rotate_quant_act(const uint16_t* x, int64_t m, int64_t k, int8_t* q_x, float* s_x,
                             void* stream) {
    int st;
    if ((st = check_rows(m)) || (st = check_k(k))) return st;
    if (m == 0) return CONVROT_OK;
    if (!x || !q_x || !s_x) return CONVROT_ERR_NULL;
    if (!aligned16(x) || !aligned16(q_x) || !aligned16(s_x)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_rotate_quant_bf16(x, m, k, q_x, s_x, (hipStream_t)stream));
}

int convrot_swiglu_rotate_quant_act(const uint16_t* gu, int64_t m, int64_t i, int8_t* q_h,
                                    float* s_h, void* stream) {
    int st;
    if ((st = check_rows(m)) || (st = check_k(i))) return st;
    if (m == 0) return CONVROT_OK;
    if (!gu || !q_h || !s_h) return CONVROT_ERR_NULL;
    if (!aligned16(gu) || !aligned16(q_h) || !aligned16(s_h)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_swiglu_rotate_quant(gu, m, i, q_h, s_h, (hipStream_t)stream));
}

// Load-time weight operations.  Their grids are 1-D: at most 2^31 - 1
// workgroups of 16 groups (dequantize) or of 1024 columns x 8 rows (LoRA).
static int check_weight_grid(int64_t n, int64_t k) {
    const int64_t groups = n * (k / 256);
    if ((groups + 15) / 16 > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    if (((k / 4 + 255) / 256) * ((n + 7) / 8) > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

int convrot_dequantize_weight(const int8_t* q_w, const float* s_w, int64_t n, int64_t k, float* w,
                              void* stream) {
    int st;
    if ((st = check_rows(n)) || (st = check_k(k)) || (st = check_weight_grid(n, k))) return st;
    if (n == 0) return CONVROT_OK;
    if (!q_w || !s_w || !w) return CONVROT_ERR_NULL;
    if (!aligned16(q_w) || !aligned16(s_w) || !aligned16(w)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_dequantize_weight(q_w, s_w, n, k, w, (hipStream_t)stream));
}

int convrot_lora_add(float* w, int64_t n, int64_t k, const float* lora_b, const float* lora_a,
                     int64_t rank, float scale, void* stream) {
    int st;
    if ((st = check_rows(n)) || (st = check_k(k)) || (st = check_rows(rank)) ||
        (st = check_weight_grid(n, k)))
        return st;
    if (n == 0) return CONVROT_OK;
    if (!w || (rank > 0 && (!lora_b || !lora_a))) return CONVROT_ERR_NULL;
    if (!aligned16(w) || !aligned16(lora_b) || !aligned16(lora_a)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_lora_add(w, n, k, lora_b, lora_a, rank, scale, (hipStream_t)stream));
}

size_t convrot_merge_workspace_bytes(int64_t n, int64_t k) {
    if (check_rows(n) || check_k(k)) return 0;
    return 4u * (size_t)n * (size_t)k;
}

int convrot_merge_lora(const int8_t* q_w, const float* s_w, int64_t n, int64_t k, const float* lora_b,
                       const float* lora_a, int64_t rank, float scale, int8_t* q_out, float* s_out,
                       void* workspace, size_t workspace_bytes, void* stream) {
    int st;
    if ((st = check_rows(n)) || (st = check_k(k)) || (st = check_rows(rank)) ||
        (st = check_weight_grid(n, k)))
        return st;
    if (n == 0) return CONVROT_OK;
    if (!q_w || !s_w || !q_out || !s_out || (rank > 0 && (!lora_b || !lora_a))) return CONVROT_ERR_NULL;
    if (!aligned16(q_w) || !aligned16(s_w) || !aligned16(q_out) || !aligned16(s_out) ||
        !aligned16(lora_b) || !aligned16(lora_a))
        return CONVROT_ERR_ALIGN;
    if (!workspace || workspace_bytes < convrot_merge_workspace_bytes(n, k)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CONVROT_ERR_ALIGN;
    float* w = (float*)workspace;
    hipStream_t s = (hipStream_t)stream;
    if (convrot::launch_dequantize_weight(q_w, s_w, n, k, w, s) != hipSuccess) return CONVROT_ERR_LAUNCH;
    if (convrot::launch_lora_add(w, n, k, lora_b, lora_a, rank, scale, s) != hipSuccess)
        return CONVROT_ERR_LAUNCH;
    return launched(convrot::launch_rotate_quant_f32(w, n, k, q_out, s_out, s));
}

int convrot_gemm_s32(const int8_t* q_x, const int8_t* q_w, int64_t m, int64_t n, int64_t k,
                     int32_t* acc, void* stream) {
    int st = check_gemm_shape(m, n, n, k);
    if (st) return st;
    if (m == 0 || n == 0) return CONVROT_OK;
    if ((st = check_gemm_ptrs(q_x, nullptr, false, q_w, nullptr, false, acc))) return st;
    return launched(convrot::launch_gemm(Epilogue::S32, q_x, nullptr, q_w, nullptr, m, n, k, acc,
                                         (hipStream_t)stream));
}

int convrot_gemm_dequant(const int8_t* q_x, const float* s_x, const int8_t* q_w, const float* s_w,
                         int64_t m, int64_t n, int64_t k, uint16_t* y, void* stream) {
    int st = check_gemm_shape(m, n, n, k);
    if (st) return st;
    if (m == 0 || n == 0) return CONVROT_OK;
    if ((st = check_gemm_ptrs(q_x, s_x, true, q_w, s_w, true, y))) return st;
    return launched(convrot::launch_gemm(Epilogue::BF16, q_x, s_x, q_w, s_w, m, n, k, y,
                                         (hipStream_t)stream));
}

int convrot_gemm_swiglu(const int8_t* q_x, const float* s_x, const int8_t* q_w, const float* s_w,
                        int64_t m, int64_t i, int64_t k, uint16_t* y, void* stream) {
    if (i < 0 || i > (int64_t)INT32_MAX / 2) return CONVROT_ERR_SHAPE;
    int st = check_gemm_shape(m, i, 2 * i, k);
    if (st) return st;
    if (m == 0 || i == 0) return CONVROT_OK;
    if ((st = check_gemm_ptrs(q_x, s_x, true, q_w, s_w, true, y))) return st;
    return launched(convrot::launch_gemm(Epilogue::SWIGLU, q_x, s_x, q_w, s_w, m, i, k, y,
                                         (hipStream_t)stream));
}

}  // extern "C"

namespace convrot {

int linear_args(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w, const float* s_w,
                int64_t n, int64_t n_rows_w, const uint16_t* y) {
    if (n < 0 || n > (int64_t)INT32_MAX / 2) return CONVROT_ERR_SHAPE;
    int st;
    if ((st = check_gemm_shape(m, n, n_rows_w, k))) return st;
    if (m == 0 || n == 0) return CONVROT_OK;
    return check_gemm_ptrs(x, nullptr, false, q_w, s_w, true, y);
}

int linear_common(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w, const float* s_w,
                  int64_t n, int64_t n_rows_w, uint16_t* y, void* workspace, size_t workspace_bytes,
                  bool swiglu, void* stream) {
    int st;
    if ((st = linear_args(x, m, k, q_w, s_w, n, n_rows_w, y))) return st;
    if (m == 0 || n == 0) return CONVROT_OK;
    if (!workspace || workspace_bytes < ws_bytes(m, k)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CONVROT_ERR_ALIGN;
    int8_t* q_x = (int8_t*)workspace;
    float* s_x = (float*)((char*)workspace + (size_t)m * (size_t)k);
    hipStream_t s = (hipStream_t)stream;
    if (convrot::launch_rotate_quant_bf16(x, m, k, q_x, s_x, s) != hipSuccess) return CONVROT_ERR_LAUNCH;
    return launched(convrot::launch_gemm(swiglu ? Epilogue::SWIGLU : Epilogue::BF16, q_x, s_x, q_w,
                                         s_w, m, n, k, y, s));
}

}  // namespace convrot

extern "C" {

int convrot_linear(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w, const float* s_w,
                   int64_t n, uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
    return convrot::linear_common(x, m, k, q_w, s_w, n, n, y, workspace, workspace_bytes, false, stream);
}

int convrot_linear_swiglu(const uint16_t* x, int64_t m, int64_t k, const int8_t* q_w,
                          const float* s_w, int64_t i, uint16_t* y, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (i < 0 || i > (int64_t)INT32_MAX / 2) return CONVROT_ERR_SHAPE;
    return convrot::linear_common(x, m, k, q_w, s_w, i, 2 * i, y, workspace, workspace_bytes, true, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ attention

namespace {

// The flash kernel addresses one head's V^T blocks (s_pad x 128 fp16) through a
// 32-bit buffer range, so s_pad * 256 must stay below 2^32: s_pad <= 2^24 - 64.
constexpr int64_t kAttnMaxS = ((int64_t)1 << 24) - 64;

inline size_t align256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// Region offsets of the attention workspace (see convrot.h); returns the
// total size, or 0 for invalid sizes.
bool attn_sizes_ok(int64_t s, int64_t heads, int64_t head_dim) {
    return s >= 0 && s <= kAttnMaxS && heads >= 0 && head_dim == CONVROT_ATTN_HEAD_DIM &&
           heads <= (int64_t)INT32_MAX / (kAttnMaxS / 64);
}

size_t attn_layout(int64_t s, int64_t heads, int64_t head_dim, size_t off[5]) {
    if (!attn_sizes_ok(s, heads, head_dim)) return 0;
    const size_t S = (size_t)s, H = (size_t)heads, P = (size_t)convrot::attn_pad_keys(s);
    size_t o[6];
    o[0] = 0;
    o[1] = align256(o[0] + H * S * 128);
    o[2] = align256(o[1] + H * S * 4);
    o[3] = align256(o[2] + H * P * 128);
    o[4] = align256(o[3] + H * P * 4);
    o[5] = align256(o[4] + H * P * 128 * 2);
    if (off)
        for (int i = 0; i < 5; ++i) off[i] = o[i];
    return o[5];
}

int check_attn(int64_t s, int64_t heads, int64_t head_dim, int64_t ld) {
    if (!attn_sizes_ok(s, heads, head_dim)) return CONVROT_ERR_SHAPE;
    if (ld < heads * CONVROT_ATTN_HEAD_DIM || (ld % 8) != 0) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

}  // namespace

extern "C" {

size_t convrot_attention_workspace(int64_t s, int64_t heads, int64_t head_dim, size_t offsets[5]) {
    return attn_layout(s, heads, head_dim, offsets);
}

int convrot_attention_prep(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld,
                           int64_t s, int64_t heads, int64_t head_dim, void* workspace,
                           size_t workspace_bytes, void* stream) {
    if (int st = check_attn(s, heads, head_dim, ld)) return st;
    if (s == 0 || heads == 0) return CONVROT_OK;
    if (!q || !k || !v) return CONVROT_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return CONVROT_ERR_ALIGN;
    size_t off[5];
    const size_t need = attn_layout(s, heads, head_dim, off);
    if (!workspace || workspace_bytes < need) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CONVROT_ERR_ALIGN;
    uint8_t* w = (uint8_t*)workspace;
    return launched(convrot::launch_attn_prep(q, k, v, ld, s, heads, (int8_t*)(w + off[0]),
                                              (float*)(w + off[1]), (int8_t*)(w + off[2]),
                                              (float*)(w + off[3]), w + off[4], (hipStream_t)stream));
}

int convrot_attention_prepared(const void* workspace, size_t workspace_bytes, int64_t s,
                               int64_t heads, int64_t head_dim, uint16_t* out, int64_t ld_out,
                               void* stream) {
    if (int st = check_attn(s, heads, head_dim, ld_out)) return st;
    if (s == 0 || heads == 0) return CONVROT_OK;
    if (!out) return CONVROT_ERR_NULL;
    if (!aligned16(out)) return CONVROT_ERR_ALIGN;
    size_t off[5];
    const size_t need = attn_layout(s, heads, head_dim, off);
    if (!workspace || workspace_bytes < need) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CONVROT_ERR_ALIGN;
    const uint8_t* w = (const uint8_t*)workspace;
    return launched(convrot::launch_attn_flash((const int8_t*)(w + off[0]), (const float*)(w + off[1]),
                                               (const int8_t*)(w + off[2]), (const float*)(w + off[3]),
                                               w + off[4], s, heads, out, ld_out, (hipStream_t)stream));
}

int convrot_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld, int64_t s,
                      int64_t heads, int64_t head_dim, uint16_t* out, int64_t ld_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (int st = check_attn(s, heads, head_dim, ld)) return st;
    if (int st = check_attn(s, heads, head_dim, ld_out)) return st;
    if (s == 0 || heads == 0) return CONVROT_OK;
    if (!out) return CONVROT_ERR_NULL;
    if (!aligned16(out)) return CONVROT_ERR_ALIGN;
    if (int st = convrot_attention_prep(q, k, v, ld, s, heads, head_dim, workspace, workspace_bytes,
                                        stream))
        return st;
    return convrot_attention_prepared(workspace, workspace_bytes, s, heads, head_dim, out, ld_out,
                                      stream);
}

}  // extern "C"

// ------------------------------------------------------------------ MXFP4

namespace {

int check_mx_k(int64_t k, int rotate = 0) {
    if (k <= 0 || (k % (rotate ? 256 : 128)) != 0 || k > CONVROT_MX_MAX_K) return CONVROT_ERR_SHAPE;
    return CONVROT_OK;
}

int check_mx_rows(int64_t r, int64_t k) {
    // (the rotated pass launches r * k / 4096 workgroups, fewer than the plain one)
    if (r < 0 || r > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    if (r * (k / 8) > (int64_t)INT32_MAX * 256) return CONVROT_ERR_SHAPE;   // quantize grid
    return CONVROT_OK;
}

size_t mx_scales_offset(int64_t m, int64_t k) { return ((size_t)m * (size_t)(k / 2) + 255u) & ~(size_t)255u; }

}  // namespace

extern "C" {

int convrot_mx_quantize_act(const uint16_t* x, int64_t m, int64_t k, int rotate, uint8_t* codes,
                            uint8_t* scales, void* stream) {
    if (int st = check_mx_k(k, rotate)) return st;
    if (int st = check_mx_rows(m, k)) return st;
    if (m == 0) return CONVROT_OK;
    if (!x || !codes || !scales) return CONVROT_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_mx_quant_bf16(x, m, k, rotate != 0, codes, scales, (hipStream_t)stream));
}

int convrot_mx_quantize_weight(const float* w, int64_t n, int64_t k, int rotate, uint8_t* codes,
                               uint8_t* scales, void* stream) {
    if (int st = check_mx_k(k, rotate)) return st;
    if (int st = check_mx_rows(n, k)) return st;
    if (n == 0) return CONVROT_OK;
    if (!w || !codes || !scales) return CONVROT_ERR_NULL;
    if (!aligned16(w) || !aligned16(codes) || !aligned16(scales)) return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_mx_quant_f32(w, n, k, rotate != 0, codes, scales, (hipStream_t)stream));
}

int convrot_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, uint16_t* out,
                    void* stream) {
    if (int st = check_mx_k(k)) return st;
    if (m < 0 || n < 0 || m > (int64_t)INT32_MAX || n > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    if (((m + 255) / 256) * ((n + 255) / 256) > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    if ((m > 0 && m * (k / 2) > (int64_t)UINT32_MAX) || (n > 0 && n * (k / 2) > (int64_t)UINT32_MAX))
        return CONVROT_ERR_SHAPE;   // 32-bit buffer ranges of one operand
    if (m == 0 || n == 0) return CONVROT_OK;
    if (!a_codes || !a_scales || !b_codes || !b_scales || !out) return CONVROT_ERR_NULL;
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales) ||
        !aligned16(out))
        return CONVROT_ERR_ALIGN;
    return launched(convrot::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, m, n, k, out,
                                            (hipStream_t)stream));
}

size_t convrot_mx_workspace_bytes(int64_t m, int64_t k) {
    if (check_mx_k(k) || check_mx_rows(m, k)) return 0;
    return mx_scales_offset(m, k) + (size_t)m * (size_t)(k / 32);
}

int convrot_mx_linear(const uint16_t* x, int64_t m, int64_t k, int rotate, const uint8_t* w_codes,
                      const uint8_t* w_scales, int64_t n, uint16_t* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
    if (int st = check_mx_k(k, rotate)) return st;
    if (int st = check_mx_rows(m, k)) return st;
    if (n < 0 || n > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    if (((m + 255) / 256) * ((n + 255) / 256) > (int64_t)INT32_MAX) return CONVROT_ERR_SHAPE;
    if ((m * (k / 2) > (int64_t)UINT32_MAX) || (n * (k / 2) > (int64_t)UINT32_MAX)) return CONVROT_ERR_SHAPE;
    if (m == 0 || n == 0) return CONVROT_OK;
    if (!x || !w_codes || !w_scales || !out) return CONVROT_ERR_NULL;
    if (!aligned16(x) || !aligned16(w_codes) || !aligned16(w_scales) || !aligned16(out))
        return CONVROT_ERR_ALIGN;
    if (!workspace || workspace_bytes < convrot_mx_workspace_bytes(m, k)) return CONVROT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return CONVROT_ERR_ALIGN;
    uint8_t* codes = (uint8_t*)workspace;
    uint8_t* scales = codes + mx_scales_offset(m, k);
    hipStream_t s = (hipStream_t)stream;
    if (convrot::launch_mx_quant_bf16(x, m, k, rotate != 0, codes, scales, s) != hipSuccess)
        return CONVROT_ERR_LAUNCH;
    return launched(convrot::launch_gemm_mx(codes, scales, w_codes, w_scales, m, n, k, out, s));
}

}  // extern "C"
