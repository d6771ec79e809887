// Device arithmetic of the GEMM epilogues and the rotate+quantize passes
// that must be reproducible bit for bit, evaluated op for op as the layer's
// definition fixes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Two fp32 values -> packed bf16 bits (lo = a, hi = b), round to nearest
// even: one v_cvt_pk_bf16_f32 on gfx950 (fp32 denormals are kept, so a
// denormal value rounds to the bf16 denormal below or above it).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Fixed fp32 exponential (Cody-Waite reduction with ln 2 split into a 15-bit
// head and its tail, degree-7 Taylor polynomial in Horner form with fused
// multiply-adds, exact 2^k scaling).  Valid for x in [-86, 88.72].
__device__ __forceinline__ float exp_cw_core(float x) {
    const float kf = __builtin_rintf(x * 0x1.715476p+0f);
    float r = __builtin_fmaf(-kf, 0x1.62e4p-1f, x);
    r = __builtin_fmaf(-kf, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)kf);
}

// 1 + exp(x) as silu's denominator needs it, branch-free.  The fixed
// exponential is +inf above 88.72 and 0 below -86.  Below -86 the polynomial
// evaluated at the clamp point -86 gives about 4.4e-38, far below half an
// ulp of 1 (2^-24), so 1 + that rounds to exactly 1, as 1 + 0 does; hence
// clamping the argument into [-86, 88.72] with one med3 and selecting +inf
// above the range reproduces the definition's 1 + exp(x) bit for bit.
__device__ __forceinline__ float one_plus_exp_cw(float x) {
    const float xin = __builtin_amdgcn_fmed3f(x, -86.0f, 88.72f);
    const float v = exp_cw_core(xin);
    return 1.0f + (x > 88.72f ? __builtin_inff() : v);
}

// silu(g) * u with silu(g) = g / (1 + exp(-g)) (one IEEE division), before
// any bf16 rounding: the output-side SwiGLU pass, whose h feeds the int8
// quantizer, so that its codes are reproducible bit for bit.
__device__ __forceinline__ float swiglu_f32(float g, float u) {
    return (g / one_plus_exp_cw(-g)) * u;
}

}  // namespace convrot
