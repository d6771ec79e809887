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

// The same h = silu(g) * u, fast, for the output-side pass: the exponential
// and the reciprocal on the transcendental unit.  -log2(e) is split into C_HI
// (15 significant bits, so g * C_HI is exact for every bf16 g) and C_LO ln 2,
// and 2^(g C_LO) is taken to first order (the dropped square term stays below
// 1e-7 relatively wherever the exponential is finite):
//   a = exp2(g C_HI), e = a + a (g C_LO ln 2),
//   d = (1 + e) 2^-64 (one fma: 1 + exp(-g) rounded once, then scaled),
//   h = ((g * rcp(d)) 2^-64) * u.
// The 2^-64 keeps the reciprocal's result normal for every finite d, so the
// quotient g / (1 + exp(-g)) comes out with full precision down to g = -88.5;
// for bf16 g <= -89 exp2 overflows, d = inf and the quotient is -0, as in the
// definition, whose exponential overflows there too.  With exp2 and rcp each
// within 2 ulps, h lies within about 20 fp32 steps (units in the last place
// of its bit pattern) of swiglu_f32(g, u); a CPU model over every finite bf16
// g, with exp2 and rcp pushed 2 ulps off in either direction, never exceeds
// 10.  So whenever the low 16 bits of this h are more than SWIGLU_FAST_MARGIN
// steps from 0x8000 (the bf16 rounding midpoint) and h is finite and below
// 2^127, its bf16 rounding equals that of swiglu_f32(g, u) bit for bit;
// elsewhere (this includes |g| >= 2^64, where g * rcp(d) overflows) the caller
// evaluates swiglu_f32.  Subnormal h needs no exception: fp32 subnormals are
// kept, and both evaluations end in the same multiply by u of a normal (or
// zero) quotient.
constexpr float SWIGLU_C_HI = -0x1.7154p+0f;
constexpr float SWIGLU_C_LO_LN2 = -0x1.480fb6p-18f;
constexpr uint32_t SWIGLU_FAST_MARGIN = 32;
__device__ __forceinline__ float swiglu_fast(float g, float u) {
    const float a = __builtin_amdgcn_exp2f(g * SWIGLU_C_HI);
    const float e = __builtin_fmaf(a, g * SWIGLU_C_LO_LN2, a);
    const float d = __builtin_fmaf(e, 0x1p-64f, 0x1p-64f);
    return ((g * __builtin_amdgcn_rcpf(d)) * 0x1p-64f) * u;
}
// true when the fast value h decides the bf16 rounding of swiglu_f32
__device__ __forceinline__ bool swiglu_fast_ok(float h) {
    const uint32_t low = __float_as_uint(h) & 0xFFFFu;
    const bool far = (low - (0x8000u - SWIGLU_FAST_MARGIN)) > 2u * SWIGLU_FAST_MARGIN;
    return far && __builtin_fabsf(h) < 0x1p127f;
}
// true when the fast value is the definition's h exactly, wherever it lies:
// for bf16 g in [16.75, 2^64), exp(-g) is below 2^-24 (at 16.625, the bf16
// gate below, it is 1 % above), so the definition's 1 + exp(-g) rounds to 1
// and its quotient is g.  The fast e, a few ulps from exp(-g), leaves
// d = 2^-64 exactly there; the reciprocal of a power of two is exact (2^64),
// g 2^64 2^-64 = g below 2^64, and both evaluations round the same product
// g u.  Such products of two bf16 values are often exact bf16 ties, which
// swiglu_fast_ok turns away.
__device__ __forceinline__ bool swiglu_fast_exact(float g) {
    return g >= 16.75f && g < 0x1p64f;
}

}  // namespace convrot
