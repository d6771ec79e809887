// K-ROT: group-wise Hadamard-256 rotation fused with per-row absmax int8
// quantization, for gfx950.
//
// What it computes (cloud-worker RESEARCH.md, "Weight families": ConvRot is a
// group-wise Hadamard rotation written as a convolution; h3-rs README, model
// file table: "int8 per-row + ConvRot (Hadamard-256)"; h3-rs README, "Speed":
// activations are quantized per row with the rotation done inside the
// quantizer):
//   v      = row . blockdiag(H/16) over contiguous groups of 256, fp32 butterfly
//            with spans 1, 2, 4, ..., 128 in that order, each butterfly output
//            one RNE add or subtract;
//   s      = max |v| / 127 (correctly rounded);
//   q      = rint(v / s) with a correctly rounded quotient, half to even.
// The row comes from one of three sources: bf16 activations, fp32 weights
// (load time), or fc1's bf16 gate/up output, from which the source forms
// h = bf16(silu(g) * u) element by element before the rotation (SwiGLU moved
// from fc1's epilogue to the front of the down projection's quantizer).
//
// Layout of the work.  One workgroup per row.  A 256-element group is handled
// by 16 lanes; lane b of the 16 loads the 16 contiguous elements of block b
// (16 * b .. 16 * b + 15), so a wave handles 4 groups per pass with coalesced
// 32-byte (bf16) or 64-byte (fp32) loads.
//   phase 1: spans 1, 2, 4, 8 pair elements inside a block: in registers;
//   transpose the 16 x 16 block matrix through LDS (lane j now holds the
//            elements j, 16 + j, ..., 240 + j);
//   phase 2: spans 16, 32, 64, 128 pair blocks: again in registers.
// The stage order is therefore the same as the textbook order, so the fp32
// results are the same bits.  The rotated row stays in registers until the
// row-wide absmax has been reduced through LDS, then every element is
// quantized; the codes go back through LDS to natural order and leave as one
// 16-byte store per lane.  Rows longer than 128 groups make a second pass that
// recomputes the rotation instead of holding it.
//
// The 1/16 normalization is folded: the butterfly runs unnormalized, the row
// maximum is scaled by 1/16 (exact, and equal to the maximum of the scaled
// values because rounding is monotone), and the reciprocal is scaled by 1/16.
//
// Quotients.  v / s is needed correctly rounded only to decide rint.  The fast
// path computes p = v * RN(1/s) (relative error below 2^-23, so within
// 2.3e-5 of RN(v / s) for |v / s| <= 127); whenever p lies within 2^-14 of a
// half-integer the element takes the exact IEEE division instead, so the code
// always equals rint(RN(v / s)).  Rows with s < 2^-100 take the exact
// division for every element.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fixed_math.h"
#include "fwht.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kMaxPasses = 4;   // groups held in registers per lane-slot

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Streaming loads: each input byte is read once, so they bypass cache reuse.
struct Bf16x16 {    // 16 raw bf16 values
    v4u a, b;
};
__device__ __forceinline__ Bf16x16 fetch16(const uint16_t* __restrict__ p) {
    const v4u* q = reinterpret_cast<const v4u*>(p);
    return Bf16x16{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1)};
}
// bf16 -> fp32 is exact: the bits move to the top half.
__device__ __forceinline__ void widen16(const Bf16x16& r, float v[16]) {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Input sources: how a lane obtains the 16 fp32 values at element offset
// off (a multiple of 16) of row `row` of a k-wide input, in two steps: fetch
// issues the loads into a Raw register block, expand turns it into values.
// The rows kernel fetches every pass of a lane before expanding any, so all
// of a lane's loads are in flight together even when expand branches.
struct Bf16Rows {   // activations, bf16 [rows, k]
    const uint16_t* x;
    typedef Bf16x16 Raw;
    __device__ __forceinline__ Raw fetch(int64_t row, int64_t k, int64_t off) const {
        return fetch16(x + row * k + off);
    }
    __device__ __forceinline__ void expand(const Raw& r, float v[16]) const { widen16(r, v); }
};

struct F32Rows {    // weights, fp32 [rows, k]
    const float* x;
    struct Raw {
        v4f t[4];
    };
    // Ordinary loads here: for fp32 rows they stream about 1.4x faster than
    // the nontemporal form the bf16 sources use (same kernel, 28672 x 5376
    // and 5376 x 14336 weights on MI355X: 5.4-5.5 against 3.9-4.0 TB/s).
    __device__ __forceinline__ Raw fetch(int64_t row, int64_t k, int64_t off) const {
        const v4f* q = reinterpret_cast<const v4f*>(x + row * k + off);
        Raw r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r.t[i] = q[i];
        return r;
    }
    __device__ __forceinline__ void expand(const Raw& r, float v[16]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[4 * i] = r.t[i].x;
            v[4 * i + 1] = r.t[i].y;
            v[4 * i + 2] = r.t[i].z;
            v[4 * i + 3] = r.t[i].w;
        }
    }
};

// SwiGLU on fc1's bf16 output [rows, 2k] (hybrid model card, "Native NVFP4
// projection benchmarks": an "FFN output + SwiGLU" projection): gate columns
// [0, k), up columns [k, 2k), h = bf16(silu(g) * u), widened exactly; the
// rotation then runs on h as on any bf16 activation row.  Each h is first
// evaluated fast (swiglu_fast); only the elements whose fast value lies near
// a bf16 rounding midpoint (or is huge, infinite or NaN) are evaluated again
// by the definition (swiglu_f32), so every bf16 h is the definition's.
struct SwiGluRows {
    const uint16_t* gu;
    struct Raw {
        Bf16x16 g, u;
    };
    __device__ __forceinline__ Raw fetch(int64_t row, int64_t k, int64_t off) const {
        const uint16_t* r = gu + row * 2 * k;
        return Raw{fetch16(r + off), fetch16(r + k + off)};
    }
    __device__ __forceinline__ void expand(const Raw& r, float v[16]) const {
        float g[16], u[16], h[16];
        widen16(r.g, g);
        widen16(r.u, u);
        // Each element's check is a lane mask; the definition runs under
        // it, element by element.  (Collecting the checks into a per-lane
        // bit mask first held 16 more registers and cost a workgroup per
        // CU.)
        bool ok[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            h[e] = swiglu_fast(g[e], u[e]);
            ok[e] = swiglu_fast_ok(h[e]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (!ok[e]) {
                // The empty asm keeps this test inside the rare branch, not
                // hoisted into every element's path.
                float gk = g[e];
                asm volatile("" : "+v"(gk));
                if (!swiglu_fast_exact(gk)) h[e] = swiglu_f32(g[e], u[e]);
            }
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
            const uint32_t b = pack_bf16(h[e], h[e + 1]);
            v[e] = __uint_as_float(b << 16);
            v[e + 1] = __uint_as_float(b & 0xffff0000u);
        }
    }
};

// The exact path of one element: rint of the correctly rounded quotient
// (v_un / 16 is exact), saturated at +-127.
__device__ __forceinline__ float quant_exact(float v_un, float s) {
    const float n = __builtin_rintf((v_un * 0.0625f) / s);
    return __builtin_fminf(__builtin_fmaxf(n, -127.0f), 127.0f);
}

// Quantize one slot's 16 rotated values (elements j + 16 b) and store the
// group's 256 codes in natural order: bytes are staged in the slot's tile and
// read back as one 16-byte chunk per lane (elements 16 j .. 16 j + 15).
// Eight values at a time, the fast products are rounded first; only when one
// of the eight lies within 2^-14 of a half-integer (or the row's scale is
// tiny) does the lane enter the exact path, and there each element makes the
// same test, so every code is rint(RN(v / s)) whichever path it took.  (Eight
// rather than sixteen keeps the rounded values of one half in registers
// without lowering occupancy.)
__device__ __forceinline__ void quant_store(float* tile, int j, const float t[16], float r16,
                                            float s, bool zero, bool exact_all, bool ok,
                                            int8_t* __restrict__ dst) {
    uint8_t* cb = reinterpret_cast<uint8_t*>(tile) + j;
#pragma unroll
    for (int h = 0; h < 16; h += 8) {
        float n[8];
        float dev = 0.0f;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const float p = t[h + b] * r16;
            n[b] = __builtin_rintf(p);
            dev = __builtin_fmaxf(dev, __builtin_fabsf(p - n[b]));
        }
        if (zero) {
#pragma unroll
            for (int b = 0; b < 8; ++b) n[b] = 0.0f;
        } else if (exact_all || dev > 0.5f - 0x1p-14f) {
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const float p = t[h + b] * r16;
                if (exact_all || __builtin_fabsf(p - n[b]) > 0.5f - 0x1p-14f) n[b] = quant_exact(t[h + b], s);
            }
        }
#pragma unroll
        for (int b = 0; b < 8; ++b) cb[(h + b) * 16] = (uint8_t)(int8_t)(int)n[b];
    }
    wave_fence();
    if (ok) {
        const v4u c16 = *reinterpret_cast<const v4u*>(cb - j + j * 16);
        *reinterpret_cast<v4u*>(dst + j * 16) = c16;
    }
    wave_fence();
}

// One workgroup per row; W = blockDim / 64 waves hold 4 groups each per pass
// and P passes of the row in registers; all of a lane's loads are issued
// before any transform.  The row maximum goes through LDS (one workgroup
// barrier per row).
template <typename Src, int P>
__global__ __launch_bounds__(kMaxWaves * 64) void rotate_quant_rows_kernel(
    Src src, int64_t k, int8_t* __restrict__ q, float* __restrict__ s_out) {
    extern __shared__ float smem[];
    __shared__ float red[kMaxWaves];
    const int64_t row = blockIdx.x;
    const int G = (int)(k >> 8);
    const int W = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int sub = lane >> 4;
    const int j = lane & 15;
    int8_t* qr = q + row * k;
    float* tile = smem + wave * kWaveFloats + sub * kTile;

    typename Src::Raw raw[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        if (g < G) raw[p] = src.fetch(row, k, (int64_t)g * 256 + j * 16);
    }
    float vals[P][16];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        if (g < G) {
            src.expand(raw[p], vals[p]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) vals[p][i] = 0.0f;
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        butterfly16(vals[p]);
        transpose_phase2(tile, j, vals[p]);
#pragma unroll
        for (int b = 0; b < 16; ++b) amax = __builtin_fmaxf(amax, __builtin_fabsf(vals[p][b]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < W; ++w) amax = __builtin_fmaxf(amax, red[w]);

    const float s = (amax * 0.0625f) / 127.0f;
    if (threadIdx.x == 0) s_out[row] = s;
    const bool zero = !(s > 0.0f);
    const bool exact_all = !(s >= 0x1p-100f);
    const float r16 = zero ? 0.0f : (1.0f / s) * 0.0625f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        quant_store(tile, j, vals[p], r16, s, zero, exact_all, g < G, qr + (int64_t)g * 256);
    }
}

// Rows longer than 32 W groups: one workgroup per row, the rotation is
// computed twice (once for the row maximum, once to quantize) rather than
// held in registers.
template <typename Src>
__global__ __launch_bounds__(kMaxWaves * 64) void rotate_quant_long_kernel(
    Src src, int64_t k, int passes, int8_t* __restrict__ q, float* __restrict__ s_out) {
    extern __shared__ float smem[];
    __shared__ float red[kMaxWaves];
    const int64_t row = blockIdx.x;
    const int G = (int)(k >> 8);
    const int W = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int sub = lane >> 4;
    const int j = lane & 15;
    int8_t* qr = q + row * k;
    float* tile = smem + wave * kWaveFloats + sub * kTile;

    float amax = 0.0f;
    for (int p = 0; p < passes; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        float t[16];
        if (g < G) {
            src.expand(src.fetch(row, k, (int64_t)g * 256 + j * 16), t);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = 0.0f;
        }
        butterfly16(t);
        transpose_phase2(tile, j, t);
#pragma unroll
        for (int b = 0; b < 16; ++b) amax = __builtin_fmaxf(amax, __builtin_fabsf(t[b]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < W; ++w) amax = __builtin_fmaxf(amax, red[w]);

    const float s = (amax * 0.0625f) / 127.0f;
    if (threadIdx.x == 0) s_out[row] = s;
    const bool zero = !(s > 0.0f);
    const bool exact_all = !(s >= 0x1p-100f);
    const float r16 = zero ? 0.0f : (1.0f / s) * 0.0625f;
    for (int p = 0; p < passes; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        float t[16];
        if (g < G) {
            src.expand(src.fetch(row, k, (int64_t)g * 256 + j * 16), t);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = 0.0f;
        }
        butterfly16(t);
        transpose_phase2(tile, j, t);
        quant_store(tile, j, t, r16, s, zero, exact_all, g < G, qr + (int64_t)g * 256);
    }
}

template <typename Src>
hipError_t launch(Src src, int64_t rows, int64_t k, int8_t* q, float* s, hipStream_t stream) {
    const int G = (int)(k / 256);
    // Register-resident groups per lane-slot: at least two once a row spans
    // more than one wave's four groups (each lane then has two 16-element
    // loads in flight and the row needs half the waves, so more rows fit on a
    // CU: measured 1.8x faster for 21-group rows than one group per slot),
    // and more only when 32 groups per pass would not cover the row.
    int P = (G + 4 * kMaxWaves - 1) / (4 * kMaxWaves);
    if (P == 1 && G > 4) P = 2;
    if (P <= kMaxPasses) {
        const int W = (G + 4 * P - 1) / (4 * P);
        dim3 block(64 * W);
        const size_t lds = (size_t)W * kWaveFloats * sizeof(float);
        dim3 grid((unsigned)rows);
        switch (P) {
            case 1: rotate_quant_rows_kernel<Src, 1><<<grid, block, lds, stream>>>(src, k, q, s); break;
            case 2: rotate_quant_rows_kernel<Src, 2><<<grid, block, lds, stream>>>(src, k, q, s); break;
            case 3: rotate_quant_rows_kernel<Src, 3><<<grid, block, lds, stream>>>(src, k, q, s); break;
            default: rotate_quant_rows_kernel<Src, 4><<<grid, block, lds, stream>>>(src, k, q, s); break;
        }
    } else {
        dim3 grid((unsigned)rows);
        dim3 block(64 * kMaxWaves);
        const size_t lds = (size_t)kMaxWaves * kWaveFloats * sizeof(float);
        rotate_quant_long_kernel<Src><<<grid, block, lds, stream>>>(src, k, P, q, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant_bf16(const uint16_t* x, int64_t rows, int64_t k, int8_t* q,
                                    float* s, hipStream_t stream) {
    return launch(Bf16Rows{x}, rows, k, q, s, stream);
}

hipError_t launch_rotate_quant_f32(const float* x, int64_t rows, int64_t k, int8_t* q, float* s,
                                   hipStream_t stream) {
    return launch(F32Rows{x}, rows, k, q, s, stream);
}

hipError_t launch_swiglu_rotate_quant(const uint16_t* gu, int64_t rows, int64_t i, int8_t* q,
                                      float* s, hipStream_t stream) {
    return launch(SwiGluRows{gu}, rows, i, q, s, stream);
}

}  // namespace convrot
