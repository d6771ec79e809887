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

#include "kernels.h"

namespace convrot {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kMaxPasses = 4;   // groups held in registers per lane-slot

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Streaming loads: each input byte is read once, so they bypass cache reuse.
__device__ __forceinline__ void load16(const uint16_t* __restrict__ p, float v[16]) {
    const v4u* q = reinterpret_cast<const v4u*>(p);
    v4u a = __builtin_nontemporal_load(q);
    v4u b = __builtin_nontemporal_load(q + 1);
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

__device__ __forceinline__ void load16(const float* __restrict__ p, float v[16]) {
    const v4f* q = reinterpret_cast<const v4f*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v4f t = __builtin_nontemporal_load(q + i);
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
    }
}

// Four butterfly stages on 16 registers: spans 1, 2, 4, 8 of the index.
__device__ __forceinline__ void butterfly16(float v[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i & h) continue;
            float a = v[i];
            float b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
}

struct Smem {
    float tr[kMaxWaves][4][16][17];     // per-wave 16 x 16 transposes, padded
    uint8_t codes[kMaxWaves][4][256];   // per-wave code staging
    float red[kMaxWaves];
};

template <typename Tin>
__device__ __forceinline__ void rotate_group(const Tin* __restrict__ xr, int g, bool ok, int wave,
                                             int sub, int j, Smem& sm, float out[16]) {
    float v[16];
    if (ok) {
        load16(xr + (int64_t)g * 256 + j * 16, v);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    butterfly16(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.tr[wave][sub][j][i] = v[i];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 16; ++b) out[b] = sm.tr[wave][sub][b][j];
    __syncthreads();
    butterfly16(out);
}

__device__ __forceinline__ int quant_one(float v_un, float r16, float s, bool exact_all) {
    float p = v_un * r16;
    float n = __builtin_rintf(p);
    if (exact_all || __builtin_fabsf(p - n) > 0.5f - 0x1p-14f) {
        n = __builtin_rintf((v_un * 0.0625f) / s);
        n = __builtin_fminf(__builtin_fmaxf(n, -127.0f), 127.0f);
    }
    return (int)n;
}

// P = groups per lane-slot held in registers (two-pass when TWO_PASS).
template <typename Tin, int P, bool TWO_PASS>
__global__ __launch_bounds__(kMaxWaves * 64) void rotate_quant_kernel(
    const Tin* __restrict__ x, int64_t k, int passes, int8_t* __restrict__ q,
    float* __restrict__ s_out) {
    __shared__ Smem sm;
    const int64_t row = blockIdx.x;
    const int G = (int)(k >> 8);
    const int W = blockDim.x >> 6;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int sub = lane >> 4;
    const int j = lane & 15;
    const Tin* xr = x + row * k;

    float vals[P][16];
    float amax = 0.0f;
    const int npass = TWO_PASS ? passes : P;
    for (int p = 0; p < npass; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        const bool ok = g < G;
        float t[16];
        rotate_group(xr, g, ok, wave, sub, j, sm, t);
#pragma unroll
        for (int b = 0; b < 16; ++b) amax = __builtin_fmaxf(amax, __builtin_fabsf(t[b]));
        if (!TWO_PASS) {
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
                if (pp == p) {
#pragma unroll
                    for (int b = 0; b < 16; ++b) vals[pp][b] = t[b];
                }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = __builtin_fmaxf(amax, __shfl_xor(amax, off, 64));
    if (lane == 0) sm.red[wave] = amax;
    __syncthreads();
    amax = sm.red[0];
    for (int w = 1; w < W; ++w) amax = __builtin_fmaxf(amax, sm.red[w]);

    const float s = (amax * 0.0625f) / 127.0f;
    if (threadIdx.x == 0) s_out[row] = s;
    const bool zero = !(s > 0.0f);
    const bool exact_all = !(s >= 0x1p-100f);
    const float r16 = zero ? 0.0f : (1.0f / s) * 0.0625f;

    for (int p = 0; p < npass; ++p) {
        const int g = (p * W + wave) * 4 + sub;
        const bool ok = g < G;
        float t[16];
        if (TWO_PASS) {
            rotate_group(xr, g, ok, wave, sub, j, sm, t);
        } else {
#pragma unroll
            for (int pp = 0; pp < P; ++pp)
                if (pp == p) {
#pragma unroll
                    for (int b = 0; b < 16; ++b) t[b] = vals[pp][b];
                }
        }
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            int c = zero ? 0 : quant_one(t[b], r16, s, exact_all);
            sm.codes[wave][sub][b * 16 + j] = (uint8_t)(int8_t)c;
        }
        __syncthreads();
        if (ok) {
            uint4 c16 = *reinterpret_cast<const uint4*>(&sm.codes[wave][sub][j * 16]);
            *reinterpret_cast<uint4*>(q + row * k + (int64_t)g * 256 + j * 16) = c16;
        }
        __syncthreads();
    }
}

template <typename Tin>
hipError_t launch(const Tin* x, int64_t rows, int64_t k, int8_t* q, float* s, hipStream_t stream) {
    const int G = (int)(k / 256);
    // Prefer the fewest register-resident groups per slot, then the fewest waves.
    int P = (G + 4 * kMaxWaves - 1) / (4 * kMaxWaves);
    dim3 grid((unsigned)rows);
    if (P <= kMaxPasses) {
        int W = (G + 4 * P - 1) / (4 * P);
        dim3 block(64 * W);
        switch (P) {
            case 1: rotate_quant_kernel<Tin, 1, false><<<grid, block, 0, stream>>>(x, k, 1, q, s); break;
            case 2: rotate_quant_kernel<Tin, 2, false><<<grid, block, 0, stream>>>(x, k, 2, q, s); break;
            case 3: rotate_quant_kernel<Tin, 3, false><<<grid, block, 0, stream>>>(x, k, 3, q, s); break;
            default: rotate_quant_kernel<Tin, 4, false><<<grid, block, 0, stream>>>(x, k, 4, q, s); break;
        }
    } else {
        dim3 block(64 * kMaxWaves);
        rotate_quant_kernel<Tin, 1, true><<<grid, block, 0, stream>>>(x, k, P, q, s);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant_bf16(const uint16_t* x, int64_t rows, int64_t k, int8_t* q,
                                    float* s, hipStream_t stream) {
    return launch(x, rows, k, q, s, stream);
}

hipError_t launch_rotate_quant_f32(const float* x, int64_t rows, int64_t k, int8_t* q, float* s,
                                   hipStream_t stream) {
    return launch(x, rows, k, q, s, stream);
}

}  // namespace convrot
