// MXFP4 quantization of rows (activations in bf16, weights in fp32), for
// the MXFP4 analog of the hybrid layers (Minimax_h3_hybrid model card,
// "Checkpoints": QKV and the FFN input in a 4-bit block format, the output
// projections int8 ConvRot).
//
// Per block of 32 consecutive elements of a row (OCP Microscaling MXFP4):
//   e      = floor(log2(max |v|)) - 2, clamped to [-127, 127]; stored as the
//            E8M0 code e + 127 (an all-zero block gets code 0);
//   y      = v * 2^-e (exact);
//   code   = sign bit of v | the E2M1 magnitude code of |y| rounded to the
//            nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 (ties to the even
//            mantissa bit, saturating at 6);
//   packed: element 2j in the low nibble of byte j.
// Scales are stored chunk-major, as the GEMM streams them: the scale of block
// b of row r (of `rows`) is byte (b / 4) * rows * 4 + r * 4 + b % 4, i.e. a
// [k/128][rows][4] array, so that the four scales of one 128-element chunk of
// consecutive rows are contiguous.
// The rounding is gfx950's FP4 conversion (v_cvt_scalef32_pk_fp4_f32, with a
// scale of 1 on the exactly scaled y): it rounds to the nearest E2M1 value,
// ties to the even mantissa bit, saturates at 6 and keeps the sign of zero.
// A probe of the instruction against that definition (every 1/64 step of
// [-8, 8], each midpoint 0.25 ... 5 and its neighbours, +-0, denormals,
// saturating values and scales 2^-126 ... 2^127) matched on all 3675 pairs;
// the parity tests compare every code with the oracle's.
//
// Rotated variant: the rows are first rotated along K with the orthonormal
// Hadamard of size 256, group by group, exactly as the int8 ConvRot
// quantizer rotates them (the same butterfly, stage order and 1/16), and the
// rotated values are then quantized as above.  Rotating both operands keeps
// their product unchanged, and spreads the outlier channels that would
// otherwise set the scale of their whole 32-element block.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwht.h"
#include "kernels.h"

namespace convrot {
namespace {

struct Bf16Src {
    const uint16_t* p;
    __device__ __forceinline__ void load8(int64_t off, float v[8]) const {
        const uint4 raw = *reinterpret_cast<const uint4*>(p + off);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = __uint_as_float(w[e] << 16);
            v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
};

struct F32Src {
    const float* p;
    __device__ __forceinline__ void load8(int64_t off, float v[8]) const {
        const float4 a = *reinterpret_cast<const float4*>(p + off);
        const float4 b = *reinterpret_cast<const float4*>(p + off + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// Two values already scaled into the E2M1 range -> byte SEL of `old` (the
// first value in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack(uint32_t old, float y0, float y1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, y0, y1, 1.0f, SEL);
}

// One thread per 8 elements; 4 consecutive threads form a 32-element block.
template <typename Src>
__global__ __launch_bounds__(256) void mx_quant_kernel(Src src, int64_t rows, int64_t k,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_row = k / 8;
    const bool live = t < rows * per_row;
    const int64_t tt = live ? t : rows * per_row - 1;   // keep every lane in the shuffles
    const int64_t row = tt / per_row;
    const int64_t col = (tt - row * per_row) * 8;
    float v[8];
    src.load8(row * k + col, v);
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 2, 64));
    // E8M0 code = e + 127 = biased exponent of amax - 2, clamped at 0 (a
    // zero or denormal amax has floor(log2) <= -127 and clamps to e = -127)
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    const int scode = ef >= 2 ? ef - 2 : 0;
    // 2^-e = 2^(127 - scode), a normal float for scode in [0, 252]
    const float inv_scale = __uint_as_float((uint32_t)(254 - scode) << 23);
    // y = v * 2^-e is exact (a normal power of two, no overflow since |y| < 8)
    uint32_t packed = 0;
    packed = e2m1_pack<0>(packed, v[0] * inv_scale, v[1] * inv_scale);
    packed = e2m1_pack<1>(packed, v[2] * inv_scale, v[3] * inv_scale);
    packed = e2m1_pack<2>(packed, v[4] * inv_scale, v[5] * inv_scale);
    packed = e2m1_pack<3>(packed, v[6] * inv_scale, v[7] * inv_scale);
    if (live) {
        *reinterpret_cast<uint32_t*>(codes + row * (k / 2) + col / 2) = packed;
        if ((col & 31) == 0) {
            const int64_t b = col / 32;
            scales[(b >> 2) * rows * 4 + row * 4 + (b & 3)] = (uint8_t)scode;
        }
    }
}

// Rotated variant: one 256-group per 16 lanes (4 per wave, 16 per
// workgroup).  Lane j loads elements 16 j .. 16 j + 15, the butterfly runs as
// in the rotate pass, and the normalized results go back through the lane's
// tile to natural order; lanes 2p and 2p + 1 then hold one 32-element block.
template <typename Src>
__global__ __launch_bounds__(256) void rot_mx_quant_kernel(Src src, int64_t rows, int64_t k,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales) {
    __shared__ float tiles[16 * kTile];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane >> 4;
    const int j = lane & 15;
    const int64_t G = k >> 8;
    const int64_t gid = (int64_t)blockIdx.x * 16 + wave * 4 + sub;
    const bool ok = gid < rows * G;
    const int64_t row = ok ? gid / G : 0;
    const int64_t col = (ok ? gid % G : 0) * 256 + j * 16;
    float* tile = tiles + (wave * 4 + sub) * kTile;

    float v[16];
    if (ok) {
        src.load8(row * k + col, v);
        src.load8(row * k + col + 8, v + 8);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    butterfly16(v);
    transpose_phase2(tile, j, v);          // lane j: rotated elements j + 16 b (unnormalized)
#pragma unroll
    for (int b = 0; b < 16; ++b) tile[b * 17 + j] = v[b] * 0.0625f;
    wave_fence();
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = tile[j * 17 + i];   // elements 16 j .. 16 j + 15
    wave_fence();
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[e]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1, 64));
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
    const int scode = ef >= 2 ? ef - 2 : 0;
    const float inv_scale = __uint_as_float((uint32_t)(254 - scode) << 23);
    uint32_t lo = 0, hi = 0;
    lo = e2m1_pack<0>(lo, v[0] * inv_scale, v[1] * inv_scale);
    lo = e2m1_pack<1>(lo, v[2] * inv_scale, v[3] * inv_scale);
    lo = e2m1_pack<2>(lo, v[4] * inv_scale, v[5] * inv_scale);
    lo = e2m1_pack<3>(lo, v[6] * inv_scale, v[7] * inv_scale);
    hi = e2m1_pack<0>(hi, v[8] * inv_scale, v[9] * inv_scale);
    hi = e2m1_pack<1>(hi, v[10] * inv_scale, v[11] * inv_scale);
    hi = e2m1_pack<2>(hi, v[12] * inv_scale, v[13] * inv_scale);
    hi = e2m1_pack<3>(hi, v[14] * inv_scale, v[15] * inv_scale);
    if (ok) {
        *reinterpret_cast<uint2*>(codes + row * (k / 2) + col / 2) = make_uint2(lo, hi);
        if ((j & 1) == 0) {
            const int64_t b = col / 32;
            scales[(b >> 2) * rows * 4 + row * 4 + (b & 3)] = (uint8_t)scode;
        }
    }
}

template <typename Src>
hipError_t launch_rot(Src src, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales,
                      hipStream_t stream) {
    const int64_t groups = rows * (k / 256);
    const unsigned grid = (unsigned)((groups + 15) / 16);
    hipLaunchKernelGGL(rot_mx_quant_kernel<Src>, dim3(grid), dim3(256), 0, stream, src, rows, k, codes,
                       scales);
    return hipGetLastError();
}

template <typename Src>
hipError_t launch(Src src, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    const int64_t threads = rows * (k / 8);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(mx_quant_kernel<Src>, dim3(grid), dim3(256), 0, stream, src, rows, k, codes, scales);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quant_bf16(const uint16_t* x, int64_t rows, int64_t k, bool rotate, uint8_t* codes,
                                uint8_t* scales, hipStream_t stream) {
    return rotate ? launch_rot(Bf16Src{x}, rows, k, codes, scales, stream)
                  : launch(Bf16Src{x}, rows, k, codes, scales, stream);
}

hipError_t launch_mx_quant_f32(const float* x, int64_t rows, int64_t k, bool rotate, uint8_t* codes,
                               uint8_t* scales, hipStream_t stream) {
    return rotate ? launch_rot(F32Src{x}, rows, k, codes, scales, stream)
                  : launch(F32Src{x}, rows, k, codes, scales, stream);
}

}  // namespace convrot
