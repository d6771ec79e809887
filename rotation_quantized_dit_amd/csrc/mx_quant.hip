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
// Rounding needs no table: the magnitude code counts the midpoints that |y|
// passes, with >= where the tie goes up to the even code (0.75, 1.75, 3.5)
// and > where it stays at the even code below (0.25, 1.25, 2.5, 5).
#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ uint32_t e2m1_code(float x, float inv_scale) {
    const float y = __builtin_fabsf(x * inv_scale);
    const uint32_t m = (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
                       (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
                       (uint32_t)(y > 5.0f);
    return ((__float_as_uint(x) >> 28) & 8u) | m;
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
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) packed |= e2m1_code(v[e], inv_scale) << (4 * e);
    if (live) {
        *reinterpret_cast<uint32_t*>(codes + row * (k / 2) + col / 2) = packed;
        if ((col & 31) == 0) scales[row * (k / 32) + col / 32] = (uint8_t)scode;
    }
}

template <typename Src>
hipError_t launch(Src src, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
    const int64_t threads = rows * (k / 8);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(mx_quant_kernel<Src>, dim3(grid), dim3(256), 0, stream, src, rows, k, codes, scales);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_quant_bf16(const uint16_t* x, int64_t rows, int64_t k, uint8_t* codes,
                                uint8_t* scales, hipStream_t stream) {
    return launch(Bf16Src{x}, rows, k, codes, scales, stream);
}

hipError_t launch_mx_quant_f32(const float* x, int64_t rows, int64_t k, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
    return launch(F32Src{x}, rows, k, codes, scales, stream);
}

}  // namespace convrot
