// Load-time weight operations for gfx950: dequantizing ConvRot weights back to
// the unrotated basis and adding a low-rank (LoRA) delta, so that a LoRA can
// be merged into the int8 weights at load (h3-rs README, "Speed": LoRAs are
// merged at load by dequantizing, adding and requantizing; model file table:
// quantized weights are dequantized per layer by kernels).  Requantization is
// the weight path of the rotate+quantize pass.
//
//   dequantize:  W[n][c] = RN((H q_n / 16)[c] * s[n]) per 256-group; the code
//                rotation is exact in fp32 (every butterfly partial sum is an
//                integer below 2^15), so the multiply is the only rounding.
//   LoRA add:    W[n][c] += scale * sum_j B[n][j] * A[j][c], the sum over j in
//                increasing order as a chain of fused multiply-adds from 0,
//                then one multiply and one add (no contraction: the library is
//                built with -ffp-contract=off).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwht.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

// One 256-group per 16 lanes, 4 groups per wave, 16 per workgroup: lane j
// loads the 16 codes of block j, the butterfly runs on their exact fp32
// values, the scaled results go back through the lane's tile to natural order
// and leave as four 16-byte stores.
__global__ __launch_bounds__(256) void dequantize_weight_kernel(const int8_t* __restrict__ q,
                                                                const float* __restrict__ s,
                                                                int64_t n, int64_t k,
                                                                float* __restrict__ w) {
    __shared__ float tiles[16 * kTile];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int sub = lane >> 4;
    const int j = lane & 15;
    const int64_t G = k >> 8;
    const int64_t gid = (int64_t)blockIdx.x * 16 + wave * 4 + sub;
    const bool ok = gid < n * G;
    const int64_t row = ok ? gid / G : 0;
    const int64_t group_off = row * k + (ok ? gid % G : 0) * 256;
    const int64_t off = group_off + j * 16;
    float* tile = tiles + (wave * 4 + sub) * kTile;

    float v[16];
    if (ok) {
        const v4i c = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(q + off));
        const int cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = (float)(int8_t)(cw[i >> 2] >> (8 * (i & 3)));
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
    butterfly16(v);
    transpose_phase2(tile, j, v);          // lane j now holds elements j + 16 b
    const float sc = ok ? s[row] : 0.0f;
#pragma unroll
    for (int b = 0; b < 16; ++b) tile[b * 17 + j] = (v[b] * 0.0625f) * sc;
    wave_fence();
    // Lane j takes elements 64 i + 4 j .. + 3 (i = 0..3), so that each of
    // the four stores covers 256 contiguous bytes across the 16 lanes of a
    // group: whole cache lines, which the nontemporal stores need (lane j
    // writing its own 64 bytes instead measured 1.8x slower with ordinary
    // stores and 3.5x slower with nontemporal ones).
    float o[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * i + e] = tile[(4 * i + (j >> 2)) * 17 + 4 * (j & 3) + e];
    wave_fence();
    if (ok) {
        v4f* dst = reinterpret_cast<v4f*>(w + group_off + 4 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(v4f{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]}, dst + 16 * i);
    }
}

// W += scale * (B . A): a thread owns 4 consecutive columns of kRows
// consecutive rows, so each 16-byte row of A it loads serves kRows rows.
constexpr int kRows = 8;

__global__ __launch_bounds__(256) void lora_add_kernel(float* __restrict__ w, int64_t n, int64_t k,
                                                       const float* __restrict__ b,
                                                       const float* __restrict__ a, int64_t rank,
                                                       float scale, int64_t col_blocks) {
    const int64_t c0 = ((int64_t)(blockIdx.x % col_blocks) * 256 + threadIdx.x) * 4;
    const int64_t r0 = (int64_t)(blockIdx.x / col_blocks) * kRows;
    if (c0 >= k) return;   // k % 256 == 0, so c0 < k covers all four columns
    // The rows of W this thread updates are loaded first, so that their
    // memory latency overlaps the rank loop.
    v4f x[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
        if (r0 + r < n) x[r] = *reinterpret_cast<const v4f*>(w + (r0 + r) * k + c0);
    float acc[kRows][4];
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[r][e] = 0.0f;
    for (int64_t jj = 0; jj < rank; ++jj) {
        const v4f av = *reinterpret_cast<const v4f*>(a + jj * k + c0);
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            const int64_t row = r0 + r;
            const float bv = row < n ? b[row * rank + jj] : 0.0f;
            acc[r][0] = __builtin_fmaf(bv, av.x, acc[r][0]);
            acc[r][1] = __builtin_fmaf(bv, av.y, acc[r][1]);
            acc[r][2] = __builtin_fmaf(bv, av.z, acc[r][2]);
            acc[r][3] = __builtin_fmaf(bv, av.w, acc[r][3]);
        }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int64_t row = r0 + r;
        if (row >= n) break;
        v4f y = x[r];
        y.x = y.x + scale * acc[r][0];
        y.y = y.y + scale * acc[r][1];
        y.z = y.z + scale * acc[r][2];
        y.w = y.w + scale * acc[r][3];
        // (the rows are written once here; a wave's 64 stores are 1 KiB
        // contiguous, and the nontemporal form measured 5 % faster)
        __builtin_nontemporal_store(y, reinterpret_cast<v4f*>(w + row * k + c0));
    }
}

}  // namespace

hipError_t launch_dequantize_weight(const int8_t* q, const float* s, int64_t n, int64_t k,
                                    float* w, hipStream_t stream) {
    const int64_t groups = n * (k / 256);
    dim3 grid((unsigned)((groups + 15) / 16));
    dequantize_weight_kernel<<<grid, dim3(256), 0, stream>>>(q, s, n, k, w);
    return hipGetLastError();
}

hipError_t launch_lora_add(float* w, int64_t n, int64_t k, const float* b, const float* a,
                           int64_t rank, float scale, hipStream_t stream) {
    const int64_t col_blocks = (k / 4 + 255) / 256;
    dim3 grid((unsigned)(col_blocks * ((n + kRows - 1) / kRows)));
    lora_add_kernel<<<grid, dim3(256), 0, stream>>>(w, n, k, b, a, rank, scale, col_blocks);
    return hipGetLastError();
}

}  // namespace convrot
