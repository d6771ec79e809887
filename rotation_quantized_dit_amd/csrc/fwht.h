// The Hadamard-256 butterfly as the rotate passes run it: a 256-element
// group is held by 16 lanes, lane j starting with elements 16 j .. 16 j + 15.
// Spans 1, 2, 4, 8 run in registers, a 16 x 16 transpose through a
// wave-private LDS tile follows, then spans 16 .. 128 in registers; the stage
// order is the textbook ascending order, so fp32 results are the same bits.
#pragma once

#include <hip/hip_runtime.h>

namespace convrot {

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

// LDS per wave: four 16 x 17 fp32 transpose tiles, one per 256-element
// group the wave holds at a time (the 17th column pads the banks: tiles sit
// 272 words apart, i.e. 16 banks apart modulo 64); a pass may reuse it
// afterwards (to stage codes or outputs).  Transposes are private to one wave, and a
// wave executes its LDS instructions in order, so they need no workgroup
// barrier, only a compiler fence.
inline constexpr int kTile = 16 * 17;
inline constexpr int kWaveFloats = 4 * kTile;

__device__ __forceinline__ void wave_fence() {
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Phase 2 of the butterfly for the 16 values of one lane-slot, after phase 1
// ran on its contiguous block: transpose through the slot's tile, then spans
// 16..128.  Returns the rotated (unnormalized) values of elements
// j, 16 + j, ..., 240 + j.
__device__ __forceinline__ void transpose_phase2(float* tile, int j, float v[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[j * 17 + i] = v[i];
    wave_fence();
#pragma unroll
    for (int b = 0; b < 16; ++b) v[b] = tile[b * 17 + j];
    wave_fence();
    butterfly16(v);
}

}  // namespace convrot
