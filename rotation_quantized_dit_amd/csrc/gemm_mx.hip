// MXFP4 x MXFP4 -> fp32 GEMM with a bf16 epilogue on the gfx950 scaled
// MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, both operands FP4 E2M1), for the
// MXFP4 analog of the hybrid layers (Minimax_h3_hybrid model card,
// "Checkpoints": QKV and the FFN input in a 4-bit block format).
//
//   y[m][n] = bf16_rne( sum_k a[m][k] b[n][k] ),  a = A code * 2^(A scale of
//   its 32-block), likewise b; the hardware applies both block scales inside
//   the MFMA and accumulates in fp32.
//
// Operands: codes [rows, K/2] bytes (element 2j in the low nibble of byte j)
// and E8M0 scales chunk-major, [K/128][rows][4] bytes (the 4 block scales of
// one 128-element chunk of consecutive rows are contiguous).  In bytes, a
// 64-element k-step of FP4 occupies 32 bytes of a row and each lane takes 16
// of them (lanes 0-31 the first 32 elements, lanes 32-63 the next 32),
// exactly the layout of the int8 operands of K-GEMM, so the tiling is that
// kernel's: a 384 x 256 tile, 8 waves (two per SIMD) in a 4 x 2 grid of
// 96 x 128 wave tiles (3 x 4 MFMA blocks, 192 fp32 accumulators per lane),
// 64 bytes (128 elements) of K per stage through a 3-slot LDS ring of direct
// buffer loads, XOR-swizzled 64-byte rows, one fragment set per k-step.
// The 96 x 128 wave tile reads 7 fragments per 12 MFMAs (against 6 per 8
// for 64 x 128) and the 384-row tile copies 17 % fewer bytes per flop than a
// 256-row one; both measured about 8 % faster on the FFN-input shape.
//
// Each stage also carries the tile's scale words (one 32-bit word per row:
// the 4 block scales of its 128 elements), 384 + 256 words copied as three
// 1 KiB direct loads: waves 0 and 1 take the A rows (the upper half of wave
// 1's copy reads rows past the tile into unused space), wave 2 the B rows.
// So that the copy needs no branch, waves 3-7 issue the same load on an
// empty buffer resource (every lane out of range: no memory is read) into a
// spare 1 KiB of LDS.  For k-step s a lane reads the one byte it needs,
// block 2 s + lane / 32 of its row, with a byte load from LDS.
//
// Ragged rows are clamped to the last row for loading and masked at the
// store; K must be a multiple of 128.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fixed_math.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int BM = 384;
constexpr int BN = 256;
constexpr int BK = 64;                       // bytes of codes per row per stage (128 elements)
constexpr int MA = BM / 128;                 // 32-row A blocks per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int SA_BYTES = 2048;               // 384 A scale words (+ the unused half of the second copy)
constexpr int SB_BYTES = 1024;               // 256 B scale words
constexpr int STAGE_BYTES = A_STAGE + B_STAGE + SA_BYTES + SB_BYTES;
constexpr int STAGES = 3;
constexpr int COPIES = MA + 3;               // per wave per stage: A, B and one scale copy
constexpr int SPARE = STAGES * STAGE_BYTES;  // 1 KiB that the idle scale copies fill
constexpr int PITCH = 136;
constexpr int STASH_WAVE_BYTES = 32 * PITCH * 4;
constexpr int STASH_BYTES = NWAVES * STASH_WAVE_BYTES;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = RING_BYTES > STASH_BYTES ? RING_BYTES : STASH_BYTES;
constexpr int GROUP_M = 4;                   // M-tiles per raster group
static_assert(SPARE + 1024 <= LDS_BYTES, "spare area");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rsrc, uint8_t* dst, uint32_t voff,
                                       uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voff, soff, 0, 0);
#endif
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

struct Tile {
    int tm, tn;
};

__device__ __forceinline__ Tile map_tile(int b, int MT, int NT) {
    const int T = MT * NT;
    const int xcd = b & 7;
    const int j = b >> 3;
    const int base = T >> 3, rem = T & 7;
    const int t = xcd * base + (xcd < rem ? xcd : rem) + j;
    const int group = t / (GROUP_M * NT);
    const int first_m = group * GROUP_M;
    const int gm = (MT - first_m) < GROUP_M ? (MT - first_m) : GROUP_M;
    const int within = t - group * GROUP_M * NT;
    return Tile{first_m + within % gm, within / gm};
}

__global__ __launch_bounds__(NTHREADS, 1) void gemm_mx_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int M, int N, int K, uint16_t* __restrict__ out, int MT, int NT) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const Tile tile = map_tile(blockIdx.x, MT, NT);
    const int m0 = tile.tm * BM;
    const int n0 = tile.tn * BN;
    const int rows_a = (M - m0) < BM ? (M - m0) : BM;
    const int rows_b = (N - n0) < BN ? (N - n0) : BN;
    const int KB = K / 2;
    const int KT = K / 128;

    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(A + (int64_t)m0 * KB, (uint32_t)rows_a * (uint32_t)KB);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(B + (int64_t)n0 * KB, (uint32_t)rows_b * (uint32_t)KB);
    // scale copies: waves 0 and 1 the tile's A scale words (rows 256 w + 4 l .. +3; the upper half of
    // wave 1's copy reads rows past the tile into the unused end of the A scale area), wave 2 the B
    // words; waves 3-7 issue the same instruction on an empty resource into a spare area (no branch)
    const __amdgpu_buffer_rsrc_t rsrc_s =
        wave < 2 ? make_rsrc(SA + (int64_t)m0 * 4, (uint32_t)((int64_t)(KT - 1) * M * 4 + rows_a * 4))
        : wave == 2 ? make_rsrc(SB + (int64_t)n0 * 4, (uint32_t)((int64_t)(KT - 1) * N * 4 + rows_b * 4))
                    : make_rsrc(SB, 0u);
    const uint32_t chunk_stride = wave < 2 ? (uint32_t)M * 4u : wave == 2 ? (uint32_t)N * 4u : 0u;
    const uint32_t voff_s = (uint32_t)(wave < 2 ? 1024 * wave : 0) + 16u * (uint32_t)lane;
    const int s_dst = wave < 2 ? A_STAGE + B_STAGE + 1024 * wave
                      : wave == 2 ? A_STAGE + B_STAGE + SA_BYTES : SPARE;
    uint32_t voff[MA + 2];
#pragma unroll
    for (int i = 0; i < MA + 2; ++i) {
        const int rr = i < MA ? 16 * (MA * wave + i) + (lane >> 2) : 32 * wave + 16 * (i - MA) + (lane >> 2);
        const int lim = i < MA ? rows_a : rows_b;
        const int src_row = rr < lim ? rr : lim - 1;
        voff[i] = (uint32_t)src_row * (uint32_t)KB + 16u * (uint32_t)((lane & 3) ^ swz(rr));
    }
    auto issue = [&](int kt, int slot) {
        uint8_t* st = lds + slot * STAGE_BYTES;
        const uint32_t soff = (uint32_t)kt * BK;
#pragma unroll
        for (int i = 0; i < MA; ++i) copy16(rsrc_a, st + 16 * 64 * MA * wave + 1024 * i, voff[i], soff);
        copy16(rsrc_b, st + A_STAGE + 32 * 64 * wave, voff[MA], soff);
        copy16(rsrc_b, st + A_STAGE + 32 * 64 * wave + 1024, voff[MA + 1], soff);
        copy16(rsrc_s, (wave < 3 ? st : lds) + s_dst, voff_s, (uint32_t)kt * chunk_stride);
    };

    v16f acc[MA][4];
#pragma unroll
    for (int a = 0; a < MA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    // Per-lane byte offsets within a stage.  The swizzle of every fragment
    // row of a lane is (lane >> 2) & 3 (the rows differ by multiples of 32),
    // so each operand needs one lane offset per k-step, the blocks following
    // at fixed distances (2048 bytes per 32 code rows, 128 per 32 scale words).
    const int sw = (lane >> 2) & 3;
    const int a_lane = (32 * MA * wm + (lane & 31)) * BK;
    const int b_lane = A_STAGE + (128 * wn + (lane & 31)) * BK;
    const int sa_lane = A_STAGE + B_STAGE + 4 * (32 * MA * wm + (lane & 31)) + g;
    const int sb_lane = A_STAGE + B_STAGE + SA_BYTES + 4 * (128 * wn + (lane & 31)) + g;
    auto read_frags = [&](const uint8_t* st, int s, v4i (&af)[MA], v4i (&bf)[4], int (&sa)[MA], int (&sb)[4]) {
        const int c = 16 * ((2 * s + g) ^ sw);
        const uint8_t* pa = st + (a_lane + c);
        const uint8_t* pb = st + (b_lane + c);
#pragma unroll
        for (int a = 0; a < MA; ++a) af[a] = *reinterpret_cast<const v4i*>(pa + 2048 * a);
#pragma unroll
        for (int b = 0; b < 4; ++b) bf[b] = *reinterpret_cast<const v4i*>(pb + 2048 * b);
        const uint8_t* psa = st + sa_lane;
        const uint8_t* psb = st + sb_lane;
#pragma unroll
        for (int a = 0; a < MA; ++a) sa[a] = psa[128 * a + 2 * s];
#pragma unroll
        for (int b = 0; b < 4; ++b) sb[b] = psb[128 * b + 2 * s];
    };
    auto mma = [&](const v4i (&af)[MA], const v4i (&bf)[4], const int (&sa)[MA], const int (&sb)[4]) {
#pragma unroll
        for (int a = 0; a < MA; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const v8i av = {af[a].x, af[a].y, af[a].z, af[a].w, 0, 0, 0, 0};
                const v8i bv = {bf[b].x, bf[b].y, bf[b].z, bf[b].w, 0, 0, 0, 0};
                acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[a][b], 4, 4, 0, sa[a], 0,
                                                                            sb[b]);
            }
    };

#pragma unroll
    for (int st = 0; st < STAGES; ++st)
        if (st < KT) issue(st, st);
    {
        const int ahead = (KT - 1) < (STAGES - 1) ? (KT - 1) : (STAGES - 1);
        if (ahead >= 2) wait_vmcnt<2 * COPIES>();
        else if (ahead == 1) wait_vmcnt<COPIES>();
        else wait_vmcnt<0>();
    }
    lds_barrier();

    int slot = 0;
    int kt = 0;
    v4i fa[MA], fb[4];
    int sa[MA], sb[4];
    // Steady state (a refill per stage) as straight-line code, so that the
    // scheduling barriers hold the order: k-step 0's reads and MFMAs, k-step
    // 1's reads, the wait for stage kt + 1 and the barrier, the refill, k-step
    // 1's MFMAs.
    for (; kt + STAGES < KT; ++kt) {
        const int next = slot + 1 == STAGES ? 0 : slot + 1;
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + slot * STAGE_BYTES, 0, fa, fb, sa, sb);
        mma(fa, fb, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + slot * STAGE_BYTES, 1, fa, fb, sa, sb);
        wait_vmcnt<COPIES>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + STAGES, slot);
        mma(fa, fb, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
        slot = next;
    }
    for (; kt < KT; ++kt) {
        const int next = slot + 1 == STAGES ? 0 : slot + 1;
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + slot * STAGE_BYTES, 0, fa, fb, sa, sb);
        mma(fa, fb, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + slot * STAGE_BYTES, 1, fa, fb, sa, sb);
        wait_vmcnt<0>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        mma(fa, fb, sa, sb);
        __builtin_amdgcn_sched_barrier(0);
        slot = next;
    }

    lds_barrier();
    float* stash = reinterpret_cast<float*>(lds + wave * STASH_WAVE_BYTES);
    const int grow0 = m0 + 32 * MA * wm;
    const int cg = lane % 16, ro = lane / 16;
    const int col0 = n0 + 128 * wn + 8 * cg;
    const bool vec_cols = (col0 + 8 <= N) && (N % 8 == 0);
#pragma unroll
    for (int a = 0; a < MA; ++a) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                stash[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * PITCH + 32 * b + (lane & 31)] = acc[a][b][r];
        asm volatile("" ::: "memory");
#pragma nounroll
        for (int it = 0; it < 8; ++it) {
            const int lr = 4 * it + ro;
            const int grow = grow0 + 32 * a + lr;
            const v4f a0 = *reinterpret_cast<const v4f*>(stash + lr * PITCH + 8 * cg);
            const v4f a1 = *reinterpret_cast<const v4f*>(stash + lr * PITCH + 8 * cg + 4);
            if (grow >= M) continue;
            const v4u pk = {pack_bf16(a0.x, a0.y), pack_bf16(a0.z, a0.w), pack_bf16(a1.x, a1.y),
                            pack_bf16(a1.z, a1.w)};
            if (vec_cols) {
                *reinterpret_cast<v4u*>(out + (int64_t)grow * N + col0) = pk;
            } else {
                const uint32_t pw[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (col0 + e < N) out[(int64_t)grow * N + col0 + e] = (uint16_t)(pw[e >> 1] >> (16 * (e & 1)));
            }
        }
        asm volatile("" ::: "memory");
    }
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, uint16_t* out,
                          hipStream_t stream) {
    const int MT = (int)((m + BM - 1) / BM);
    const int NT = (int)((n + BN - 1) / BN);
    hipLaunchKernelGGL(gemm_mx_kernel, dim3((unsigned)(MT * NT)), dim3(NTHREADS), 0, stream, a_codes,
                       a_scales, b_codes, b_scales, (int)m, (int)n, (int)k, out, MT, NT);
    return hipGetLastError();
}

}  // namespace convrot
