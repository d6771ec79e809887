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
// one 128-element chunk of consecutive rows are contiguous).  In bytes, a 64-element k-step of FP4
// occupies 32 bytes of a row and each lane takes 16 of them (lanes 0-31 the
// first 32 elements, lanes 32-63 the next 32), exactly the layout of the
// int8 operands of K-GEMM; so the tiling below is that kernel's 256-row
// variant: a 256 x 256 tile, 8 waves (two per SIMD) in a 4 x 2 grid of
// 64 x 128 wave tiles, 64 bytes (128 elements) of K per stage through a
// 4-slot LDS ring of direct buffer loads, XOR-swizzled 64-byte rows.
// Each stage also carries one 32-bit word per tile row: the 4 block scales
// of that row's 128 elements, copied by 4-byte direct loads (one per wave:
// waves 0-3 the 256 A rows, waves 4-7 the 256 B rows), 256 contiguous bytes
// per copy in the chunk-major layout (row-major scales would put each lane's
// word in a different cache line, which measured 30 % slower).  For k-step s a lane
// reads the one byte it needs, block 2 s + lane / 32 of its row, with a byte
// load from LDS, so the scale operand needs no vector instruction.
//
// Ragged rows are clamped to the last row for loading and masked at the
// store; K must be a multiple of 128.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fixed_math.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;                       // bytes of codes per row per stage (128 elements)
constexpr int MA = BM / 128;                 // 32-row A blocks per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int S_STAGE = 4 * (BM + BN);       // scale words
constexpr int STAGE_BYTES = A_STAGE + B_STAGE + S_STAGE;
constexpr int STAGES = 4;
constexpr int COPIES = MA + 2 + 1;           // per wave per stage: A, B and one scale copy
constexpr int PITCH = 136;
constexpr int STASH_WAVE_BYTES = 32 * PITCH * 4;
constexpr int STASH_BYTES = NWAVES * STASH_WAVE_BYTES;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = RING_BYTES > STASH_BYTES ? RING_BYTES : STASH_BYTES;
constexpr int GROUP_M = 8;
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

// Hardware barrier for the ring (copies completed by the preceding vmcnt
// wait, this wave's LDS reads by lgkmcnt(0)).
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
__device__ __forceinline__ void copy4(__amdgpu_buffer_rsrc_t rsrc, uint8_t* dst, uint32_t voff,
                                      uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 4, voff, soff, 0, 0);
#endif
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

struct Tile {
    int tm, tn;
};

// Tile ids dealt round-robin to the 8 XCDs are remapped so that each XCD
// walks a contiguous range of a grouped raster (GROUP_M row tiles per group).
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
    const int KB = K / 2;                    // code bytes per row

    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(A + (int64_t)m0 * KB, (uint32_t)rows_a * (uint32_t)KB);
    const __amdgpu_buffer_rsrc_t rsrc_b = make_rsrc(B + (int64_t)n0 * KB, (uint32_t)rows_b * (uint32_t)KB);
    // scales of this tile's rows: chunk kt at byte kt * rows_total * 4 from
    // the tile's first row (the resource spans every chunk of those rows)
    const int KT_ = K / 128;
    const __amdgpu_buffer_rsrc_t rsrc_s =
        wave < 4 ? make_rsrc(SA + (int64_t)m0 * 4, (uint32_t)((int64_t)(KT_ - 1) * M * 4 + rows_a * 4))
                 : make_rsrc(SB + (int64_t)n0 * 4, (uint32_t)((int64_t)(KT_ - 1) * N * 4 + rows_b * 4));
    const uint32_t chunk_stride = (uint32_t)(wave < 4 ? M : N) * 4u;

    // Copy sources: copy i < MA of wave w fills A rows 16 (MA w + i) .. +15,
    // copies MA, MA + 1 fill B rows 32 w + 16 (i - MA) .. +15 (lane l: row
    // l / 4 of the 16, chunk position l % 4 holding logical chunk
    // (l % 4) ^ swz(row)); the scale copy of wave w takes row 64 (w % 4) + l
    // of A (waves 0-3) or B (waves 4-7).
    uint32_t voff[MA + 2];
#pragma unroll
    for (int i = 0; i < MA + 2; ++i) {
        const int rr = i < MA ? 16 * (MA * wave + i) + (lane >> 2) : 32 * wave + 16 * (i - MA) + (lane >> 2);
        const int lim = i < MA ? rows_a : rows_b;
        const int src_row = rr < lim ? rr : lim - 1;
        voff[i] = (uint32_t)src_row * (uint32_t)KB + 16u * (uint32_t)((lane & 3) ^ swz(rr));
    }
    const int srow = 64 * (wave & 3) + lane;
    const int slim = wave < 4 ? rows_a : rows_b;
    const uint32_t voff_s = (uint32_t)(srow < slim ? srow : slim - 1) * 4u;
    auto issue = [&](int kt, int slot) {
        uint8_t* st = lds + slot * STAGE_BYTES;
        const uint32_t soff = (uint32_t)kt * BK;
#pragma unroll
        for (int i = 0; i < MA; ++i) copy16(rsrc_a, st + 16 * 64 * MA * wave + 1024 * i, voff[i], soff);
        copy16(rsrc_b, st + A_STAGE + 32 * 64 * wave, voff[MA], soff);
        copy16(rsrc_b, st + A_STAGE + 32 * 64 * wave + 1024, voff[MA + 1], soff);
        copy4(rsrc_s, st + A_STAGE + B_STAGE + 256 * wave, voff_s, (uint32_t)kt * chunk_stride);
    };

    int a_row[MA], b_row[4];
#pragma unroll
    for (int a = 0; a < MA; ++a) a_row[a] = 32 * MA * wm + 32 * a + (lane & 31);
#pragma unroll
    for (int b = 0; b < 4; ++b) b_row[b] = 128 * wn + 32 * b + (lane & 31);

    v16f acc[MA][4];
#pragma unroll
    for (int a = 0; a < MA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    int a_off[2][MA], b_off[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + g;
#pragma unroll
        for (int a = 0; a < MA; ++a) a_off[s][a] = a_row[a] * BK + 16 * (c ^ swz(a_row[a]));
#pragma unroll
        for (int b = 0; b < 4; ++b) b_off[s][b] = A_STAGE + b_row[b] * BK + 16 * (c ^ swz(b_row[b]));
    }
    // Byte offsets (within a stage) of this lane's scale bytes for k-step s:
    // block 2 s + g of the lane's A rows and B rows.
    int sa_off[2][MA], sb_off[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int a = 0; a < MA; ++a) sa_off[s][a] = A_STAGE + B_STAGE + 4 * a_row[a] + 2 * s + g;
#pragma unroll
        for (int b = 0; b < 4; ++b) sb_off[s][b] = A_STAGE + B_STAGE + 4 * BM + 4 * b_row[b] + 2 * s + g;
    }
    // Fragments and scale bytes of k-step s of a stage.
    auto read_frags = [&](const uint8_t* st, int s, v4i (&af)[MA], v4i (&bf)[4], int (&sa)[MA], int (&sb)[4]) {
#pragma unroll
        for (int a = 0; a < MA; ++a) af[a] = *reinterpret_cast<const v4i*>(st + a_off[s][a]);
#pragma unroll
        for (int b = 0; b < 4; ++b) bf[b] = *reinterpret_cast<const v4i*>(st + b_off[s][b]);
#pragma unroll
        for (int a = 0; a < MA; ++a) sa[a] = st[sa_off[s][a]];
#pragma unroll
        for (int b = 0; b < 4; ++b) sb[b] = st[sb_off[s][b]];
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

    static_assert(MA == 2 && COPIES == 5, "the interleave patterns below count 8 MFMAs, 12 reads, 5 copies");
    const int KT = K / 128;
    // conditional prologue and branchy wait, as in K-GEMM (an unconditional
    // one makes the compiler drain the ring before every stage's first read)
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
        if (st < KT) issue(st, st);
    {
        const int ahead = (KT - 1) < (STAGES - 1) ? (KT - 1) : (STAGES - 1);
        if (ahead >= 3) wait_vmcnt<3 * COPIES>();
        else if (ahead >= 2) wait_vmcnt<2 * COPIES>();
        else if (ahead == 1) wait_vmcnt<COPIES>();
        else wait_vmcnt<0>();
    }
    lds_barrier();

    // Software pipeline (as K-GEMM's 256-row variant): in stage kt, k-step 0
    // runs on register set 0 while k-step 1's operands are read into set 1;
    // after the barrier, k-step 1 runs on set 1 while the slot is refilled
    // with stage kt + STAGES and stage kt + 1's k-step 0 is read into set 0.
    int kt = 0;
    int slot = 0;
    v4i fa0[MA], fb0[4], fa1[MA], fb1[4];
    int sa0[MA], sb0[4], sa1[MA], sb1[4];
    read_frags(lds, 0, fa0, fb0, sa0, sb0);
    for (; kt + STAGES < KT; ++kt) {
        const int next = slot + 1 == STAGES ? 0 : slot + 1;
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + slot * STAGE_BYTES, 1, fa1, fb1, sa1, sb1);
        mma(fa0, fb0, sa0, sb0);
        // 8 MFMAs, 12 LDS reads (6 fragments, 6 scale bytes)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
        }
#pragma unroll
        for (int i = 4; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(STAGES - 2) * COPIES>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + next * STAGE_BYTES, 0, fa0, fb0, sa0, sb0);
        issue(kt + STAGES, slot);
        mma(fa1, fb1, sa1, sb1);
        // 8 MFMAs, 12 LDS reads and the 5 copies of the refill
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one direct copy
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
        for (int i = 5; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        slot = next;
    }
    for (; kt + 1 < KT; ++kt) {
        const int next = slot + 1 == STAGES ? 0 : slot + 1;
        read_frags(lds + slot * STAGE_BYTES, 1, fa1, fb1, sa1, sb1);
        mma(fa0, fb0, sa0, sb0);
        const int after = KT - 2 - kt;
        if (after >= 2) wait_vmcnt<2 * COPIES>();
        else if (after >= 1) wait_vmcnt<COPIES>();
        else wait_vmcnt<0>();
        lds_barrier();
        read_frags(lds + next * STAGE_BYTES, 0, fa0, fb0, sa0, sb0);
        mma(fa1, fb1, sa1, sb1);
        slot = next;
    }
    read_frags(lds + slot * STAGE_BYTES, 1, fa1, fb1, sa1, sb1);
    mma(fa0, fb0, sa0, sb0);
    mma(fa1, fb1, sa1, sb1);

    // Epilogue: each wave parks a 32 x 128 block of fp32 accumulators in its
    // part of the freed ring and writes it back as bf16, 8 consecutive columns
    // of one row per lane per 16-byte store.
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
