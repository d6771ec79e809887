// K-GEMM: int8 x int8 -> int32 contraction on CDNA4 MFMA with fused epilogues,
// for gfx950.
//
// What it computes (h3-rs README, "Speed": an int8 GEMM whose epilogue writes
// bf16 directly, with SwiGLU fused into fc1's epilogue by pairing gate and up
// rows; h3-rs README, model file table: weights are int8 with one scale per
// row):
//   acc[m][n] = sum_k q_x[m][k] * q_w[n][k]                      (exact int32)
//   S32    : out = acc
//   BF16   : y[m][n] = bf16_rne(((float)acc * s_x[m]) * s_w[n])
//   SWIGLU : g = fp32 dequant of column j, u = of column i + j (weight rows
//            [0, i) are the gate, [i, 2i) the up projection);
//            y[m][j] = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)),
//            evaluated with the hardware base-2 exponential and reciprocal
//            (see swiglu_hw).
//
// Tiling.  A workgroup of 8 waves (two per SIMD) owns a BM x 256 tile of acc
// (BM tokens; for SwiGLU 128 gate columns + the matching 128 up columns).
// Waves form a 4 (rows) x 2 (columns) grid; each owns 32 MA x 128 (MA =
// BM / 128) as MA x 4 blocks of v_mfma_i32_32x32x32_i8 (32 x 32 outputs,
// 32 bytes of K per instruction, 16 int32 accumulators per lane per block).
// For SwiGLU a wave's 128 columns are 64 gate columns and the 64 up columns of
// the same outputs, so every lane holds g and u of its elements.  K advances
// 64 bytes per stage through an LDS ring of STAGES slots.
//
// Why two waves per SIMD: each SIMD issues at most one instruction per wave
// every few cycles, and the fragment reads, the ring refills and their
// address set-up of one wave would otherwise sit in the gaps of that same
// wave's MFMA stream; with a second wave on the SIMD the matrix core takes
// MFMAs from whichever wave has one ready.
//
// Operand streaming.  Both operands are K-contiguous rows (q_x is [M, K] and
// q_w is [N, K]), which is the MFMA operand layout: a lane takes 16
// contiguous bytes of one row.  Global -> LDS copies use the direct buffer
// load (buffer_load_dwordx4 ... lds: 64 lanes x 16 B land contiguously in
// LDS, no VGPR staging); the per-lane row offset is a fixed register, the
// K position a scalar offset, so one copy costs one M0 move and one load.
// Each LDS row is 64 bytes (4 chunks of 16 B); chunk c of row r is stored at
// position c ^ ((r >> 2) & 3), which makes the 16-byte fragment reads of 16
// consecutive rows hit distinct banks.  The XOR is applied on the global
// side, so the copies stay contiguous in LDS.
//
// Scheduling.  Workgroups are dealt round-robin to the 8 XCDs; the tile id is
// remapped so that each XCD walks a contiguous range of tiles in a grouped
// raster (GROUP_M M-tiles per group, N fastest within a group), so workgroups
// that run together on one XCD share A and B panels in that XCD's L2.  With 2
// M-tiles per group the 32 tiles an XCD runs at once span 2 A panels and 16 B
// panels: each A panel is fetched from HBM about once, and the weight panels,
// re-read once per group, stay in the 256 MB Infinity Cache.  (8 M-tiles per
// group re-read A panels four times as often, beyond what the cache holds for
// the 462 MB activation of the down projection; 2 measured 4-5 % faster there.)
//
// Ragged edges: rows past M or N are clamped to the last row for loading and
// masked at the store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fixed_math.h"
#include "kernels.h"

namespace convrot {
namespace {

#ifndef CONVROT_GEMM_BM
#define CONVROT_GEMM_BM 384
#endif
constexpr int BM = CONVROT_GEMM_BM;   // tile rows (tokens): 4 wave rows x 32 MA
constexpr int BN = 256;               // tile columns (weight rows)
constexpr int BK = 64;
constexpr int MA = BM / 128;          // 32-row A blocks per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int STAGE_BYTES = A_STAGE + B_STAGE;
// copies per wave per stage: MA of A (16 rows each) and 2 of B
constexpr int COPIES = MA + 2;
// Epilogue staging: each wave parks 32 rows x 128 int32 at a time, rows
// padded to PITCH int32 to spread banks; it reuses the ring's memory.
constexpr int PITCH = 136;
constexpr int STASH_WAVE_BYTES = 32 * PITCH * 4;
constexpr int STASH_BYTES = NWAVES * STASH_WAVE_BYTES;
// as many ring stages (at most 4) as fit in 160 KiB of LDS with the stash
// (which reuses the ring) and the tile's row scales
constexpr int lds_for(int stages) {
    return (stages * STAGE_BYTES > STASH_BYTES ? stages * STAGE_BYTES : STASH_BYTES) + 4 * BM;
}
constexpr int STAGES = lds_for(4) <= 160 * 1024 ? 4 : 3;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = RING_BYTES > STASH_BYTES ? RING_BYTES : STASH_BYTES;
#ifndef CONVROT_GEMM_GROUP_M
#define CONVROT_GEMM_GROUP_M 2
#endif
constexpr int GROUP_M = CONVROT_GEMM_GROUP_M;   // M-tiles per raster group
static_assert(BM % 128 == 0 && MA >= 2 && MA <= 3, "tile rows");
static_assert(LDS_BYTES + 4 * BM <= 160 * 1024, "LDS budget");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the LDS ring.  Completion of the direct copies is
// established by the explicit vmcnt wait that precedes it, and the fragment
// reads of the previous stage by an lgkmcnt(0) wait; so only the hardware
// barrier is needed, plus a compiler barrier that keeps LDS accesses on their
// side of it.  (A fenced __syncthreads() would drain every outstanding
// prefetch with vmcnt(0).)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    // lgkmcnt(0): this wave's fragment reads are complete before any wave can
    // pass the barrier and refill the slot they read.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One direct copy: 64 lanes x 16 bytes from rsrc + voff + soff into LDS at
// dst + 16 * lane.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t rsrc, int8_t* dst, uint32_t voff,
                                       uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voff, soff, 0, 0);
#endif
}

// Buffer resource over [base, base + bytes) (raw, no stride; gfx9 dword 3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const int8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float dequant(int acc, float sx, float sw) {
    float f = (float)acc;
    f = f * sx;
    return f * sw;
}

// silu(g) * u for the fused epilogue, on the transcendental unit:
// e = v_exp_f32(-g log2(e)), then (g * v_rcp_f32(1 + e)) * u.  Its result is a
// bf16 output, which the layer's contract bounds relative to the exact value:
// the argument's rounding moves e by at most |g log2 e| 2^-23 ln 2 (< 1.1e-5
// relative for |g log2 e| < 128; beyond that e is 0 or +inf and the result is
// g u or -0), the exponential and the reciprocal are each within 1 ulp, so
// the fp32 result is within about 1.2e-5 of silu(g) u relatively and the bf16
// result within one bf16 ulp (2^-8) of it.  Where 1 + e exceeds 2^126 the
// reciprocal may flush to zero, a result below |g u| 2^-126 in magnitude.
// (The output-side SwiGLU pass, whose silu decides int8 codes, keeps the
// fixed exponential of fixed_math.h so that those codes match bit for bit.)
__device__ __forceinline__ float swiglu_hw(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(g * -0x1.715476p+0f);
    return (g * __builtin_amdgcn_rcpf(1.0f + e)) * u;
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

template <Epilogue EP>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ sx, const int8_t* __restrict__ B,
    const float* __restrict__ sw, int M, int N, int K, void* __restrict__ out, int MT, int NT) {
    __shared__ __attribute__((aligned(1024))) int8_t lds[LDS_BYTES];
    __shared__ float sx_lds[BM];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1;   // band of 32 MA rows of the tile
    const int wn = wave & 1;    // column half of the tile
    const Tile tile = map_tile(blockIdx.x, MT, NT);
    const int m0 = tile.tm * BM;
    const int rows_a = (M - m0) < BM ? (M - m0) : BM;

    // Epilogue scales, loaded before the main loop so that their latency is
    // hidden: s_x of the tile's rows into LDS (read back per output row), and
    // s_w of the lane's 8 output columns (gate and up columns for SwiGLU) into
    // registers.  (Keeping these register loads outstanding across the main
    // loop also keeps the compiler from draining the ring's copies before the
    // first fragment read of every stage, as it does when no other vector
    // load is pending there.)
    constexpr int EPI_CG = EP == Epilogue::SWIGLU ? 8 : 16;   // column groups per wave row
    const int epi_cg = lane % EPI_CG;
    const int epi_ro = lane / EPI_CG;
    const int epi_col0 = EP == Epilogue::SWIGLU ? tile.tn * (BN / 2) + 64 * wn + 8 * epi_cg
                                                : tile.tn * BN + 128 * wn + 8 * epi_cg;
    float swa[8], swb[8];
    if constexpr (EP != Epilogue::S32) {
        if (tid < BM) sx_lds[tid] = sx[tid < rows_a ? m0 + tid : M - 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = (epi_col0 + e) < N ? (epi_col0 + e) : (N - 1);
            swa[e] = sw[c];
            swb[e] = EP == Epilogue::SWIGLU ? sw[N + c] : 0.0f;
        }
    }

    // Copy sources.  Copy i < MA of wave w fills A slab rows 16 (MA w + i) ..
    // +15 of a stage; copy MA + i (i = 0, 1) fills B slab rows 32 w + 16 i ..
    // +15.  Lane l writes row (l / 4) of its 16 at chunk position l % 4,
    // which holds logical chunk (l % 4) ^ swz(row).  Offsets are relative to a
    // per-panel buffer resource (the tile's A rows; its gate rows; its up rows).
    int b_first;   // first weight row of this tile (gate rows for SwiGLU)
    if constexpr (EP == Epilogue::SWIGLU)
        b_first = tile.tn * (BN / 2);
    else
        b_first = tile.tn * BN;
    const int b_span = EP == Epilogue::SWIGLU ? BN / 2 : BN;
    const int rows_b = (N - b_first) < b_span ? (N - b_first) : b_span;
    const __amdgpu_buffer_rsrc_t rsrc_a = make_rsrc(A + (int64_t)m0 * K, (uint32_t)rows_a * (uint32_t)K);
    __amdgpu_buffer_rsrc_t rsrc_b;
    if constexpr (EP == Epilogue::SWIGLU) {
        // waves 0-3 copy B rows 0-127 (gate), waves 4-7 rows 128-255 (up)
        const int64_t first = wave < 4 ? b_first : (int64_t)N + b_first;
        rsrc_b = make_rsrc(B + first * K, (uint32_t)rows_b * (uint32_t)K);
    } else {
        rsrc_b = make_rsrc(B + (int64_t)b_first * K, (uint32_t)rows_b * (uint32_t)K);
    }
    uint32_t voff[COPIES];
#pragma unroll
    for (int i = 0; i < COPIES; ++i) {
        const int rr = i < MA ? 16 * (MA * wave + i) + (lane >> 2)           // A slab row
                              : 32 * wave + 16 * (i - MA) + (lane >> 2);    // B slab row
        const int c = (lane & 3) ^ swz(rr);
        int src_row;
        if (i < MA) {
            src_row = rr < rows_a ? rr : rows_a - 1;
        } else if constexpr (EP == Epilogue::SWIGLU) {
            const int j = rr & 127;   // the gate or up row of output column b_first + j
            src_row = j < rows_b ? j : rows_b - 1;
        } else {
            src_row = rr < rows_b ? rr : rows_b - 1;
        }
        voff[i] = (uint32_t)src_row * (uint32_t)K + 16u * (uint32_t)c;
    }
    auto issue = [&](int kt, int slot) {
        int8_t* a_dst = lds + slot * STAGE_BYTES + 16 * 64 * MA * wave;
        int8_t* b_dst = lds + slot * STAGE_BYTES + A_STAGE + 32 * 64 * wave;
        const uint32_t soff = (uint32_t)kt * BK;
#pragma unroll
        for (int i = 0; i < MA; ++i) copy16(rsrc_a, a_dst + 1024 * i, voff[i], soff);
        copy16(rsrc_b, b_dst, voff[MA], soff);
        copy16(rsrc_b, b_dst + 1024, voff[MA + 1], soff);
    };

    // LDS rows of this lane's fragments: A blocks a < MA (rows of the wave's
    // band), B blocks b = 0..3 (for SwiGLU: b = 0, 1 gate, 2, 3 up).
    int a_row[MA], b_row[4];
#pragma unroll
    for (int a = 0; a < MA; ++a) a_row[a] = 32 * MA * wm + 32 * a + (lane & 31);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if constexpr (EP == Epilogue::SWIGLU)
            b_row[b] = (b < 2 ? 0 : 128) + 64 * wn + 32 * (b & 1) + (lane & 31);
        else
            b_row[b] = 128 * wn + 32 * b + (lane & 31);
    }

    v16i acc[MA][4];
#pragma unroll
    for (int a = 0; a < MA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    // Byte offsets (within a stage) of this lane's 16-byte fragment reads for
    // the two 32-byte k-steps of a stage.
    int a_off[2][MA], b_off[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + (lane >> 5);
#pragma unroll
        for (int a = 0; a < MA; ++a) a_off[s][a] = a_row[a] * BK + 16 * (c ^ swz(a_row[a]));
#pragma unroll
        for (int b = 0; b < 4; ++b) b_off[s][b] = A_STAGE + b_row[b] * BK + 16 * (c ^ swz(b_row[b]));
    }
    auto read_frags = [&](const int8_t* st, int s, v4i (&af)[MA], v4i (&bf)[4]) {
#pragma unroll
        for (int a = 0; a < MA; ++a) af[a] = *reinterpret_cast<const v4i*>(st + a_off[s][a]);
#pragma unroll
        for (int b = 0; b < 4; ++b) bf[b] = *reinterpret_cast<const v4i*>(st + b_off[s][b]);
    };
    auto mma = [&](const v4i (&af)[MA], const v4i (&bf)[4]) {
#pragma unroll
        for (int a = 0; a < MA; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bf[b], acc[a][b], 0, 0, 0);
    };

    // Software pipeline.  All STAGES slots are filled up front.  Each stage
    // holds two 32-byte k-steps; in stage kt:
    //   k-step 0: MFMAs interleaved with the fragment reads of k-step 1;
    //   barrier:  stage kt + 1 has landed (vmcnt) and every wave has read both
    //             k-steps of stage kt (lgkmcnt before the barrier);
    //   k-step 1: MFMAs interleaved with the refill of stage kt's slot with
    //             stage kt + STAGES and the reads of stage kt + 1's k-step 0.
    // At stage kt's barrier the stages after kt + 1 may stay in flight
    // (STAGES - 2 of them, COPIES copies each).  With 384-row tiles the reads
    // refill the registers of the fragments the MFMAs have finished with;
    // the 256-row variant has room for two fragment sets, runs a steady-state
    // loop while a refill remains and peels the last stages.
    constexpr int NREAD = MA + 4;        // fragment reads per k-step
    constexpr int NMFMA = 4 * MA;        // MFMAs per k-step
    const int KT = K / BK;
    // (The conditional issue and the branch on the stages ahead are kept in
    // this form on purpose: with an unconditional prologue the compiler
    // inserts a full vmcnt(0) before the first fragment read of every stage
    // of the main loop, which drains the prefetch.)
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
        if (st < KT) issue(st, st);
    {
        const int ahead = (KT - 1) < (STAGES - 1) ? (KT - 1) : (STAGES - 1);
        if (STAGES >= 4 && ahead >= 3) wait_vmcnt<(STAGES >= 4 ? 3 : 2) * COPIES>();
        else if (ahead >= 2) wait_vmcnt<2 * COPIES>();
        else if (ahead == 1) wait_vmcnt<COPIES>();
        else wait_vmcnt<0>();
    }
    lds_barrier();

    int kt = 0;
    int slot = 0;                        // slot of stage kt
    if constexpr (MA == 3) {
        // 192 accumulators leave room for one fragment set only.  Each k-step
        // issues its MFMAs row by row (A block 0 with B blocks 0-3, then A
        // block 1, then A block 2), and every fragment register is refilled
        // with the next k-step's fragment as soon as the last MFMA that reads
        // it has issued: A blocks 0 and 1 after their rows, the B blocks and
        // A block 2 during the last row.  The reads of one k-step thus run
        // under the MFMAs of the one before, with no second register set.
        // (Reading all seven fragments first and then issuing the MFMAs left
        // the matrix core idle at every k-step for the read latency whenever
        // the two waves of a SIMD reached their reads together, as they do
        // after each barrier; measured 4-5 % slower on both FFN GEMMs.)
        v4i fa[MA], fb[4];
        auto mma_refill = [&](const int8_t* st, int s) {
#pragma unroll
            for (int a = 0; a < MA - 1; ++a) {
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[a], fb[b], acc[a][b], 0, 0, 0);
                fa[a] = *reinterpret_cast<const v4i*>(st + a_off[s][a]);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                acc[MA - 1][b] =
                    __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[MA - 1], fb[b], acc[MA - 1][b], 0, 0, 0);
                fb[b] = *reinterpret_cast<const v4i*>(st + b_off[s][b]);
            }
            fa[MA - 1] = *reinterpret_cast<const v4i*>(st + a_off[s][MA - 1]);
        };
        read_frags(lds, 0, fa, fb);
        for (; kt < KT; ++kt) {
            const int next = slot + 1 == STAGES ? 0 : slot + 1;
            const bool refill = kt + STAGES < KT;
            __builtin_amdgcn_sched_barrier(0);
            // k-step 0 of stage kt, reading k-step 1 of the same slot
            mma_refill(lds + slot * STAGE_BYTES, 1);
            __builtin_amdgcn_sched_barrier(0);
            // stage kt + 1 must have landed before its fragments are read
            const int after = KT - 2 - kt;   // stages behind kt + 1 in flight (<= STAGES - 2)
            if (after >= 1) wait_vmcnt<COPIES>();
            else wait_vmcnt<0>();
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (refill) issue(kt + STAGES, slot);
            __builtin_amdgcn_sched_barrier(0);
            // k-step 1 of stage kt, reading k-step 0 of stage kt + 1 (after
            // the last stage this reads a landed slot whose values go unused)
            mma_refill(lds + next * STAGE_BYTES, 0);
            __builtin_amdgcn_sched_barrier(0);
            slot = next;
        }
    } else {
    v4i fa0[MA], fb0[4], fa1[MA], fb1[4];
    read_frags(lds, 0, fa0, fb0);
    for (; kt + STAGES < KT; ++kt) {
        const int next = slot + 1 == STAGES ? 0 : slot + 1;
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + slot * STAGE_BYTES, 1, fa1, fb1);
        mma(fa0, fb0);
#pragma unroll
        for (int i = 0; i < NREAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NREAD, 0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(STAGES - 2) * COPIES>();
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(lds + next * STAGE_BYTES, 0, fa0, fb0);
        issue(kt + STAGES, slot);
        mma(fa1, fb1);
#pragma unroll
        for (int i = 0; i < COPIES; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one direct copy
        }
#pragma unroll
        for (int i = COPIES; i < NREAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMFMA - NREAD, 0);
        __builtin_amdgcn_sched_barrier(0);
        slot = next;
    }
    // Peeled tail: the stages with a successor, then the last.
    for (; kt + 1 < KT; ++kt) {
        const int next = slot + 1 == STAGES ? 0 : slot + 1;
        read_frags(lds + slot * STAGE_BYTES, 1, fa1, fb1);
        mma(fa0, fb0);
        const int after = KT - 2 - kt;   // stages behind kt + 1 still in flight (<= STAGES - 2)
        if (STAGES >= 4 && after >= 2) wait_vmcnt<2 * COPIES>();
        else if (after >= 1) wait_vmcnt<COPIES>();
        else wait_vmcnt<0>();
        lds_barrier();
        read_frags(lds + next * STAGE_BYTES, 0, fa0, fb0);
        mma(fa1, fb1);
        slot = next;
    }
    read_frags(lds + slot * STAGE_BYTES, 1, fa1, fb1);
    mma(fa0, fb0);
    mma(fa1, fb1);
    }

    // Epilogue.  Block (a, b), lane l, register r of the MFMA accumulators
    // holds row 32 a + 8 (r / 4) + 4 (l / 32) + r % 4 and column 32 b + l % 32
    // of the wave's 32 MA x 128 sub-tile.  Row block by row block, each wave
    // parks its 32 x 128 int32 accumulators in its own part of the (now free)
    // ring, then reads them back row-contiguous: every lane takes 8
    // consecutive columns of one row, applies the scales and the epilogue math
    // in a compact loop, and writes one 16-byte store.
    lds_barrier();   // every wave is done reading the ring
    int32_t* stash = reinterpret_cast<int32_t*>(lds + wave * STASH_WAVE_BYTES);
    const int grow0 = m0 + 32 * MA * wm;


    auto stash_block = [&](int a) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                stash[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * PITCH + 32 * b + (lane & 31)] =
                    acc[a][b][r];
        asm volatile("" ::: "memory");
    };

    const int col0 = epi_col0;
    const int cg = epi_cg;
    const int ro = epi_ro;
    const bool vec_cols = (col0 + 8 <= N) && (N % 8 == 0);
    if constexpr (EP == Epilogue::SWIGLU) {
        // lane -> 8 output columns (gate j, up i + j) and a row phase of 8
        uint16_t* y = reinterpret_cast<uint16_t*>(out);
#pragma unroll
        for (int a = 0; a < MA; ++a) {
            stash_block(a);
#pragma nounroll
            for (int it = 0; it < 4; ++it) {
                const int lr = 8 * it + ro;
                const int grow = grow0 + 32 * a + lr;
                const float sxr = sx_lds[32 * MA * wm + 32 * a + lr];
                const v4i g0 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 8 * cg);
                const v4i g1 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 8 * cg + 4);
                const v4i u0 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 64 + 8 * cg);
                const v4i u1 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 64 + 8 * cg + 4);
                const int ga[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
                const int ua[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                float h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float g = dequant(ga[e], sxr, swa[e]);
                    const float u = dequant(ua[e], sxr, swb[e]);
                    h[e] = swiglu_hw(g, u);
                }
                const v4u pk = {pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]), pack_bf16(h[4], h[5]),
                                pack_bf16(h[6], h[7])};
                if (grow < M) {
                    if (vec_cols) {
                        *reinterpret_cast<v4u*>(y + (int64_t)grow * N + col0) = pk;
                    } else {
                        const uint32_t pw[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col0 + e < N)
                                y[(int64_t)grow * N + col0 + e] = (uint16_t)(pw[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
    } else {
        // lane -> 8 output columns and a row phase of 4
#pragma unroll
        for (int a = 0; a < MA; ++a) {
            stash_block(a);
#pragma nounroll
            for (int it = 0; it < 8; ++it) {
                const int lr = 4 * it + ro;
                const int grow = grow0 + 32 * a + lr;
                const v4i a0 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 8 * cg);
                const v4i a1 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 8 * cg + 4);
                if (grow >= M) continue;
                if constexpr (EP == Epilogue::S32) {
                    int32_t* o = reinterpret_cast<int32_t*>(out);
                    if (vec_cols) {
                        *reinterpret_cast<v4i*>(o + (int64_t)grow * N + col0) = a0;
                        *reinterpret_cast<v4i*>(o + (int64_t)grow * N + col0 + 4) = a1;
                    } else {
                        const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col0 + e < N) o[(int64_t)grow * N + col0 + e] = av[e];
                    }
                } else {
                    uint16_t* y = reinterpret_cast<uint16_t*>(out);
                    const float sxr = sx_lds[32 * MA * wm + 32 * a + lr];
                    const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
                    float h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[e] = dequant(av[e], sxr, swa[e]);
                    const v4u pk = {pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]), pack_bf16(h[4], h[5]),
                                    pack_bf16(h[6], h[7])};
                    if (vec_cols) {
                        *reinterpret_cast<v4u*>(y + (int64_t)grow * N + col0) = pk;
                    } else {
                        const uint32_t pw[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (col0 + e < N)
                                y[(int64_t)grow * N + col0 + e] = (uint16_t)(pw[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(Epilogue ep, const int8_t* q_x, const float* s_x, const int8_t* q_w,
                       const float* s_w, int64_t m, int64_t n, int64_t k, void* out,
                       hipStream_t stream) {
    const int MT = (int)((m + BM - 1) / BM);
    const int tn = ep == Epilogue::SWIGLU ? BN / 2 : BN;
    const int NT = (int)((n + tn - 1) / tn);
    dim3 grid((unsigned)(MT * NT));
    dim3 block(NTHREADS);
    switch (ep) {
        case Epilogue::S32:
            gemm_kernel<Epilogue::S32><<<grid, block, 0, stream>>>(q_x, s_x, q_w, s_w, (int)m, (int)n,
                                                                    (int)k, out, MT, NT);
            break;
        case Epilogue::BF16:
            gemm_kernel<Epilogue::BF16><<<grid, block, 0, stream>>>(q_x, s_x, q_w, s_w, (int)m,
                                                                     (int)n, (int)k, out, MT, NT);
            break;
        case Epilogue::SWIGLU:
            gemm_kernel<Epilogue::SWIGLU><<<grid, block, 0, stream>>>(q_x, s_x, q_w, s_w, (int)m,
                                                                       (int)n, (int)k, out, MT, NT);
            break;
    }
    return hipGetLastError();
}

}  // namespace convrot
