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
// Tiling.  A workgroup of 8 waves (two per SIMD) owns a 384 x 256 tile of acc
// (384 tokens; for SwiGLU 128 gate columns + the matching 128 up columns).
// Waves form a 4 (rows) x 2 (columns) grid; each owns 96 x 128 as 3 x 4 blocks
// of v_mfma_i32_32x32x32_i8 (32 x 32 outputs, 32 bytes of K per instruction,
// 16 int32 accumulators per lane per block, 192 in all).  For SwiGLU a wave's
// 128 columns are 64 gate columns and the 64 up columns of the same outputs,
// so every lane holds g and u of its elements.  Two waves per SIMD let the
// matrix core take MFMAs from whichever wave has one ready while the other
// waits on a fragment read, a copy or the stage barrier.
//
// Operand streaming.  Both operands are K-contiguous rows (q_x is [M, K] and
// q_w is [N, K]), which is the MFMA operand layout: a lane takes 16
// contiguous bytes of one row.  K advances 64 bytes per stage through a ring
// of 4 LDS slots (40 KiB each, the whole 160 KiB).  Global -> LDS copies are
// direct buffer loads (buffer_load_dwordx4 ... lds: 64 lanes x 16 B land
// contiguously in LDS, no VGPR staging): each wave copies 48 rows of A and 32
// rows of B per stage, five copies.  Each LDS row is 64 bytes (4 chunks of
// 16 B); chunk c of row r is stored at position c ^ ((r >> 2) & 3), so the
// 16-byte fragment reads of 16 consecutive rows hit distinct banks; the XOR
// is applied on the global side, so the copies stay contiguous in LDS.
//
// The copies are issued from inline assembly.  The compiler's wait-count pass
// treats any LDS read that follows an LDS-writing buffer load it cannot prove
// disjoint as dependent on it, and drains every outstanding copy (vmcnt(0))
// before the fragment reads of each stage, which removes the prefetch.  Here
// the ring discipline (explicit vmcnt waits and the stage barrier) orders
// copies and reads, so the copies are hidden from that pass; M0, which holds
// the LDS destination, is passed as an input operand, so the compiler knows
// it is set.
//
// Main loop (one stage = two k-steps of 12 MFMAs per wave), unrolled over
// the four slots of the ring so that every LDS offset is an immediate (K is
// a multiple of 256, so the stage count is a multiple of four):
//   - the MFMAs run in a fixed order (A0 x B0..B3, then A1/A2 alternating
//     over B0..B3), and each fragment register is refilled with the next
//     k-step's fragment right after its last use, which spreads the seven
//     reads over the k-step and gives each at least four MFMAs of latency;
//   - the stage barrier sits after the fourth MFMA of the second k-step, so
//     each wave enters it with MFMAs in flight; before it, a vmcnt wait
//     makes this wave's copies of the next stage complete, and lgkmcnt(0)
//     makes its reads of the current slot complete;
//   - after the barrier the current slot is refilled with the stage four
//     ahead: three copies spread over the rest of that k-step, the last two
//     in the next stage's first k-step.
// Past the last stage the copies are still issued (so every stage has the
// same shape and the vmcnt counts stay uniform) but with the voffset
// pushed beyond the buffer's range: the hardware returns zeros without a
// memory access and they land in slots no one reads again.
//
// Scheduling.  Workgroups are dealt round-robin to the 8 XCDs; the tile id is
// remapped so that each XCD walks a contiguous range of tiles in a grouped
// raster (2 M-tiles per group, N fastest within a group), so workgroups that
// run together on one XCD share A and B panels in that XCD's L2, and the
// weight panels, re-read once per group, stay in the 256 MB Infinity Cache.
//
// Ragged edges: a panel's rows past M or N lie past its buffer resource's
// range and load as zeros; their outputs are masked at the store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fixed_math.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int BM = 384;               // tile rows (tokens): 4 wave rows x 96
constexpr int BN = 256;               // tile columns (weight rows)
constexpr int BK = 64;                // K bytes per stage
constexpr int MA = 3;                 // 32-row A blocks per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int STAGE_BYTES = A_STAGE + B_STAGE;
constexpr int STAGES = 4;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
// copies per wave per stage: MA of A (16 rows each) and 2 of B
constexpr int COPIES = MA + 2;
// copies of a refill issued in the k-step after the stage barrier; the rest
// go out in the next stage's first k-step
constexpr int COPIES_NOW = 3;
// Epilogue staging: each wave parks 32 rows of its outputs at a time in the
// ring's memory (bf16 outputs as bf16; the int32 output as int32, rows
// padded to PITCH int32 to spread banks), and the tile's row scales follow
// the largest of those areas.
constexpr int PITCH = 136;
constexpr int STASH_WAVE_BYTES = 32 * PITCH * 4;
constexpr int STASH_BYTES = NWAVES * STASH_WAVE_BYTES;
constexpr int SX_OFFSET = STASH_BYTES;
constexpr int GROUP_M = 2;            // M-tiles per raster group
static_assert(RING_BYTES <= 160 * 1024, "LDS budget");
static_assert(SX_OFFSET + 4 * BM <= RING_BYTES, "row scales after the stash, inside the ring");
static_assert(STAGES * COPIES < 64, "vmcnt range");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// lgkmcnt(0): every LDS read of this wave has returned.
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier for the LDS ring: this wave's fragment reads are complete
// (lgkmcnt(0)) before any wave can pass it and refill the slot they read.
// Completion of the copies is established by the explicit vmcnt wait before
// it.  (A fenced __syncthreads() would drain every outstanding copy.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    wait_lds_reads();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Buffer resource words over [base, base + bytes) (raw, no stride; gfx9
// dword 3), uniform across the wave.
__device__ __forceinline__ v4u rsrc_words(const int8_t* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    v4u r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000u;
    return r;
}

// One direct copy: 64 lanes x 16 bytes from rsrc + voff + soff into LDS at
// lds_addr + 16 * lane.  The load writes no VGPR; its address operands are
// read at issue.
__device__ __forceinline__ void copy16(v4u rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr));
}

// Past-the-end offset for copies of stages beyond the last: beyond any
// buffer's num_records (< 2^31), so the load returns zeros and touches no memory.
constexpr uint32_t OOB = 0x80000000u;

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
    __shared__ __attribute__((aligned(1024))) int8_t lds[RING_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave >> 1;   // band of 96 rows of the tile
    const int wn = wave & 1;    // column half of the tile
    const Tile tile = map_tile(blockIdx.x, MT, NT);
    const int m0 = tile.tm * BM;
    const int rows_a = (M - m0) < BM ? (M - m0) : BM;

    // Epilogue scales: s_x of the tile's row tid into a register before the
    // main loop (parked in LDS after it, where the ring was); s_w of the
    // lane's 8 output columns is loaded after the loop (fewer registers live
    // across it).
    constexpr int EPI_CG = EP == Epilogue::SWIGLU ? 8 : 16;   // column groups per wave row
    const int epi_cg = lane % EPI_CG;
    const int epi_ro = lane / EPI_CG;
    const int epi_col0 = EP == Epilogue::SWIGLU ? tile.tn * (BN / 2) + 64 * wn + 8 * epi_cg
                                                : tile.tn * BN + 128 * wn + 8 * epi_cg;
    float sx_own = 0.0f;
    if constexpr (EP != Epilogue::S32) {
        if (tid < BM) sx_own = sx[tid < rows_a ? m0 + tid : M - 1];
    }

    // Copy sources.  Copy i < MA of wave w fills A slab rows 16 (MA w + i) ..
    // +15 of a stage; copy MA + i (i = 0, 1) fills B slab rows 32 w + 16 i ..
    // +15.  Lane l writes row (l / 4) of its 16 at chunk position l % 4,
    // which holds logical chunk (l % 4) ^ swz(row).  Offsets are relative to a
    // per-panel buffer resource (the tile's A rows; its gate rows; its up
    // rows), whose range ends at the panel's last row.
    int b_first;   // first weight row of this tile (gate rows for SwiGLU)
    if constexpr (EP == Epilogue::SWIGLU)
        b_first = tile.tn * (BN / 2);
    else
        b_first = tile.tn * BN;
    const int b_span = EP == Epilogue::SWIGLU ? BN / 2 : BN;
    const int rows_b = (N - b_first) < b_span ? (N - b_first) : b_span;
    const v4u rsrc_a = rsrc_words(A + (int64_t)m0 * K, (uint32_t)rows_a * (uint32_t)K);
    v4u rsrc_b;
    if constexpr (EP == Epilogue::SWIGLU) {
        // waves 0-3 copy B rows 0-127 (gate), waves 4-7 rows 128-255 (up)
        const int64_t first = wave < 4 ? b_first : (int64_t)N + b_first;
        rsrc_b = rsrc_words(B + first * K, (uint32_t)rows_b * (uint32_t)K);
    } else {
        rsrc_b = rsrc_words(B + (int64_t)b_first * K, (uint32_t)rows_b * (uint32_t)K);
    }
    // Row r of a panel is read at r K + its swizzled chunk.  Rows past the
    // panel's last row lie past the buffer's range and read as zeros (their
    // outputs are masked at the store).  A wave's copies are 16 rows apart
    // and share one swizzle, ((r >> 2) & 3) = ((lane >> 4) & 3).
    const uint32_t chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t voff_a = (uint32_t)(16 * MA * wave + (lane >> 2)) * (uint32_t)K + chunk;
    const uint32_t voff_b = (uint32_t)(32 * (EP == Epilogue::SWIGLU ? (wave & 3) : wave) + (lane >> 2)) * (uint32_t)K + chunk;
    const uint32_t row16 = 16u * (uint32_t)K;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int8_t*)lds);
    // copy i of the stage at K byte soff into ring slot `slot` (oob: 0 or OOB)
    auto issue = [&](int i, uint32_t soff, uint32_t oob, int slot) {
        const uint32_t dst = i < MA ? lds_base + slot * STAGE_BYTES + 1024 * (MA * wave + i)
                                    : lds_base + slot * STAGE_BYTES + A_STAGE + 2048 * wave + 1024 * (i - MA);
        const uint32_t vo = i < MA ? voff_a + (uint32_t)i * row16 : voff_b + (uint32_t)(i - MA) * row16;
        copy16(i < MA ? rsrc_a : rsrc_b, dst, vo + oob, soff);
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

    v16i acc[MA][4];
#pragma unroll
    for (int a = 0; a < MA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    // Prologue: fill every slot (stages past the last go out of range), wait
    // for stage 0, read its first k-step's fragments.
    const int KT = K / BK;
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
        for (int i = 0; i < COPIES; ++i) issue(i, (uint32_t)st * BK, st < KT ? 0u : OOB, st);
    wait_vmcnt<(STAGES - 1) * COPIES>();
    lds_barrier();
    v4i fa[MA], fb[4];
#pragma unroll
    for (int a = 0; a < MA; ++a) fa[a] = *reinterpret_cast<const v4i*>(lds + a_off[0][a]);
#pragma unroll
    for (int b = 0; b < 4; ++b) fb[b] = *reinterpret_cast<const v4i*>(lds + b_off[0][b]);
    // nothing of the prologue (scalar loads included) stays pending in
    // lgkmcnt, so the loop's waits on its fragment reads can be exact
    wait_lds_reads();
    __builtin_amdgcn_sched_barrier(0);

    // The fixed MFMA order of a k-step (slot i: A block SA[i] x B block SB[i])
    // and the refill points: A0 after slot 3, B0 after 5, B1 after 7, B2
    // after 9, B3, A1 and A2 after 11.
    constexpr int SA[12] = {0, 0, 0, 0, 1, 2, 1, 2, 1, 2, 1, 2};
    constexpr int SB[12] = {0, 1, 2, 3, 0, 0, 1, 1, 2, 2, 3, 3};
    auto mfma = [&](int i) {
        acc[SA[i]][SB[i]] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[SA[i]], fb[SB[i]], acc[SA[i]][SB[i]], 0, 0, 0);
    };
    auto refill = [&](int i, const int8_t* st, int s) {
        if (i == 3) fa[0] = *reinterpret_cast<const v4i*>(st + a_off[s][0]);
        if (i == 5) fb[0] = *reinterpret_cast<const v4i*>(st + b_off[s][0]);
        if (i == 7) fb[1] = *reinterpret_cast<const v4i*>(st + b_off[s][1]);
        if (i == 9) fb[2] = *reinterpret_cast<const v4i*>(st + b_off[s][2]);
        if (i == 11) {
            fb[3] = *reinterpret_cast<const v4i*>(st + b_off[s][3]);
            fa[1] = *reinterpret_cast<const v4i*>(st + a_off[s][1]);
            fa[2] = *reinterpret_cast<const v4i*>(st + a_off[s][2]);
        }
    };
    // copy j (< COPIES_NOW) of a refill goes out after slot CS[j] of the
    // k-step that follows the barrier; copies COPIES_NOW.. after slots 0 and 6
    // of the next stage's first k-step
    constexpr int CS[COPIES_NOW] = {4, 7, 10};
    constexpr int BARRIER_AFTER = 3;

    // One stage with its ring slot known at compile time (every LDS offset an
    // immediate); K is a multiple of 256, so the stage count is a multiple
    // of STAGES and the loop runs whole rounds.
    static_assert(256 % (STAGES * BK) == 0, "whole rounds of STAGES stages");
    auto stage = [&](auto slot_c, int kt) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int next = slot + 1 == STAGES ? 0 : slot + 1;
        constexpr int prev_slot = slot == 0 ? STAGES - 1 : slot - 1;
        const uint32_t oob = kt + STAGES < KT ? 0u : OOB;
        // the deferred copies belong to the previous stage's refill (before the
        // first refill: stage STAGES - 1 again, the same bytes into its slot)
        const uint32_t prev_soff = kt > 0 ? (uint32_t)(kt - 1 + STAGES) * BK : (uint32_t)(STAGES - 1) * BK;
        const uint32_t prev_oob = kt > 0 && kt - 1 + STAGES >= KT ? OOB : 0u;
        const uint32_t soff = (uint32_t)(kt + STAGES) * BK;
        const int8_t* cur = lds + slot * STAGE_BYTES;
        const int8_t* nxt = lds + next * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mfma(i);
            refill(i, cur, 1);
            if (i == 0) issue(COPIES_NOW, prev_soff, prev_oob, prev_slot);
            if (i == 6) issue(COPIES_NOW + 1, prev_soff, prev_oob, prev_slot);
        }
#pragma unroll
        for (int i = 0; i <= BARRIER_AFTER; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mfma(i);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(STAGES - 2) * COPIES>();
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if (i > BARRIER_AFTER) mfma(i);
            if (i == BARRIER_AFTER) {
#pragma unroll
                for (int j = 0; j <= BARRIER_AFTER; ++j) refill(j, nxt, 0);
            } else if (i > BARRIER_AFTER) {
                refill(i, nxt, 0);
            }
#pragma unroll
            for (int j = 0; j < COPIES_NOW; ++j)
                if (CS[j] == i) issue(j, soff, oob, slot);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(STAGES == 4, "rounds of four stages");
    for (int kt = 0; kt < KT; kt += 4) {
        stage(std::integral_constant<int, 0>{}, kt);
        stage(std::integral_constant<int, 1>{}, kt + 1);
        stage(std::integral_constant<int, 2>{}, kt + 2);
        stage(std::integral_constant<int, 3>{}, kt + 3);
    }
    const int prev_slot = STAGES - 1;
    const uint32_t prev_soff = (uint32_t)(KT - 1 + STAGES) * BK;
    // the deferred copies of the last refill (out of range), then no copy may
    // still be writing the ring, which the epilogue reuses
#pragma unroll
    for (int i = COPIES_NOW; i < COPIES; ++i) issue(i, prev_soff, OOB, prev_slot);
    wait_vmcnt<0>();

    // Epilogue.  Block (a, b), lane l, register r of the MFMA accumulators
    // holds row 32 a + 8 (r / 4) + 4 (l / 32) + r % 4 and column 32 b + l % 32
    // of the wave's 96 x 128 sub-tile.  For bf16 outputs each lane forms its
    // values where they lie (dequant, and for SwiGLU silu(g) u from the gate
    // block b and the up block b + 2 of the same outputs) and parks them as
    // bf16 in its wave's part of the (now free) ring, 32 rows at a time;
    // the rows are then read back contiguous, 16 bytes per lane, and leave
    // as one 16-byte store.  The int32 output parks the accumulators
    // themselves.
    const int l31 = lane & 31, hl = lane >> 5;
    // s_w of the lane's accumulator columns: b = 0..3 (BF16), or the gate
    // (b = 0, 1) and up (b = 2, 3) rows of h column 32 (b & 1) + l % 32
    float swv[4];
    if constexpr (EP != Epilogue::S32) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            int c;
            if constexpr (EP == Epilogue::SWIGLU)
                c = tile.tn * (BN / 2) + 64 * wn + 32 * (bb & 1) + l31;
            else
                c = tile.tn * BN + 128 * wn + 32 * bb + l31;
            c = c < N ? c : N - 1;
            swv[bb] = sw[(EP == Epilogue::SWIGLU && bb >= 2 ? N : 0) + c];
        }
    }
    lds_barrier();   // every wave is done reading the ring
    float* sx_lds = reinterpret_cast<float*>(lds + SX_OFFSET);
    if constexpr (EP != Epilogue::S32) {
        if (tid < BM) sx_lds[tid] = sx_own;
        lds_barrier();
    }
    const int grow0 = m0 + 32 * MA * wm;
    const int col0 = epi_col0;
    const int cg = epi_cg;
    const int ro = epi_ro;
    const bool vec_cols = (col0 + 8 <= N) && (N % 8 == 0);

    if constexpr (EP == Epilogue::S32) {
        int32_t* stash = reinterpret_cast<int32_t*>(lds + wave * STASH_WAVE_BYTES);
        int32_t* o = reinterpret_cast<int32_t*>(out);
#pragma unroll
        for (int a = 0; a < MA; ++a) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int bb = 0; bb < 4; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    stash[(8 * (r >> 2) + 4 * hl + (r & 3)) * PITCH + 32 * bb + l31] = acc[a][bb][r];
            asm volatile("" ::: "memory");
#pragma nounroll
            for (int it = 0; it < 8; ++it) {
                const int lr = 4 * it + ro;
                const int grow = grow0 + 32 * a + lr;
                const v4i a0 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 8 * cg);
                const v4i a1 = *reinterpret_cast<const v4i*>(stash + lr * PITCH + 8 * cg + 4);
                if (grow >= M) continue;
                if (vec_cols) {
                    *reinterpret_cast<v4i*>(o + (int64_t)grow * N + col0) = a0;
                    *reinterpret_cast<v4i*>(o + (int64_t)grow * N + col0 + 4) = a1;
                } else {
                    const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col0 + e < N) o[(int64_t)grow * N + col0 + e] = av[e];
                }
            }
        }
    } else {
        // bf16 rows of 64 (SwiGLU) or 128 outputs, padded to P16 bf16 so that
        // the two lane halves (rows r and r + 4) write disjoint banks
        constexpr int NB = EP == Epilogue::SWIGLU ? 2 : 4;     // output blocks per wave row
        constexpr int P16 = 32 * NB + 8;
        constexpr int ITS = EP == Epilogue::SWIGLU ? 4 : 8;    // read-back rows per lane
        constexpr int ROW_STEP = 32 / ITS;
        uint16_t* st16 = reinterpret_cast<uint16_t*>(lds + wave * (32 * P16 * 2));
        uint16_t* y = reinterpret_cast<uint16_t*>(out);
#pragma unroll
        for (int a = 0; a < MA; ++a) {
            // row scales of the lane's 16 rows: 32 a + 8 q + 4 (l / 32) + p
            float sxr[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4f t4 = *reinterpret_cast<const v4f*>(sx_lds + 32 * MA * wm + 32 * a + 8 * q + 4 * hl);
                sxr[4 * q] = t4.x;
                sxr[4 * q + 1] = t4.y;
                sxr[4 * q + 2] = t4.z;
                sxr[4 * q + 3] = t4.w;
            }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float v0, v1;
                    if constexpr (EP == Epilogue::SWIGLU) {
                        v0 = swiglu_hw(dequant(acc[a][bb][r], sxr[r], swv[bb]),
                                       dequant(acc[a][bb + 2][r], sxr[r], swv[bb + 2]));
                        v1 = swiglu_hw(dequant(acc[a][bb][r + 1], sxr[r + 1], swv[bb]),
                                       dequant(acc[a][bb + 2][r + 1], sxr[r + 1], swv[bb + 2]));
                    } else {
                        v0 = dequant(acc[a][bb][r], sxr[r], swv[bb]);
                        v1 = dequant(acc[a][bb][r + 1], sxr[r + 1], swv[bb]);
                    }
                    const uint32_t pk = pack_bf16(v0, v1);
                    const int row = 8 * (r >> 2) + 4 * hl + (r & 3);   // rows row, row + 1
                    st16[row * P16 + 32 * bb + l31] = (uint16_t)pk;
                    st16[(row + 1) * P16 + 32 * bb + l31] = (uint16_t)(pk >> 16);
                }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int it = 0; it < ITS; ++it) {
                const int lr = ROW_STEP * it + ro;
                const int grow = grow0 + 32 * a + lr;
                const v4u pk = *reinterpret_cast<const v4u*>(st16 + lr * P16 + 8 * cg);
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
