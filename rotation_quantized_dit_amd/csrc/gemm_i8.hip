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
// Waves form a 4 (rows) x 2 (columns) grid; each owns 96 x 128 as 6 x 8 blocks
// of v_mfma_i32_16x16x64_i8 (16 x 16 outputs, 64 bytes of K per instruction,
// 4 int32 accumulators per lane per block, 192 in all).  For SwiGLU a wave's
// 128 columns are 64 gate columns and the 64 up columns of the same outputs,
// so every lane holds g and u of its elements.  Two waves per SIMD let the
// matrix core take MFMAs from whichever wave has one ready while the other
// waits on a fragment read, a copy or the stage barrier.
//
// Why 16 x 16 x 64.  The chip runs this kernel at its power limit, so the
// rate is set by the energy per operation.  For the same int8 work and the
// same LDS fragment bytes, the 16 x 16 form moves a quarter of the
// accumulator bytes through the register file per operation (4 registers read
// and written per 32 K ops against 16 per 64 K) and holds the higher clock:
// a loop of either form at the power limit, with this kernel's fragment
// traffic, sustained 3.35 against 2.96 POP/s, and this kernel runs 8-11 %
// faster than the same design on v_mfma_i32_32x32x32_i8.

// Operand streaming.  Both operands are K-contiguous rows (q_x is [M, K] and
// q_w is [N, K]), which is the MFMA operand layout: a lane takes 16
// contiguous bytes of one row (row l % 16 of a 16-row block, chunk l / 16).
// K advances 64 bytes per stage through a ring of 3 LDS slots (40 KiB each;
// a fourth slot measured 0.6-0.7 % slower).  Global -> LDS copies are
// direct buffer loads (buffer_load_dwordx4 ... lds: 64 lanes x 16 B land
// contiguously in LDS, no VGPR staging): each wave copies 48 rows of A and 32
// rows of B per stage, five copies.  Each LDS row is 64 bytes (4 chunks of
// 16 B); chunk c of row r is stored at position c ^ ((r >> 1) & 3), so the
// fragment reads (16 consecutive rows at each of the 4 chunks) are free of
// bank conflicts; the XOR is applied on the global side, so the copies stay
// contiguous in LDS.  (The swizzle (r >> 2) & 3, conflict-free for 32 x 32
// fragments, costs this read pattern a 2-way conflict: 8 LDS cycles per
// ds_read_b128 instead of 4, measured with SQ_LDS_IDX_ACTIVE.)
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
// Main loop (one stage = 48 MFMAs per wave, 64 bytes of K), unrolled over the
// three slots of the ring, with a peeled remainder of one or two stages:
//   - the stage runs as 8 phases, one per B block j: every A block times B
//     block j.  The six A fragments stay in registers for the stage and B is
//     double-buffered, B block j + 1 read at the start of phase j (224
//     registers of accumulators and fragments);
//   - the stage barrier sits after the fourth MFMA of phase 6, so each wave
//     enters it with MFMAs in flight; before it, a vmcnt wait makes this
//     wave's copies of the next stage complete, and lgkmcnt(0) makes its
//     reads of the current slot complete;
//   - phase 7 then reads the next slot: its first B block at the phase's
//     start and each A block right after that block's last MFMA;
//   - after the barrier the current slot is refilled with the stage three
//     ahead: three copies spread over the rest of the stage, the last two
//     in the next stage's first phases.
// Past the last stage the copies are still issued (so every stage has the
// same shape and the vmcnt counts stay uniform) but with the voffset
// pushed beyond the buffer's range: the hardware returns zeros without a
// memory access and they land in slots no one reads again.
//
// Scheduling.  Workgroups are dealt round-robin to the 8 XCDs; the tile id is
// remapped so that each XCD walks a contiguous range of tiles in a grouped
// raster (N fastest within a group of 2 M-tiles, or of 4 when there are at
// least 64 N-tiles), so workgroups that run together on one XCD share A and B
// panels in that XCD's L2, and the weight panels, re-read once per group,
// stay in the 256 MB Infinity Cache.  (Wide weights, such as the 112 N-tiles
// of FFN-up: 4 M-tiles per group re-read them half as often at the same
// speed; with 21 N-tiles, as in FFN-down, 4 per group measured 3.6 % slower.)
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
constexpr int WROWS = 96;             // tile rows per wave (BM / 4)
constexpr int A_COPIES = 3;           // 16-row copies of A per wave per stage (WROWS / 2 / 16)
constexpr int NA = 6;                 // 16-row A blocks per wave (MFMA rows)
constexpr int NB = 8;                 // 16-column B blocks per wave (MFMA columns)
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int STAGE_BYTES = A_STAGE + B_STAGE;
constexpr int STAGES = 3;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
// copies per wave per stage: A_COPIES of A (16 rows each) and 2 of B
constexpr int COPIES = A_COPIES + 2;
// copies of a refill issued in the k-step after the stage barrier; the rest
// go out in the next stage's first k-step
constexpr int COPIES_NOW = 3;
// Epilogue staging: each wave parks 32 rows of its outputs at a time in the
// ring's memory (bf16 outputs as bf16; the int32 output as int32, rows
// padded to PITCH int32 to spread banks), and the tile's row scales follow
// the largest of those areas.
constexpr int PITCH = 140;
constexpr int STASH_WAVE_BYTES = 16 * PITCH * 4;
constexpr int STASH_BYTES = NWAVES * STASH_WAVE_BYTES;
constexpr int SX_OFFSET = STASH_BYTES;
constexpr int GROUP_M = 2;            // M-tiles per raster group (twice that for >= 64 N-tiles)
static_assert(RING_BYTES <= 160 * 1024, "LDS budget");
static_assert(SX_OFFSET + 4 * BM <= RING_BYTES, "row scales after the stash, inside the ring");
static_assert(STAGES * COPIES < 64, "vmcnt range");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// a + b for a lane value a and a constant b, computed where it stands (the
// compiler neither hoists nor folds it)
template <int B>
__device__ __forceinline__ int opaque_add(int a) {
    int r;
    asm volatile("v_add_u32_e32 %0, %2, %1" : "=v"(r) : "v"(a), "i"(B));
    return r;
}

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
    const int G = NT >= 64 ? 2 * GROUP_M : GROUP_M;
    const int group = t / (G * NT);
    const int first_m = group * G;
    const int gm = (MT - first_m) < G ? (MT - first_m) : G;
    const int within = t - group * G * NT;
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

    // Epilogue scales are loaded after the main loop (no register of theirs
    // lives across it): s_x of the tile's row tid, parked in LDS where the ring
    // was, and s_w of the lane's output columns.
    constexpr int EPI_CG = EP == Epilogue::SWIGLU ? 8 : 16;   // column groups per wave row
    const int epi_cg = lane % EPI_CG;
    const int epi_ro = lane / EPI_CG;
    const int epi_col0 = EP == Epilogue::SWIGLU ? tile.tn * (BN / 2) + 64 * wn + 8 * epi_cg
                                                : tile.tn * BN + 128 * wn + 8 * epi_cg;

    // Copy sources.  Copy i < A_COPIES of wave w fills A slab rows
    // 16 (A_COPIES w + i) .. +15 of a stage; copy A_COPIES + i (i = 0, 1)
    // fills B slab rows 32 w + 16 i .. +15.  Lane l writes row (l / 4) of its
    // 16 at chunk position l % 4, which holds logical chunk
    // (l % 4) ^ ((row >> 1) & 3).  Offsets are relative to a per-panel buffer
    // resource (the tile's A rows; its gate rows; its up rows), whose range
    // ends at the panel's last row.
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
    // and share one swizzle, ((r >> 1) & 3) = ((lane >> 3) & 3).
    const uint32_t chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 3) & 3));
    const uint32_t voff_a = (uint32_t)(16 * A_COPIES * wave + (lane >> 2)) * (uint32_t)K + chunk;
    const uint32_t voff_b = (uint32_t)(32 * (EP == Epilogue::SWIGLU ? (wave & 3) : wave) + (lane >> 2)) * (uint32_t)K + chunk;
    const uint32_t row16 = 16u * (uint32_t)K;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int8_t*)lds);
    // copy i of the stage at K byte soff into ring slot `slot` (oob: 0 or OOB)
    auto issue = [&](int i, uint32_t soff, uint32_t oob, int slot) {
        const uint32_t dst = i < A_COPIES
                                 ? lds_base + slot * STAGE_BYTES + 1024 * (A_COPIES * wave + i)
                                 : lds_base + slot * STAGE_BYTES + A_STAGE + 2048 * wave + 1024 * (i - A_COPIES);
        const uint32_t vo = i < A_COPIES ? voff_a + (uint32_t)i * row16 : voff_b + (uint32_t)(i - A_COPIES) * row16;
        copy16(i < A_COPIES ? rsrc_a : rsrc_b, dst, vo + oob, soff);
    };

    // Fragment reads.  v_mfma_i32_16x16x64_i8 takes, in lane l, row l % 16 of
    // a 16-row block and the 16 bytes of K at chunk l / 16 of the stage's 64.
    // Every block starts at a row that is a multiple of 16, so the swizzle
    // (row >> 1) & 3 depends on the lane alone and block i of a panel lies
    // 1 KiB after block i - 1: one base offset per operand.
    const int fr = lane & 15;
    const int fpos = 16 * ((lane >> 4) ^ ((fr >> 1) & 3));
    const int a_base = (WROWS * wm + fr) * BK + fpos;
    const int b_base = A_STAGE + ((EP == Epilogue::SWIGLU ? 64 : 128) * wn + fr) * BK + fpos;
    // B block j of the wave: rows 16 j of its 128 (BF16, S32); for SwiGLU
    // blocks 0-3 are gate rows 64 wn + 16 j and blocks 4-7 the up rows of the
    // same outputs, 128 rows further
    constexpr int BOFF[NB] = {0, 1, 2, 3, EP == Epilogue::SWIGLU ? 8 : 4, EP == Epilogue::SWIGLU ? 9 : 5,
                              EP == Epilogue::SWIGLU ? 10 : 6, EP == Epilogue::SWIGLU ? 11 : 7};

    v4i acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = v4i{0, 0, 0, 0};

    // Prologue: fill every slot (stages past the last go out of range), wait
    // for stage 0, read its A fragments and its first B fragment.
    const int KT = K / BK;
#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
        for (int i = 0; i < COPIES; ++i) issue(i, (uint32_t)st * BK, st < KT ? 0u : OOB, st);
    wait_vmcnt<(STAGES - 1) * COPIES>();
    lds_barrier();
    v4i fa[NA], fb[2];
#pragma unroll
    for (int a = 0; a < NA; ++a) fa[a] = *reinterpret_cast<const v4i*>(lds + a_base + 1024 * a);
    fb[0] = *reinterpret_cast<const v4i*>(lds + b_base);
    // nothing of the prologue (scalar loads included) stays pending in
    // lgkmcnt, so the loop's waits on its fragment reads can be exact
    wait_lds_reads();
    __builtin_amdgcn_sched_barrier(0);

    // A stage is NB phases of NA MFMAs: phase j multiplies every A block with
    // B block j (in fb[j & 1]), and B block j + 1 is read at the start of
    // phase j.  The stage barrier follows MFMA BARRIER_AT (in phase NB - 2);
    // phase NB - 1 then reads the next slot: its first B block at the phase's
    // start and each A block right after that block's last MFMA.
    constexpr int BARRIER_AT = NA * (NB - 2) + 3;
    // copy j (< COPIES_NOW) of a refill goes out after MFMA CS[j] of the
    // stage, after the barrier; copies COPIES_NOW.. after MFMAs 0 and 12 of
    // the next stage
    constexpr int CS[COPIES_NOW] = {BARRIER_AT + 2, BARRIER_AT + 4, BARRIER_AT + 6};
    static_assert(BARRIER_AT + 6 < NA * NB, "copies inside the stage");

    // One stage with its ring slot known at compile time (every slot offset a
    // constant); the loop runs in rounds of STAGES, then the remainder.
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
        // fragment bases in this stage's slot (B only) and the next stage's,
        // formed here by an opaque add so that the compiler keeps three
        // registers rather than one per slot and block across the loop
        const int8_t* cur_b = lds + opaque_add<slot * STAGE_BYTES>(b_base);
        const int8_t* nxt_a = lds + opaque_add<next * STAGE_BYTES>(a_base);
        const int8_t* nxt_b = lds + opaque_add<next * STAGE_BYTES>(b_base);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int idx = NA * j + i;
                __builtin_amdgcn_sched_barrier(0);
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j & 1], acc[i][j], 0, 0, 0);
                if (i == 0 && j + 1 < NB)
                    fb[(j + 1) & 1] = *reinterpret_cast<const v4i*>(cur_b + 1024 * BOFF[j + 1]);
                if (idx == 0) issue(COPIES_NOW, prev_soff, prev_oob, prev_slot);
                if (idx == 12) issue(COPIES_NOW + 1, prev_soff, prev_oob, prev_slot);
                if (idx == BARRIER_AT) {
                    __builtin_amdgcn_sched_barrier(0);
                    wait_vmcnt<(STAGES - 2) * COPIES>();
                    lds_barrier();
                }
                if (j == NB - 1) {
                    if (i == 0) fb[0] = *reinterpret_cast<const v4i*>(nxt_b);
                    fa[i] = *reinterpret_cast<const v4i*>(nxt_a + 1024 * i);
                }
#pragma unroll
                for (int c = 0; c < COPIES_NOW; ++c)
                    if (CS[c] == idx) issue(c, soff, oob, slot);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(STAGES == 3, "rounds of three stages");
    int kt = 0;
    for (; kt + 3 <= KT; kt += 3) {
        stage(std::integral_constant<int, 0>{}, kt);
        stage(std::integral_constant<int, 1>{}, kt + 1);
        stage(std::integral_constant<int, 2>{}, kt + 2);
    }
    if (kt < KT) stage(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < KT) stage(std::integral_constant<int, 1>{}, kt + 1);
    const int prev_slot = (KT - 1) % STAGES;
    const uint32_t prev_soff = (uint32_t)(KT - 1 + STAGES) * BK;
    // the deferred copies of the last refill (out of range), then no copy may
    // still be writing the ring, which the epilogue reuses
#pragma unroll
    for (int i = COPIES_NOW; i < COPIES; ++i) issue(i, prev_soff, OOB, prev_slot);
    wait_vmcnt<0>();

    // Epilogue.  Block (a, b), lane l, register r of the accumulators holds
    // row 16 a + 4 (l / 16) + r and column 16 b + l % 16 of the wave's
    // 96 x 128 sub-tile; for SwiGLU block b < 4 holds the gate and block
    // b + 4 the up value of output column 16 b + l % 16 of the wave's 64.
    // For bf16 outputs each lane forms its values where they lie and parks
    // them as bf16 in its wave's part of the (now free) ring, 16 rows at a
    // time; the rows are then read back contiguous, 16 bytes per lane, and
    // leave as one 16-byte store.  The int32 output parks the accumulators
    // themselves.
    const int q4 = lane >> 4;
    float swv[NB];
    float sx_own = 0.0f;
    if constexpr (EP != Epilogue::S32) {
        if (tid < BM) sx_own = sx[tid < rows_a ? m0 + tid : M - 1];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int c;
            if constexpr (EP == Epilogue::SWIGLU)
                c = tile.tn * (BN / 2) + 64 * wn + 16 * (b & 3) + fr;
            else
                c = tile.tn * BN + 128 * wn + 16 * b + fr;
            c = c < N ? c : N - 1;
            swv[b] = sw[(EP == Epilogue::SWIGLU && b >= 4 ? N : 0) + c];
        }
    }
    lds_barrier();   // every wave is done reading the ring
    float* sx_lds = reinterpret_cast<float*>(lds + SX_OFFSET);
    if constexpr (EP != Epilogue::S32) {
        if (tid < BM) sx_lds[tid] = sx_own;
        lds_barrier();
    }
    const int grow0 = m0 + WROWS * wm;
    const int col0 = epi_col0;
    const int cg = epi_cg;
    const int ro = epi_ro;
    const bool vec_cols = (col0 + 8 <= N) && (N % 8 == 0);

    if constexpr (EP == Epilogue::S32) {
        int32_t* stash = reinterpret_cast<int32_t*>(lds + wave * STASH_WAVE_BYTES);
        int32_t* o = reinterpret_cast<int32_t*>(out);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) stash[(4 * q4 + r) * PITCH + 16 * b + fr] = acc[a][b][r];
            asm volatile("" ::: "memory");
#pragma nounroll
            for (int it = 0; it < 4; ++it) {
                const int lr = 4 * it + ro;
                const int grow = grow0 + 16 * a + lr;
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
        // the four lane quarters (rows 4 apart) write disjoint banks
        constexpr int NBO = EP == Epilogue::SWIGLU ? 4 : 8;    // output blocks per wave row
        constexpr int P16 = 16 * NBO + 8;
        constexpr int ROW_STEP = EP == Epilogue::SWIGLU ? 8 : 4;   // rows per read-back
        constexpr int ITS = 16 / ROW_STEP;
        uint16_t* st16 = reinterpret_cast<uint16_t*>(lds + wave * (16 * P16 * 2));
        uint16_t* y = reinterpret_cast<uint16_t*>(out);
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            // row scales of the lane's rows 16 a + 4 (l / 16) + r
            const v4f s4 = *reinterpret_cast<const v4f*>(sx_lds + WROWS * wm + 16 * a + 4 * q4);
            const float sxr[4] = {s4.x, s4.y, s4.z, s4.w};
            asm volatile("" ::: "memory");
#pragma unroll
            for (int bb = 0; bb < NBO; ++bb)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    float v0, v1;
                    if constexpr (EP == Epilogue::SWIGLU) {
                        v0 = swiglu_hw(dequant(acc[a][bb][r], sxr[r], swv[bb]),
                                       dequant(acc[a][bb + 4][r], sxr[r], swv[bb + 4]));
                        v1 = swiglu_hw(dequant(acc[a][bb][r + 1], sxr[r + 1], swv[bb]),
                                       dequant(acc[a][bb + 4][r + 1], sxr[r + 1], swv[bb + 4]));
                    } else {
                        v0 = dequant(acc[a][bb][r], sxr[r], swv[bb]);
                        v1 = dequant(acc[a][bb][r + 1], sxr[r + 1], swv[bb]);
                    }
                    const uint32_t pk = pack_bf16(v0, v1);
                    const int row = 4 * q4 + r;   // rows row, row + 1
                    st16[row * P16 + 16 * bb + fr] = (uint16_t)pk;
                    st16[(row + 1) * P16 + 16 * bb + fr] = (uint16_t)(pk >> 16);
                }
            asm volatile("" ::: "memory");
#pragma unroll
            for (int it = 0; it < ITS; ++it) {
                const int lr = ROW_STEP * it + ro;
                const int grow = grow0 + 16 * a + lr;
                const v4u pk = *reinterpret_cast<const v4u*>(st16 + lr * P16 + 8 * cg);
                if (grow < M) {
                    if (vec_cols) {
                        // written once, never read here: a nontemporal store
                        // keeps the outputs from displacing the operand panels
                        // that other tiles re-read through the caches (0.7 %
                        // and 1.7 % faster on the FFN-up and FFN-down shapes)
                        __builtin_nontemporal_store(pk, reinterpret_cast<v4u*>(y + (int64_t)grow * N + col0));
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
