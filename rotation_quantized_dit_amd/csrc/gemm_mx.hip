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
// The main loop has the int8 kernel's schedule: copies issued from inline
// assembly (so the compiler does not drain them before every fragment read),
// a fixed MFMA order with each fragment register (and its block scale)
// refilled right after its last use, the stage barrier after the fourth MFMA
// of the second k-step, four of the six refill copies spread over that
// k-step and the other two in the next stage's first k-step, copies
// past the last stage pushed out of the buffer's range, and the stage loop
// unrolled over the ring's three slots so that every LDS offset is an
// immediate (without that the slot arithmetic needs registers the loop does
// not have).
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
// Ragged rows lie past their panel's buffer range, load as zeros and are
// masked at the store; K must be a multiple of 128.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
// epilogue: each wave parks 32 rows x 128 bf16 at a time, rows padded to P16
constexpr int P16 = 136;
constexpr int STASH_BYTES = NWAVES * 32 * P16 * 2;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = RING_BYTES + 1024 > STASH_BYTES ? RING_BYTES + 1024 : STASH_BYTES;   // ring + spare
constexpr int GROUP_M = 4;                   // M-tiles per raster group
static_assert(SPARE + 1024 <= LDS_BYTES, "spare area");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

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

// Buffer resource words over [base, base + bytes) (raw, no stride; gfx9
// dword 3), uniform across the wave.
__device__ __forceinline__ v4u rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    v4u r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)b);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000u;
    return r;
}
// One direct copy: 64 lanes x 16 bytes from rsrc + voff + soff into LDS at
// lds_addr + 16 * lane (M0 holds the LDS address; no VGPR is written).
__device__ __forceinline__ void dma16(v4u rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(lds_addr));
}
// Past-the-end offset for copies of stages beyond the last: beyond any
// buffer's num_records (< 2^31), so the load returns zeros and reads nothing.
constexpr uint32_t OOB = 0x80000000u;

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

    const v4u rsrc_a = rsrc_words(A + (int64_t)m0 * KB, (uint32_t)rows_a * (uint32_t)KB);
    const v4u rsrc_b = rsrc_words(B + (int64_t)n0 * KB, (uint32_t)rows_b * (uint32_t)KB);
    // scale copies: waves 0 and 1 the tile's A scale words (rows 256 w + 4 l .. +3; the upper half of
    // wave 1's copy reads rows past the tile into the unused end of the A scale area), wave 2 the B
    // words; waves 3-7 issue the same instruction on an empty resource into a spare area
    const v4u rsrc_s =
        wave < 2 ? rsrc_words(SA + (int64_t)m0 * 4, (uint32_t)((int64_t)(KT - 1) * M * 4 + rows_a * 4))
        : wave == 2 ? rsrc_words(SB + (int64_t)n0 * 4, (uint32_t)((int64_t)(KT - 1) * N * 4 + rows_b * 4))
                    : rsrc_words(SB, 0u);
    const uint32_t chunk_stride = wave < 2 ? (uint32_t)M * 4u : wave == 2 ? (uint32_t)N * 4u : 0u;
    const uint32_t voff_s = (uint32_t)(wave < 2 ? 1024 * wave : 0) + 16u * (uint32_t)lane;
    const int s_dst = wave < 2 ? A_STAGE + B_STAGE + 1024 * wave
                      : wave == 2 ? A_STAGE + B_STAGE + SA_BYTES : SPARE;
    // Row rr of a copy is read at rr * KB + its swizzled chunk; rows past the
    // tile's last row lie past the buffer's range and read as zeros (their
    // outputs are masked at the store).  Consecutive copies of a wave are 16
    // rows apart and share the swizzle ((rr >> 2) & 3 = (lane >> 4) & 3).
    const uint32_t chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t voff_a = (uint32_t)(16 * MA * wave + (lane >> 2)) * (uint32_t)KB + chunk;
    const uint32_t voff_b = (uint32_t)(32 * wave + (lane >> 2)) * (uint32_t)KB + chunk;
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds);
    // copy i of stage kt into slot: i < MA A rows, MA, MA + 1 B rows, MA + 2 the scale words
    auto issue = [&](int i, int kt, uint32_t oob, int slot) {
        const uint32_t st = lds_base + slot * STAGE_BYTES;
        const uint32_t soff = (uint32_t)kt * BK;
        if (i < MA) dma16(rsrc_a, st + 16 * 64 * MA * wave + 1024 * i, voff_a + (16u * i * KB + oob), soff);
        else if (i < MA + 2)
            dma16(rsrc_b, st + A_STAGE + 32 * 64 * wave + 1024 * (i - MA), voff_b + (16u * (i - MA) * KB + oob), soff);
        else dma16(rsrc_s, (wave < 3 ? st : lds_base) + s_dst, voff_s + oob, (uint32_t)kt * chunk_stride);
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
    const int sw = swz(lane & 31);
    const int a_lane = (32 * MA * wm + (lane & 31)) * BK;
    const int b_lane = A_STAGE + (128 * wn + (lane & 31)) * BK;
    // A row's scale word holds the block scales of its 128 elements; the
    // lanes of half g use block 2 s + g in k-step s (one byte read).
    const int sa_byte = A_STAGE + B_STAGE + 4 * (32 * MA * wm + (lane & 31)) + g;
    const int sb_byte = A_STAGE + B_STAGE + SA_BYTES + 4 * (128 * wn + (lane & 31)) + g;
    const int c0 = 16 * ((0 + g) ^ sw), c1 = 16 * ((2 + g) ^ sw);

#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
        for (int i = 0; i < COPIES; ++i) issue(i, st, st < KT ? 0u : OOB, st);
    wait_vmcnt<(STAGES - 1) * COPIES>();
    lds_barrier();

    v4i fa[MA], fb[4];
    int sa[MA], sb[4];
#pragma unroll
    for (int a = 0; a < MA; ++a) {
        fa[a] = *reinterpret_cast<const v4i*>(lds + a_lane + c0 + 2048 * a);
        sa[a] = lds[sa_byte + 128 * a];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        fb[b] = *reinterpret_cast<const v4i*>(lds + b_lane + c0 + 2048 * b);
        sb[b] = lds[sb_byte + 128 * b];
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);

    constexpr int SA_[12] = {0, 0, 0, 0, 1, 2, 1, 2, 1, 2, 1, 2};
    constexpr int SB_[12] = {0, 1, 2, 3, 0, 0, 1, 1, 2, 2, 3, 3};
    auto mfma = [&](int i, int s) {
        const int a = SA_[i], b = SB_[i];
        const v8i av = {fa[a].x, fa[a].y, fa[a].z, fa[a].w, 0, 0, 0, 0};
        const v8i bv = {fb[b].x, fb[b].y, fb[b].z, fb[b].w, 0, 0, 0, 0};
        (void)s;
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[a][b], 4, 4, 0, sa[a], 0, sb[b]);
    };
    // refill after slot i with the fragments of k-step s of stage st (and, for
    // k-step 0 of the next stage, the scale words)
    auto refill = [&](int i, const uint8_t* st, int s) {
        const int c = s == 0 ? c0 : c1;
        auto fa_ = [&](int a) {
            fa[a] = *reinterpret_cast<const v4i*>(st + a_lane + c + 2048 * a);
            sa[a] = st[sa_byte + 128 * a + 2 * s];
        };
        auto fb_ = [&](int b) {
            fb[b] = *reinterpret_cast<const v4i*>(st + b_lane + c + 2048 * b);
            sb[b] = st[sb_byte + 128 * b + 2 * s];
        };
        if (i == 3) fa_(0);
        if (i == 5) fb_(0);
        if (i == 7) fb_(1);
        if (i == 9) fb_(2);
        if (i == 11) {
            fb_(3);
            fa_(1);
            fa_(2);
        }
    };
    // copies 0-3 of a refill go out after slots CS[] of the k-step that
    // follows the barrier, copies 4 and 5 after slots 0 and 6 of the next
    // stage's first k-step (before the first refill: stage STAGES - 1
    // again, the same bytes into its slot)
    constexpr int COPIES_NOW = 4;
    constexpr int CS[COPIES_NOW] = {4, 6, 8, 10};
    constexpr int BARRIER_AFTER = 3;
    // One stage with its ring slot known at compile time (every LDS offset an
    // immediate); the stage loop runs in rounds of STAGES.
    auto stage = [&](auto slot_c, int kt) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int next = slot + 1 == STAGES ? 0 : slot + 1;
        constexpr int prev_slot = slot == 0 ? STAGES - 1 : slot - 1;
        const uint32_t oob = kt + STAGES < KT ? 0u : OOB;
        const int prev_kt = kt > 0 ? kt - 1 + STAGES : STAGES - 1;
        const uint32_t prev_oob = prev_kt < KT ? 0u : OOB;
        const uint8_t* cur = lds + slot * STAGE_BYTES;
        const uint8_t* nxt = lds + next * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mfma(i, 0);
            refill(i, cur, 1);
            if (i == 0) issue(COPIES_NOW, prev_kt, prev_oob, prev_slot);
            if (i == 6) issue(COPIES_NOW + 1, prev_kt, prev_oob, prev_slot);
        }
#pragma unroll
        for (int i = 0; i <= BARRIER_AFTER; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            mfma(i, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(STAGES - 2) * COPIES>();
        lds_barrier();
#pragma unroll
        for (int i = 0; i < 12; ++i) {
            __builtin_amdgcn_sched_barrier(0);
            if (i > BARRIER_AFTER) mfma(i, 1);
            if (i == BARRIER_AFTER) {
#pragma unroll
                for (int j = 0; j <= BARRIER_AFTER; ++j) refill(j, nxt, 0);
            } else if (i > BARRIER_AFTER) {
                refill(i, nxt, 0);
            }
#pragma unroll
            for (int j = 0; j < COPIES_NOW; ++j)
                if (CS[j] == i) issue(j, kt + STAGES, oob, slot);
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
    // the deferred copies of the last refill (out of range)
    issue(COPIES_NOW, KT - 1 + STAGES, OOB, (KT - 1) % STAGES);
    issue(COPIES_NOW + 1, KT - 1 + STAGES, OOB, (KT - 1) % STAGES);
    wait_vmcnt<0>();

    // Epilogue.  Lane l, register r of accumulator block (a, b) holds row
    // 32 a + 8 (r / 4) + 4 (l / 32) + r % 4 and column 32 b + l % 32 of the
    // wave's 96 x 128 sub-tile.  Each lane rounds its values to bf16 where
    // they lie and parks them in its wave's part of the (now free) ring, 32
    // rows at a time, rows padded to P16 bf16 so that the two lane halves
    // (rows r and r + 4) write disjoint banks; the rows are then read back
    // contiguous, 16 bytes per lane, and leave as one 16-byte store.
    lds_barrier();
    uint16_t* st16 = reinterpret_cast<uint16_t*>(lds + wave * (32 * P16 * 2));
    const int grow0 = m0 + 32 * MA * wm;
    const int cg = lane % 16, ro = lane / 16;
    const int col0 = n0 + 128 * wn + 8 * cg;
    const bool vec_cols = (col0 + 8 <= N) && (N % 8 == 0);
    const int l31 = lane & 31, hl = lane >> 5;
#pragma unroll
    for (int a = 0; a < MA; ++a) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const uint32_t pk = pack_bf16(acc[a][b][r], acc[a][b][r + 1]);
                const int row = 8 * (r >> 2) + 4 * hl + (r & 3);   // rows row, row + 1
                st16[row * P16 + 32 * b + l31] = (uint16_t)pk;
                st16[(row + 1) * P16 + 32 * b + l31] = (uint16_t)(pk >> 16);
            }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int lr = 4 * it + ro;
            const int grow = grow0 + 32 * a + lr;
            const v4u pk = *reinterpret_cast<const v4u*>(st16 + lr * P16 + 8 * cg);
            if (grow >= M) continue;
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
