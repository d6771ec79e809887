// MXFP4 x MXFP4 -> fp32 GEMM with a bf16 epilogue on the gfx950 scaled
// MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, both operands FP4 E2M1), for the
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
// 128-element k-step of FP4 occupies 64 bytes of a row and each lane of a
// 16-row block takes 16 of them (lane l: row l % 16, 32-element block l / 16),
// exactly the layout of the int8 operands of K-GEMM (64 bytes of K per
// v_mfma_i32_16x16x64_i8), so the tiling is that kernel's: a 384 x 256 tile,
// 8 waves (two per SIMD) in a 4 x 2 grid of 96 x 128 wave tiles (6 x 8 MFMA
// blocks, 192 fp32 accumulators per lane), one MFMA k-step (64 bytes, 128
// elements) per stage through a 3-slot LDS ring of direct buffer loads,
// XOR-swizzled 64-byte rows.  The 384-row tile copies 17 % fewer bytes per
// flop than a 256-row one and measured about 8 % faster on the FFN-input
// shape (with the 32 x 32 x 64 form of the MFMA).
//
// The main loop has the int8 kernel's schedule: copies issued from inline
// assembly (so the compiler does not drain them before every fragment read);
// each stage as 8 phases, one per B block, with the six A fragments held for
// the stage and B double-buffered; the stage barrier after the fourth MFMA of
// the seventh phase; the last phase reading the next slot; four of the six
// refill copies after the barrier and the other two in the next stage's first
// phases; copies past the last stage pushed out of the buffer's range; the
// stage loop unrolled over the ring's three slots.  Against the 32 x 32 x 64
// form of the same design it measured 0-2 % faster, and its main loop holds
// every value in registers.
//
// Each stage also carries the tile's scale words (one 32-bit word per row:
// the 4 block scales of its 128 elements), 384 + 256 words copied as three
// 1 KiB direct loads: waves 0 and 1 take the A rows (the upper half of wave
// 1's copy reads rows past the tile into unused space), wave 2 the B rows.
// So that the copy needs no branch, waves 3-7 issue the same load on an
// empty buffer resource (every lane out of range: no memory is read) into a
// spare 1 KiB of LDS.  For each fragment a lane reads the one scale byte it
// needs, block l / 16 of its row, with a byte load from LDS.
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
constexpr int MA = BM / 128;                 // 16-row copies of A per wave per stage (96 rows / 32)
constexpr int NA = 6;                        // 16-row A blocks per wave (MFMA rows)
constexpr int NB = 8;                        // 16-column B blocks per wave (MFMA columns)
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
// epilogue: each wave parks 16 rows x 128 bf16 at a time, rows padded to P16
constexpr int P16 = 136;
constexpr int STASH_BYTES = NWAVES * 16 * P16 * 2;
constexpr int RING_BYTES = STAGES * STAGE_BYTES;
constexpr int LDS_BYTES = RING_BYTES + 1024 > STASH_BYTES ? RING_BYTES + 1024 : STASH_BYTES;   // ring + spare
constexpr int GROUP_M = 4;                   // M-tiles per raster group
static_assert(SPARE + 1024 <= LDS_BYTES, "spare area");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

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
    // rows apart and share the swizzle ((rr >> 1) & 3 = (lane >> 3) & 3).
    const uint32_t chunk = 16u * (uint32_t)((lane & 3) ^ ((lane >> 3) & 3));
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

    v4f acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Fragment reads.  v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands
    // takes, in lane l, row l % 16 of a 16-row block and the 32 elements (16
    // bytes) of block l / 16 of the stage's 128, with that block's scale.
    // Every block starts at a row that is a multiple of 16, so the swizzle
    // (row >> 1) & 3 depends on the lane alone and block i of a panel lies
    // 1 KiB (codes) or 64 bytes (scale words) after block i - 1.
    const int fr = lane & 15;
    const int fpos = 16 * ((lane >> 4) ^ ((fr >> 1) & 3));
    const int a_base = (32 * MA * wm + fr) * BK + fpos;
    const int b_base = A_STAGE + (128 * wn + fr) * BK + fpos;
    const int sa_base = A_STAGE + B_STAGE + 4 * (32 * MA * wm + fr) + (lane >> 4);
    const int sb_base = A_STAGE + B_STAGE + SA_BYTES + 4 * (128 * wn + fr) + (lane >> 4);

#pragma unroll
    for (int st = 0; st < STAGES; ++st)
#pragma unroll
        for (int i = 0; i < COPIES; ++i) issue(i, st, st < KT ? 0u : OOB, st);
    wait_vmcnt<(STAGES - 1) * COPIES>();
    lds_barrier();

    v4i fa[NA], fb[2];
    int sa[NA], sb[2];
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        fa[a] = *reinterpret_cast<const v4i*>(lds + a_base + 1024 * a);
        sa[a] = lds[sa_base + 64 * a];
    }
    fb[0] = *reinterpret_cast<const v4i*>(lds + b_base);
    sb[0] = lds[sb_base];
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);

    // A stage is NB phases of NA MFMAs: phase j multiplies every A block with
    // B block j (in fb[j & 1]), and B block j + 1 is read at the start of
    // phase j.  The stage barrier follows MFMA BARRIER_AT (in phase NB - 2);
    // phase NB - 1 then reads the next slot: its first B block at the phase's
    // start and each A block right after that block's last MFMA.  Copies
    // 0..COPIES_NOW - 1 of a refill go out after MFMAs CS[] of the stage,
    // after the barrier, the others after MFMAs 0 and 12 of the next stage.
    constexpr int BARRIER_AT = NA * (NB - 2) + 3;
    constexpr int COPIES_NOW = 4;
    constexpr int CS[COPIES_NOW] = {BARRIER_AT + 1, BARRIER_AT + 3, BARRIER_AT + 5, BARRIER_AT + 7};
    static_assert(BARRIER_AT + 7 < NA * NB, "copies inside the stage");
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
        for (int j = 0; j < NB; ++j) {
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int idx = NA * j + i;
                __builtin_amdgcn_sched_barrier(0);
                const v8i av = {fa[i].x, fa[i].y, fa[i].z, fa[i].w, 0, 0, 0, 0};
                const v8i bv = {fb[j & 1].x, fb[j & 1].y, fb[j & 1].z, fb[j & 1].w, 0, 0, 0, 0};
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc[i][j], 4, 4, 0, sa[i], 0,
                                                                             sb[j & 1]);
                if (i == 0 && j + 1 < NB) {
                    fb[(j + 1) & 1] = *reinterpret_cast<const v4i*>(cur + b_base + 1024 * (j + 1));
                    sb[(j + 1) & 1] = cur[sb_base + 64 * (j + 1)];
                }
                if (idx == 0) issue(COPIES_NOW, prev_kt, prev_oob, prev_slot);
                if (idx == 12) issue(COPIES_NOW + 1, prev_kt, prev_oob, prev_slot);
                if (idx == BARRIER_AT) {
                    __builtin_amdgcn_sched_barrier(0);
                    wait_vmcnt<(STAGES - 2) * COPIES>();
                    lds_barrier();
                }
                if (j == NB - 1) {
                    if (i == 0) {
                        fb[0] = *reinterpret_cast<const v4i*>(nxt + b_base);
                        sb[0] = nxt[sb_base];
                    }
                    fa[i] = *reinterpret_cast<const v4i*>(nxt + a_base + 1024 * i);
                    sa[i] = nxt[sa_base + 64 * i];
                }
#pragma unroll
                for (int c = 0; c < COPIES_NOW; ++c)
                    if (CS[c] == idx) issue(c, kt + STAGES, oob, slot);
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
    // the deferred copies of the last refill (out of range)
    issue(COPIES_NOW, KT - 1 + STAGES, OOB, (KT - 1) % STAGES);
    issue(COPIES_NOW + 1, KT - 1 + STAGES, OOB, (KT - 1) % STAGES);
    wait_vmcnt<0>();

    // Epilogue.  Lane l, register r of accumulator block (a, b) holds row
    // 16 a + 4 (l / 16) + r and column 16 b + l % 16 of the wave's 96 x 128
    // sub-tile.  Each lane rounds its values to bf16 where they lie and parks
    // them in its wave's part of the (now free) ring, 16 rows at a time, rows
    // padded to P16 bf16 so that the four lane quarters (rows 4 apart) write
    // disjoint banks; the rows are then read back contiguous, 16 bytes per
    // lane, and leave as one 16-byte store.
    lds_barrier();
    uint16_t* st16 = reinterpret_cast<uint16_t*>(lds + wave * (16 * P16 * 2));
    const int grow0 = m0 + 32 * MA * wm;
    const int cg = lane % 16, ro = lane / 16;
    const int col0 = n0 + 128 * wn + 8 * cg;
    const bool vec_cols = (col0 + 8 <= N) && (N % 8 == 0);
    const int q4 = lane >> 4;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                const uint32_t pk = pack_bf16(acc[a][b][r], acc[a][b][r + 1]);
                const int row = 4 * q4 + r;   // rows row, row + 1
                st16[row * P16 + 16 * b + fr] = (uint16_t)pk;
                st16[(row + 1) * P16 + 16 * b + fr] = (uint16_t)(pk >> 16);
            }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int lr = 4 * it + ro;
            const int grow = grow0 + 16 * a + lr;
            const v4u pk = *reinterpret_cast<const v4u*>(st16 + lr * P16 + 8 * cg);
            if (grow >= M) continue;
            if (vec_cols) {
                // written once: nontemporal, as in the int8 kernel
                __builtin_nontemporal_store(pk, reinterpret_cast<v4u*>(out + (int64_t)grow * N + col0));
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
