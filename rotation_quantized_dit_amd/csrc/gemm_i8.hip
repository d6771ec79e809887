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
//            y[m][j] = bf16_rne(silu(g) * u), silu(g) = g / (1 + exp(-g)).
//
// Tiling.  A workgroup of 4 waves owns a 256 x 256 tile of acc (for SwiGLU:
// 256 tokens x 128 gate columns + the matching 128 up columns, so every lane
// holds g and u of the same output element).  Each wave owns 128 x 128 as
// 4 x 4 blocks of v_mfma_i32_32x32x32_i8 (32 x 32 outputs, 32 bytes of K per
// instruction, 16 int32 accumulators per lane per block).  K advances 64
// bytes per stage through a 3-stage LDS ring (32 KiB per stage).
//
// Operand streaming.  Both operands are K-contiguous rows (q_x is [M, K] and
// q_w is [N, K]), which is the MFMA operand layout: a lane takes 16
// contiguous bytes of one row.  Global -> LDS copies use the gfx950 direct
// load (global_load_lds_dwordx4: 64 lanes x 16 B land contiguously in LDS, no
// VGPR staging).  Each LDS row is 64 bytes (4 chunks of 16 B); chunk c of row r
// is stored at position c ^ ((r >> 2) & 3), which makes the 16-byte fragment
// reads of 16 consecutive rows hit distinct banks.  The XOR is applied on the
// global address side, so the DMA writes stay contiguous.
//
// Scheduling.  Workgroups are dealt round-robin to the 8 XCDs; the tile id is
// remapped so that each XCD walks a contiguous range of tiles in a grouped
// raster (8 M-tiles per group), so workgroups that run together on one XCD
// share A and B panels in that XCD's L2.
//
// Ragged edges: rows past M or N are clamped to the last row for loading and
// masked at the store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace convrot {
namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int STAGES = 3;
constexpr int NTHREADS = 256;
constexpr int A_STAGE = BM * BK;
constexpr int B_STAGE = BN * BK;
constexpr int STAGE_BYTES = A_STAGE + B_STAGE;
constexpr int GROUP_M = 8;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the LDS ring.  Completion of the direct global->LDS
// copies is established by the explicit vmcnt wait that precedes it, and the
// fragment reads of the previous stage by an lgkmcnt(0) wait; so only the
// hardware barrier is needed, plus a compiler barrier that keeps LDS accesses
// on their side of it.  (A fenced __syncthreads() would drain every
// outstanding prefetch with vmcnt(0).)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    // lgkmcnt(0): this wave's fragment reads are complete before any wave can
    // pass the barrier and refill the slot they read.
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Fixed fp32 exponential (Cody-Waite reduction + degree-7 Taylor, fused
// multiply-adds, exact 2^k scaling); the same algorithm the layer's
// definition fixes, evaluated op for op.
__device__ __forceinline__ float exp_cw(float x) {
    if (x > 88.72f) return __builtin_inff();
    if (x < -86.0f) return 0.0f;
    const float kf = __builtin_rintf(x * 0x1.715476p+0f);
    float r = __builtin_fmaf(-kf, 0x1.62e4p-1f, x);
    r = __builtin_fmaf(-kf, 0x1.7f7d1cp-20f, r);
    float p = 0x1.a01a02p-13f;
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)kf);
}

__device__ __forceinline__ float dequant(int acc, float sx, float sw) {
    float f = (float)acc;
    f = f * sx;
    return f * sw;
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
    __shared__ __attribute__((aligned(1024))) int8_t lds[STAGES * STAGE_BYTES];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const Tile tile = map_tile(blockIdx.x, MT, NT);
    const int m0 = tile.tm * BM;

    // Source rows of this lane's four A and four B direct loads.  Load i of
    // wave w fills LDS rows 16 * (4w + i) .. +15; lane l writes row l / 4 of
    // that slab at chunk position l % 4, which holds logical chunk
    // (l % 4) ^ swz(row).
    const int8_t* a_src[4];
    const int8_t* b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 16 * (4 * wave + i) + (lane >> 2);
        const int c = (lane & 3) ^ swz(rr);
        int am = m0 + rr;
        am = am < M ? am : M - 1;
        a_src[i] = A + (int64_t)am * K + 16 * c;
        int bn;
        if constexpr (EP == Epilogue::SWIGLU) {
            const int n0 = tile.tn * (BN / 2);
            int col = n0 + (rr & 127);
            col = col < N ? col : N - 1;
            bn = rr < 128 ? col : N + col;
        } else {
            bn = tile.tn * BN + rr;
            bn = bn < N ? bn : N - 1;
        }
        b_src[i] = B + (int64_t)bn * K + 16 * c;
    }

    auto issue = [&](int kt, int slot) {
        int8_t* a_dst = lds + slot * STAGE_BYTES + 1024 * (4 * wave);
        int8_t* b_dst = a_dst + A_STAGE;
        const int koff = kt * BK;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(a_src[i] + koff, (lds_void*)(a_dst + 1024 * i), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(b_src[i] + koff, (lds_void*)(b_dst + 1024 * i), 16, 0, 0);
    };

    // LDS offsets of this lane's fragment rows (row part only).
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_row[i] = wm * 128 + 32 * i + (lane & 31);
        if constexpr (EP == Epilogue::SWIGLU)
            b_row[i] = (i < 2 ? 0 : 128) + 64 * wn + 32 * (i & 1) + (lane & 31);
        else
            b_row[i] = wn * 128 + 32 * i + (lane & 31);
    }

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int KT = K / BK;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < KT) issue(st, st);

    for (int kt = 0; kt < KT; ++kt) {
        if (kt < KT - 1)
            wait_vmcnt<8>();
        else
            wait_vmcnt<0>();
        lds_barrier();
        if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);

        const int8_t* As = lds + (kt % STAGES) * STAGE_BYTES;
        const int8_t* Bs = As + A_STAGE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c = 2 * s + (lane >> 5);
            v4i af[4], bf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const v4i*>(As + a_row[i] * BK + 16 * (c ^ swz(a_row[i])));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const v4i*>(Bs + b_row[j] * BK + 16 * (c ^ swz(b_row[j])));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
    }

    // Epilogue.  Block (i, j) lane l register r holds acc row
    // 32 i + 8 (r / 4) + 4 (l / 32) + r % 4 and column 32 j + l % 32 of the
    // wave's 128 x 128 sub-tile.
    const int col_lane = lane & 31;
    const int row_lane = 4 * (lane >> 5);
    if constexpr (EP == Epilogue::SWIGLU) {
        uint16_t* y = reinterpret_cast<uint16_t*>(out);
        const int n0 = tile.tn * (BN / 2) + 64 * wn;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + 32 * j + col_lane;
            if (col >= N) continue;
            const float swg = sw[col];
            const float swu = sw[N + col];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + row_lane + (r & 3);
                    if (row < M) {
                        const float sxr = sx[row];
                        const float g = dequant(acc[i][j][r], sxr, swg);
                        const float u = dequant(acc[i][j + 2][r], sxr, swu);
                        const float sl = g / (1.0f + exp_cw(-g));
                        y[(int64_t)row * N + col] = bf16_rne(sl * u);
                    }
                }
            }
        }
    } else {
        const int n0 = tile.tn * BN + wn * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + 32 * j + col_lane;
            if (col >= N) continue;
            float swc = 0.0f;
            if constexpr (EP == Epilogue::BF16) swc = sw[col];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + row_lane + (r & 3);
                    if (row < M) {
                        if constexpr (EP == Epilogue::S32) {
                            reinterpret_cast<int32_t*>(out)[(int64_t)row * N + col] = acc[i][j][r];
                        } else {
                            reinterpret_cast<uint16_t*>(out)[(int64_t)row * N + col] =
                                bf16_rne(dequant(acc[i][j][r], sx[row], swc));
                        }
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
