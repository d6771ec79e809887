// K-ATTN: int8 Q.K^T / fp16 P.V attention for gfx950.
//
// What it computes (h3-rs README, "Speed": the DiT's attention multiplies int8
// Q by int8 K^T and fp16 P by fp16 V in one flash kernel; hybrid model card,
// "Notes and limitations": the evaluated implementation uses full attention):
//   per token i and head h, Q and K are quantized like any activation row of
//   the layer (s = max|x| / 127 over the head's 128 values, codes rint(x / s),
//   no rotation);
//   logit_ij = acc_ij * s_q[i] * s_k[j] / sqrt(128), acc_ij the exact int32
//   dot product of the codes; O_i = sum_j softmax_j(logit_ij) v_j with v and
//   the probabilities in fp16, sums in fp32, O written as bf16.
//
// Two kernels:
//   prep:  Q, K -> int8 codes [H][S][128] + fp32 scales [H][S]; V -> fp16,
//          transposed per 64-key block ([H][S/64][128][64]), so that the P.V
//          contraction reads 16 contiguous bytes per lane, like every other
//          MFMA operand here.  K, its scales and V are padded to a multiple of
//          64 keys with zeros (masked in the softmax).
//   flash: one workgroup of 8 waves owns 256 queries of one head, 32 per
//          wave; K, V^T and the key scales stream through a 5-slot LDS ring
//          in blocks of 64 keys (25 KiB per slot), copied with the direct
//          buffer loads into LDS.
//
// Orientation.  The logits are computed transposed, S^T = K Q^T (A = 32 keys,
// B = the wave's 32 queries, v_mfma_i32_32x32x32_i8), so that every lane owns
// one query: its running maximum, its row sum and its rescale factor are
// per-lane values with no cross-lane exchange except one swap between the two
// 32-lane halves (which hold the other 16 keys of each 32).  The output is
// also computed transposed, O^T = V^T P^T (A = 32 head dims of V^T, B = P,
// v_mfma_f32_32x32x16_f16), which leaves each lane with 64 output values of
// its own query.
//
// Key order inside P.V.  Lane l of the S^T accumulator holds keys
// 8 (r / 4) + 4 (l / 32) + (r % 4) of each 32-key block (r = 0..15).  Used
// directly as the B operand of two 16-key MFMAs (registers 0-7, then 8-15),
// those are the keys whose 16-block position has bits 2 and 3 swapped.  The
// prep kernel stores V^T with exactly that permutation inside every 32 keys,
// so no register shuffle is needed; the contraction sums over keys, so only
// the pairing of P and V matters.
//
// Softmax.  Logits are kept in base 2: e = t * c - M with t = acc * s_k (fp32)
// and c = s_q * log2(e) / sqrt(128); p = 2^e.  The reference point M is only
// raised when a block's maximum exceeds it by more than 8 (so p <= 256, well
// inside fp16), and then O and the row sum are rescaled by 2^(M_old - M_new);
// softmax is invariant to the choice of M, so this changes rounding only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fixed_math.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int D = 128;                  // head dimension
constexpr int KB = 64;                  // keys per block
constexpr int QW = 32;                  // queries per wave
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int QB = QW * NWAVES;         // queries per workgroup
constexpr int STAGES = 5;
constexpr int K_BYTES = KB * D;         // int8 key codes of a block
constexpr int V_BYTES = KB * D * 2;     // fp16 V^T of a block
constexpr int S_BYTES = KB * 4;         // key scales of a block
constexpr int STAGE_BYTES = 25 * 1024;  // K | V^T | scales, 1 KiB aligned
constexpr int COPIES = 4;               // copies per thread per block
constexpr float TAU = 8.0f;             // lazy-rescale threshold (base 2)
static_assert(K_BYTES + V_BYTES + S_BYTES <= STAGE_BYTES, "stage layout");
static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const v4i lds_v4i;
typedef __attribute__((address_space(3))) const v4f lds_v4f;
typedef __attribute__((address_space(3))) const v8h lds_v8h;
typedef __attribute__((address_space(3))) const uint8_t lds_u8;

// 32-bit LDS address of a pointer into shared memory, and back.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_u8*)p;
}
__device__ __forceinline__ lds_u8* lds_ptr(uint32_t a) { return (lds_u8*)(uintptr_t)a; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Hardware barrier for the ring: the direct copies are complete by the
// explicit vmcnt wait before it, this wave's LDS reads by lgkmcnt(0).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// Direct copies: 64 lanes x 16 (or 4) bytes from rsrc + voff + soff into LDS
// at dst + 16 (or 4) * lane.
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

// LDS rows of K and V^T are 128 bytes (8 chunks of 16); chunk c of row r is
// stored at c ^ swz(r).  A 16-byte read by 16 lanes spans 256 bytes of banks,
// so rows r and r + 2 k must differ in chunk for the 16 rows a fragment read
// touches: (r / 2) % 8 does that (r % 8 would pair rows r and r + 8).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Position of key j inside its 32-key block in V^T: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int j) {
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// max |x| over the 16 lanes of a row group (lanes 16 r .. 16 r + 15).
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ------------------------------------------------------------------ prep

// One workgroup (4 waves) per (head, 64-token block).  Q and K rows: 16 lanes
// per row, 8 values each.  V: the block is transposed through LDS.
__global__ __launch_bounds__(256) void attn_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int64_t ld, int S, int S_pad, int heads, int8_t* __restrict__ qc, float* __restrict__ sq,
    int8_t* __restrict__ kc, float* __restrict__ sk, _Float16* __restrict__ vt) {
    __shared__ _Float16 tile[D][KB + 8];
    const int nblk = S_pad / KB;
    const int h = blockIdx.x / nblk;
    const int blk = blockIdx.x - h * nblk;
    const int tid = threadIdx.x;
    const int sub = tid & 15;            // 8-value slice of a row
    const int row_in = tid >> 4;         // 16 rows per pass

    // Q and K: 4 passes of 16 rows each, for both tensors.
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = which == 0 ? q : k;
        int8_t* codes = which == 0 ? qc : kc;
        float* scales = which == 0 ? sq : sk;
        const int rows_out = which == 0 ? S : S_pad;
#pragma unroll
        for (int pass = 0; pass < KB / 16; ++pass) {
            const int tok = blk * KB + 16 * pass + row_in;
            float x[8];
            if (tok < S) {
                const uint4 raw = *reinterpret_cast<const uint4*>(src + (int64_t)tok * ld + h * D + 8 * sub);
                const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[2 * e] = __uint_as_float(w[e] << 16);
                    x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.0f;
            }
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[e]));
            amax = group16_max(amax);
            const float s = amax / 127.0f;
            uint32_t packed[2] = {0u, 0u};
            if (s != 0.0f) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float n = __builtin_rintf(x[e] / s);
                    n = __builtin_fminf(__builtin_fmaxf(n, -127.0f), 127.0f);
                    packed[e >> 2] |= ((uint32_t)(int)n & 0xffu) << (8 * (e & 3));
                }
            }
            if (tok < rows_out) {
                const int64_t r = (int64_t)h * rows_out + tok;
                *reinterpret_cast<uint2*>(codes + r * D + 8 * sub) = make_uint2(packed[0], packed[1]);
                if (sub == 0) scales[r] = s;
            }
        }
    }

    // V: 64 tokens x 128 dims -> tile[d][pos(j)] in fp16 -> 128 rows of 128 B.
#pragma unroll
    for (int pass = 0; pass < KB / 16; ++pass) {
        const int j = 16 * pass + row_in;
        const int tok = blk * KB + j;
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (tok < S) raw = *reinterpret_cast<const uint4*>(v + (int64_t)tok * ld + h * D + 8 * sub);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        const int pos = (j & ~31) | vt_pos(j & 31);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            tile[8 * sub + 2 * e][pos] = (_Float16)__uint_as_float(w[e] << 16);
            tile[8 * sub + 2 * e + 1][pos] = (_Float16)__uint_as_float(w[e] & 0xffff0000u);
        }
    }
    __syncthreads();
    _Float16* dst = vt + ((int64_t)h * nblk + blk) * (D * KB);
#pragma unroll
    for (int i = 0; i < (D * KB / 8) / 256; ++i) {
        const int c = tid + 256 * i;     // 16-byte chunk: row c / 8, part c % 8
        const int d = c >> 3, part = c & 7;
        *reinterpret_cast<uint4*>(dst + d * KB + 8 * part) =
            *reinterpret_cast<const uint4*>(&tile[d][8 * part]);
    }
}

// ------------------------------------------------------------------ flash

__global__ __launch_bounds__(NTHREADS, 1) void attn_flash_kernel(
    const int8_t* __restrict__ qc, const float* __restrict__ sq, const int8_t* __restrict__ kc,
    const float* __restrict__ sk, const _Float16* __restrict__ vt, int S, int S_pad, int heads,
    uint16_t* __restrict__ out, int64_t ld_out, float c_log2) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * STAGE_BYTES];

    const int nqb = (S + QB - 1) / QB;
    const int h = blockIdx.x / nqb;
    const int q0 = (blockIdx.x - h * nqb) * QB;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 5;             // lane half
    const int l31 = lane & 31;
    const int nb = S_pad / KB;

    // This lane's query: codes as the B operand of the four 32-byte d-steps
    // (bytes 16 (2 s + g) .. +15), and c = s_q log2(e) / sqrt(d).  An
    // all-zero query (s_q = 0) has all-zero codes, so every logit of its row
    // is 0 whatever c is; c = 1 there keeps -inf * c = -inf for masked keys.
    const int qi = q0 + QW * wave + l31;
    const int qr = qi < S ? qi : S - 1;
    const int8_t* qrow = qc + ((int64_t)h * S + qr) * D;
    v4i qf[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[s] = *reinterpret_cast<const v4i*>(qrow + 16 * (2 * s + g));
    const float c_raw = sq[(int64_t)h * S + qr] * c_log2;
    const float c = c_raw > 0.0f ? c_raw : 1.0f;

    // Copy sources (per head): K block rows 8 w + l / 8, V^T block rows
    // 16 w + 8 i + l / 8; lane l lands at chunk position l % 8 of its row,
    // which holds logical chunk (l % 8) ^ swz(row).
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + (int64_t)h * S_pad * D, (uint32_t)S_pad * D);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(vt + (int64_t)h * S_pad * D, (uint32_t)S_pad * D * 2);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sk + (int64_t)h * S_pad, (uint32_t)S_pad * 4);
    const int kr = 8 * wave + (lane >> 3);
    const uint32_t voff_k = (uint32_t)(kr * 128 + 16 * ((lane & 7) ^ swz(kr)));
    uint32_t voff_v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int vr = 16 * wave + 8 * i + (lane >> 3);
        voff_v[i] = (uint32_t)(vr * 128 + 16 * ((lane & 7) ^ swz(vr)));
    }
    auto issue = [&](int b) {
        uint8_t* st = lds + (b % STAGES) * STAGE_BYTES;
        b = b < nb ? b : nb - 1;         // past the end: reload the last block (unused)
        copy16(rk, st + 1024 * wave, voff_k, (uint32_t)b * K_BYTES);
        copy16(rv, st + K_BYTES + 2048 * wave, voff_v[0], (uint32_t)b * V_BYTES);
        copy16(rv, st + K_BYTES + 2048 * wave + 1024, voff_v[1], (uint32_t)b * V_BYTES);
        // every wave copies the same 64 scales (identical writes)
        copy4(rs, st + K_BYTES + V_BYTES, 4u * (uint32_t)lane, (uint32_t)b * S_BYTES);
    };
    auto slot = [&](int b) -> const uint8_t* { return lds + (b % STAGES) * STAGE_BYTES; };

    // Fragment byte offsets within a stage.  K: row 32 kb + l31, chunk
    // 2 s + g; V^T: row 32 db + l31, chunk 4 kb + 2 hh + g; swz(row) = swz(l31).
    // The 32-row block (kb for K, db for V^T) adds a constant 4096 bytes, so
    // each lane keeps 4 + 4 offsets and the block goes into the instruction.
    const int sw = swz(l31);
    int k_lane[4], v_lane[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) k_lane[s] = l31 * 128 + 16 * ((2 * s + g) ^ sw);
#pragma unroll
    for (int kh = 0; kh < 4; ++kh) v_lane[kh] = K_BYTES + l31 * 128 + 16 * ((2 * kh + g) ^ sw);
    // K fragment (kb, s) and V^T fragment (db, kb, hh) of a stage (used
    // outside the main loop)
    auto kfrag = [&](const uint8_t* st, int kb, int s) -> v4i {
        return *reinterpret_cast<const v4i*>(st + k_lane[s] + 4096 * kb);
    };
    auto vfrag = [&](const uint8_t* st, int db, int kb, int hh) -> v8h {
        return *reinterpret_cast<const v8h*>(st + v_lane[2 * kb + hh] + 4096 * db);
    };

    v16f o[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m_ref = -__builtin_inff();
    float lsum = 0.0f;                   // row sum of the lane's query (all keys so far)
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};

    // S^T of a block: 2 key halves x 4 d-steps of int8 MFMA (used alone, in
    // the prologue).
    auto qk = [&](const uint8_t* st, v16i (&acc)[2]) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[kb][r] = 0;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                acc[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kfrag(st, kb, s), qf[s], acc[kb], 0, 0, 0);
            }
        }
    };

    auto rescale = [&](float a) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= a;
    };

    // One pipeline step, written as the instruction stream it should become
    // (sched_barrier fences keep each chunk together):
    //   phase 1: the 8 MFMAs of S^T for the next block (K from st_k), each
    //            with the conversion t = acc * s_k of 4 logits of block kc
    //            (scales from st_s); keys past S are masked on the last block;
    //   phase 2: the 16 MFMAs of O^T += V^T P^T for the previous block (V^T
    //            from st_v, probabilities p_prev), each with 2 probabilities
    //            p = 2^(t c - M) of block kc at the current reference point M
    //            (fp16 rounding and the block's row sum);
    //   check:   if any lane's block sum exceeds 2^TAU (or is not finite: the
    //            first block, where M = -inf), some p may exceed 2^TAU; then
    //            M is raised to the block maximum, the block's p are computed
    //            again, and O (which now holds the previous block too) and
    //            the row sum are rescaled by 2^(M_old - M_new).  Otherwise no
    //            p exceeds the sum, so every p <= 2^TAU, well inside fp16.
    auto step = [&](int kc, const uint8_t* st_k, const uint8_t* st_s, const uint8_t* st_v, bool do_pv,
                    const v16i (&s_cur)[2], v16i (&s_nxt)[2], const v8h (&p_prev)[2][2],
                    v8h (&p_cur)[2][2]) {
        // Per-step fragment base addresses (9 per lane): the slots' LDS
        // addresses are wave-uniform (scalar registers), one vector add each,
        // kept opaque so that the compiler does not re-associate them with
        // the slot arithmetic; each read is then base + the 32-row block
        // offset as an immediate.
        const uint32_t ak = __builtin_amdgcn_readfirstlane(lds_addr(st_k));
        const uint32_t av = __builtin_amdgcn_readfirstlane(lds_addr(st_v));
        const uint32_t as = __builtin_amdgcn_readfirstlane(lds_addr(st_s));
        uint32_t kbase[4], vbase[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kbase[i] = ak + (uint32_t)k_lane[i];
            vbase[i] = av + (uint32_t)v_lane[i];
            asm volatile("" : "+v"(kbase[i]));
            asm volatile("" : "+v"(vbase[i]));
        }
        uint32_t sbase = as + (uint32_t)(K_BYTES + V_BYTES + 16 * g);
        asm volatile("" : "+v"(sbase));
        auto kf_at = [&](int n) -> v4i {     // MFMA n of phase 1: kb = n & 1, s = n >> 1
            return *reinterpret_cast<const lds_v4i*>(lds_ptr(kbase[n >> 1] + 4096 * (n & 1)));
        };
        auto sk_at = [&](int n) -> v4f {     // scales of logits 4 (n & 3) .. of half n >> 2
            return *reinterpret_cast<const lds_v4f*>(lds_ptr(sbase + 128 * (n >> 2) + 32 * (n & 3)));
        };
        auto vf_at = [&](int n) -> v8h {     // MFMA n of phase 2: db = n & 3, kb = n >> 3, hh = (n >> 2) & 1
            return *reinterpret_cast<const lds_v8h*>(
                lds_ptr(vbase[2 * (n >> 3) + ((n >> 2) & 1)] + 4096 * (n & 3)));
        };
        // ---- phase 1 (at raised wave priority: while one wave of a SIMD
        // issues its logits MFMAs, the other's softmax fills the gaps)
        __builtin_amdgcn_s_setprio(1);
        v4i kf[8];
        v4f skv[8];
        float t[2][16];
        kf[0] = kf_at(0);
        skv[0] = sk_at(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i + 1 < 8) {
                kf[i + 1] = kf_at(i + 1);
                skv[i + 1] = sk_at(i + 1);
            }
            {
                const int kb = i & 1, sd = i >> 1;
                s_nxt[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[i], qf[sd],
                                                                  sd == 0 ? v16i{} : s_nxt[kb], 0, 0, 0);
            }
            const int kb = i >> 2, j = i & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[kb][4 * j + e] = (float)s_cur[kb][4 * j + e] * skv[i][e];
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kc == nb - 1) {
            const int nvalid = S - kc * KB;          // 1 .. 64
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) >= nvalid) t[kb][r] = -__builtin_inff();
        }
        __builtin_amdgcn_s_setprio(0);
        // ---- phase 2
        constexpr int VD = 4;                        // V^T fragment prefetch distance
        v8h vf[16];
#pragma unroll
        for (int i = 0; i < VD; ++i) vf[i] = vf_at(i);
        float bs0 = 0.0f, bs1 = 0.0f;
        // p for logits r, r + 1 of half kb, packed into p_cur, summed into bs
        auto prob2 = [&](int kb, int r, float m, float& bs) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kb][r], c, -m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kb][r + 1], c, -m));
            // (the block sum consumes the pair in this basic block, which keeps
            // the pair here rather than sunk to its use in the next step)
            const h2 pp = {(_Float16)p0, (_Float16)p1};
            p_cur[kb][r >> 3][r & 7] = pp[0];
            p_cur[kb][r >> 3][(r & 7) + 1] = pp[1];
            bs = __builtin_amdgcn_fdot2(pp, ones, bs, false);
        };
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i + VD < 16) vf[i + VD] = vf_at(i + VD);
            if (do_pv) {
                const int db = i & 3, kb = i >> 3, hh = (i >> 2) & 1;
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i], p_prev[kb][hh], o[db], 0, 0, 0);
            }
            if (i & 1)
                prob2(i >> 3, 2 * (i & 7), m_ref, bs1);
            else
                prob2(i >> 3, 2 * (i & 7), m_ref, bs0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- check (bs: the block's row sum over both lane halves' keys)
        auto both_halves = [](float x) {
            const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
            return __uint_as_float(w[0]) + __uint_as_float(w[1]);
        };
        float bs = both_halves(bs0 + bs1);
        if (__builtin_amdgcn_ballot_w64(!(bs <= 256.0f)) != 0) {
            float mx0 = __builtin_fmaxf(t[0][0], t[0][1]);
            float mx1 = __builtin_fmaxf(t[1][0], t[1][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) {
                mx0 = __builtin_fmaxf(mx0, __builtin_fmaxf(t[0][r], t[0][r + 1]));
                mx1 = __builtin_fmaxf(mx1, __builtin_fmaxf(t[1][r], t[1][r + 1]));
            }
            float bm = __builtin_fmaxf(mx0, mx1);
            const auto w = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm), __float_as_uint(bm), false,
                                                            false);
            bm = __builtin_fmaxf(__uint_as_float(w[0]), __uint_as_float(w[1]));
            const float m_new = __builtin_fmaxf(m_ref, bm * c);   // c > 0
            const float a = __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            bs0 = 0.0f;
            bs1 = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i & 1)
                    prob2(i >> 3, 2 * (i & 7), m_ref, bs1);
                else
                    prob2(i >> 3, 2 * (i & 7), m_ref, bs0);
            }
            lsum *= a;
            if (do_pv) rescale(a);
            bs = both_halves(bs0 + bs1);
        }
        lsum += bs;
    };
    // O^T += V^T P^T for one block, alone (the last block).
    auto pv = [&](const uint8_t* st, const v8h (&p)[2][2]) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int db = i & 3, kb = i >> 3, hh = (i >> 2) & 1;
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag(st, db, kb, hh), p[kb][hh], o[db], 0, 0, 0);
        }
    };

    // Ring of STAGES slots, block b in slot b % STAGES.  Iteration kt reads
    // slot kt - 1 (V^T for P.V of block kt - 1), slot kt (key scales for the
    // softmax of block kt) and slot kt + 1 (K for the logits of block kt + 1)
    // while blocks kt + 2 and kt + 3 are in flight.
    auto iter = [&](int kt, const v16i (&s_cur)[2], v16i (&s_nxt)[2], const v8h (&p_prev)[2][2],
                    v8h (&p_cur)[2][2]) {
        wait_vmcnt<COPIES>();            // block kt + 1 has landed
        lds_barrier();                   // ... for every wave; slot kt - 2 is free
        issue(kt + 3);
        step(kt, slot(kt + 1), slot(kt), slot(kt + STAGES - 1), kt > 0, s_cur, s_nxt, p_prev, p_cur);
    };

    v16i sa[2], sb[2];
    v8h pa[2][2], pb[2][2];
    issue(0);
    issue(1);
    issue(2);
    wait_vmcnt<2 * COPIES>();            // block 0 has landed
    lds_barrier();
    qk(slot(0), sa);
    // Iterations 0 .. nb - 1; registers alternate between the (a) and (b)
    // sets, two iterations per loop trip.
    iter(0, sa, sb, pb, pa);
    int kt = 1;
    for (; kt + 1 < nb; kt += 2) {
        iter(kt, sb, sa, pa, pb);
        iter(kt + 1, sa, sb, pb, pa);
    }
    if (kt < nb) {                       // one iteration left (kt = nb - 1)
        iter(kt, sb, sa, pa, pb);
        pv(slot(nb - 1), pb);
    } else {
        pv(slot(nb - 1), pa);
    }
    wait_vmcnt<0>();                     // the trailing (unused) copies

    // O / l in bf16 (lsum already holds both lane halves' keys): lane holds
    // head dims 32 db + 8 j + 4 g + i (i = 0..3) of its query.
    if (qi < S) {
        const float inv = 1.0f / lsum;
        uint16_t* orow = out + (int64_t)qi * ld_out + h * D;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = pack_bf16(o[db][4 * j] * inv, o[db][4 * j + 1] * inv);
                const uint32_t hi = pack_bf16(o[db][4 * j + 2] * inv, o[db][4 * j + 3] * inv);
                *reinterpret_cast<uint2*>(orow + 32 * db + 8 * j + 4 * g) = make_uint2(lo, hi);
            }
    }
}

}  // namespace

int64_t attn_pad_keys(int64_t s) { return (s + KB - 1) / KB * KB; }

hipError_t launch_attn_prep(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t ld,
                            int64_t s, int64_t heads, int8_t* qc, float* sq, int8_t* kc, float* sk,
                            void* vt, hipStream_t stream) {
    const int64_t s_pad = attn_pad_keys(s);
    const unsigned grid = (unsigned)(heads * (s_pad / KB));
    hipLaunchKernelGGL(attn_prep_kernel, dim3(grid), dim3(256), 0, stream, q, k, v, ld, (int)s,
                       (int)s_pad, (int)heads, qc, sq, kc, sk, (_Float16*)vt);
    return hipGetLastError();
}

hipError_t launch_attn_flash(const int8_t* qc, const float* sq, const int8_t* kc, const float* sk,
                             const void* vt, int64_t s, int64_t heads, uint16_t* out, int64_t ld_out,
                             hipStream_t stream) {
    const int64_t s_pad = attn_pad_keys(s);
    const unsigned grid = (unsigned)(heads * ((s + QB - 1) / QB));
    // log2(e) / sqrt(128), rounded once to fp32
    const float c_log2 = (float)(1.4426950408889634 / 11.313708498984761);
    hipLaunchKernelGGL(attn_flash_kernel, dim3(grid), dim3(NTHREADS), 0, stream, qc, sq, kc, sk,
                       (const _Float16*)vt, (int)s, (int)s_pad, (int)heads, out, ld_out, c_log2);
    return hipGetLastError();
}

}  // namespace convrot
