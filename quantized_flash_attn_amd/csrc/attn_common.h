// Pieces shared by the two varlen attention kernels (E4M3 inputs in attn.hip,
// bf16 inputs in attn_bf16.hip): the workgroup shape, the tile -> sequence
// mapping, the XCD-aware workgroup order, the asynchronous tile loads, and
// the online-softmax step.  Both kernels compute non-causal softmax
// attention over packed variable-length sequences ("FP8 vision encoder
// attention", Requirements): each query attends to every key of its own
// sequence [cu[b], cu[b+1]).
#pragma once

#include "qfa_internal.h"

namespace qfa {
namespace attn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kD = 128;             // head_dim
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupThreads = kThreads / 2;
constexpr int kQB = 2;              // 16-query MFMA blocks per wave
constexpr int kBM = kWaves * kQB * 16;  // 256 queries per workgroup
constexpr int kBN = 128;            // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRsqrtD = 0.08838834764831845f;  // 1/sqrt(128)
// Rescale policy of the online softmax.  p = 2^(S c + 8 - mc), with mc the
// running row max in log2 units, is rounded to fp16 (bf16 in the BF16
// kernel) for P V.  mc may lag a tile's max by up to kRescaleSlack units, so
// p <= 2^15.5 stays below fp16's largest value (65504 ~= 2^16); when a
// tile's max exceeds it by more, mc moves kRescaleHeadroom units above that
// max, so the next 11.5 units of growth need no rescale while the largest p
// of the row stays >= 2^4, far from fp16's subnormal range (2^-14).  The
// headroom is a whole number so that the top weight right after a move is
// exactly 2^4 (a one-key row then returns its value row exactly).
constexpr float kRescaleSlack = 7.5f;
constexpr float kRescaleHeadroom = 4.0f;
constexpr int kMaxSplits = 16;                   // key ranges a split launch may use
constexpr float kMInit = -1e30f;                 // finite "no max yet": every first tile rescales, to 0 * O

// Buffer descriptor word 3 for raw byte addressing on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;

// 16x16x32 products with fp32 accumulation: bf16 operands (the BF16 kernel)
// or fp16 operands (the E4M3 kernel, whose codes are all exact in fp16).
__device__ inline v4f mfma16(bf16x8 a, bf16x8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline v4f mfma16(f16x8 a, f16x8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Maximum over the four lanes {l, l^16, l^32, l^48} that hold one query.
__device__ inline float quad_max(float x) {
    const v2i a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const v2i b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

// Sum over the four lanes that hold one query.
__device__ inline float quad_sum(float x) {
    const v2i a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    const v2i b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

__device__ inline void wait_async_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Tile id -> (sequence, query tile).  Sequence b owns the virtual tiles
// [floor(cu[b]/BM) + b, floor(cu[b+1]/BM) + b + 1): enough for its
// ceil(n_b/BM) tiles, at most one spare.  Virtual tiles per head:
// floor(T/BM) + B.  The start positions increase strictly with b, so a
// binary search over cu_seqlens finds the owner.
__device__ inline int find_sequence(const int32_t* __restrict__ cu, int num_seqs, int vt) {
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int start = cu[mid] / kBM + mid;
        if (start <= vt) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Virtual query tiles per head for the mapping above.
inline int tiles_per_head(int total_tokens, int num_seqs) { return total_tokens / kBM + num_seqs; }

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles sharing K/V share an L2.
__device__ inline int xcd_remap(int bid, int nwg) {
    const int q = nwg / 8, r = nwg % 8;
    const int x = bid % 8, k = bid / 8;
    return x * q + min(x, r) + k;
}

// p = 2^(S c + 8 - m c) for key blocks [kLo, kHi) of one key tile with nk
// valid keys, after softmax_head has masked the tile and settled m.  p of
// masked keys is exactly 0 (also where c = 0 made -inf * c a NaN).
template <int kLo, int kHi, class W>
__device__ __forceinline__ void exp_blocks(const W& w, v4f (&s)[8][kQB], int nk) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const float bias = 8.0f - w.mc[qb];
#pragma unroll
        for (int kb = kLo; kb < kHi; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s[kb][qb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], w.cexp, bias));
    }
    if (nk < kBN) {
#pragma unroll
        for (int kb = kLo; kb < kHi; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool dead = w.g4 >= nk - 16 * kb - i;
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) s[kb][qb][i] = dead ? 0.0f : s[kb][qb][i];
            }
    }
}

// Online-softmax step for one key tile with nk valid keys, first part:
// mask the keys past nk and take each query's tile max tm (log2 units).  For
// each 16-query block separately (W::kBlockRescale; else for the wave's 32
// queries together): if tm exceeds the running max mc by more than the slack
// for any of its queries, move mc to max(mc, tm + headroom) for each of them
// and rescale that block's O and l (which hold the earlier tiles) by
// 2^(mc_old - mc_new).  Then turn the scores of key blocks
// [0, kSplit) into p = 2^(S c + 8 - mc); the rest follow with
// exp_blocks<kSplit, 8>.  s[kb][qb] holds keys 16kb + 4g + i of query r16
// (lane (r16, g), g4 = 4g).  W carries mc[kQB], l[kQB], o[8][kQB] (of which
// the first W::kDB dim blocks are live), cexp and g4.
template <int kSplit, class W>
__device__ __forceinline__ void softmax_head(W& w, v4f (&s)[8][kQB], int nk) {
    if (nk < kBN) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool dead = w.g4 >= nk - 16 * kb - i;
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) s[kb][qb][i] = dead ? -INFINITY : s[kb][qb][i];
            }
    }
    float tm[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        tm[qb] = quad_max(mx) * w.cexp;
    }
    auto rescale = [&](int qb) {
        const float mc = fmaxf(w.mc[qb], tm[qb] + kRescaleHeadroom);
        const float alpha = __builtin_amdgcn_exp2f(w.mc[qb] - mc);
        w.mc[qb] = mc;
        w.l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < W::kDB; ++db) w.o[db][qb] *= alpha;
    };
    if constexpr (W::kBlockRescale) {   // one decision per 16-query block
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
            if (__any(tm[qb] - w.mc[qb] > kRescaleSlack)) rescale(qb);
    } else {                            // one decision for the wave's 32 queries
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) grow |= tm[qb] - w.mc[qb] > kRescaleSlack;
        if (__any(grow))
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) rescale(qb);
    }
    exp_blocks<0, kSplit>(w, s, nk);
}

// ---- 16-bit operand tiles in LDS (bf16 in the BF16 kernel, fp16 in the E4M3 kernel) ----
//
// A K tile (both kernels) or V tile (BF16 kernel) is [128 keys][128 dims]
// 16-bit values: rows of 256 B, 16 chunks of 16 B; logical chunk c of row r sits at
// chunk c ^ swz(r).
//   K (A operand of S = K Q^T, ds_read_b128): 16 lanes read rows r..r+15 of
//     one logical chunk; swz_k(r) = r & 15 spreads them over all 16 chunk
//     positions (all 64 banks), and any 8 consecutive lanes over 8 chunks
//     distinct modulo 8.
//   V (V^T operand, ds_read_b64_tr_b16): 32 lanes read 8-byte pieces of
//     rows {4g + e : g in 0..1, e in 0..3} (+ a multiple of 16), a 32-byte
//     span per row; swz_v(r) = (r & 7) << 1 moves the span of row r to
//     32 * (span ^ (r & 7)), 8 distinct spans covering all banks.
constexpr int kRow = 2 * kD;              // bytes per bf16 row (one head of one token)
constexpr int kTileBytes = kBN * kRow;    // 32 KiB per K or V tile
__device__ inline uint32_t swz_k(uint32_t r) { return r & 15; }
__device__ inline uint32_t swz_v(uint32_t r) { return (r & 7) << 1; }

// Lane offsets inside a tile for lane (r16, g).
//   K operand of the c-th QK^T MFMA (dims [32c, 32c + 32), lane group g
//   holding dims 32c + 8g .. + 7): row r16, logical chunk 4c + g, at
//   k_rd ^ (c << 6) (+ 16 rows per key block).
//   V^T transpose read: lane 4e + c of group g points at row 4g + e, dims
//   4c .. 4c + 3 of a 16-dim block, i.e. byte 8c + 32 (4(g & 1) + e) after
//   the swizzle; dim block db at v_rd ^ (db << 5).
__device__ inline uint32_t k_operand_offset(int r16, int g) { return (uint32_t)(r16 * kRow + 16 * (g ^ r16)); }
__device__ inline uint32_t v_operand_offset(int r16, int g) {
    const uint32_t e = (uint32_t)r16 >> 2, c = (uint32_t)r16 & 3;
    return (4 * (uint32_t)g + e) * kRow + 8 * c + 32 * (4 * ((uint32_t)g & 1) + e);
}

// Waves w and w + 4 share a SIMD, and in every slot one of them runs an MFMA
// phase (Q K^T or P V) while the other runs exponentials, packing or code
// conversion.  Without a hint the SIMD favours the older wave,
// so group B's MFMA phases drew out behind A's vector work; raising the
// priority of whichever wave is in an MFMA slot (the product, and in the
// E4M3 kernel's 16x16 layout the code conversion that follows it in the same
// slot) keeps the matrix pipe fed and leaves the vector work to fill its
// gaps.
__device__ __forceinline__ void mfma_phase_begin() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_phase_end() { __builtin_amdgcn_s_setprio(0); }

// S = K Q^T for one key tile over the first kDC 32-dim chunks of the head
// (the rest are zero padding when head_dim < 128): s[kb][qb] holds keys
// 16kb + 4g + i of query r16.  Step n multiplies K operand n (key block
// n / kDC, chunk n % kDC) into both query blocks; each operand is requested
// six steps before its MFMAs issue (the scheduling fence keeps it there), so
// a wave keeps six 1 KiB LDS reads in flight behind its matrix work.
template <int kDC = 4, class T>
__device__ __forceinline__ void qk_tile(const unsigned char* kbase, uint32_t k_rd, const T (&q)[kQB][4],
                                        v4f (&s)[8][kQB]) {
    constexpr int kSteps = 8 * kDC;
    constexpr int kAhead = 6;
    auto operand = [&](int n) {
        return *(const T*)(kbase + (k_rd ^ (uint32_t)((n % kDC) << 6)) + (n / kDC) * 16 * kRow);
    };
    T kop[8];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) kop[n] = operand(n);
#pragma unroll
    for (int n = 0; n < kSteps; ++n) {
        if (n + kAhead < kSteps) kop[(n + kAhead) & 7] = operand(n + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = n / kDC, c = n % kDC;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
            s[kb][qb] = mfma16(kop[n & 7], q[qb][c], c == 0 ? v4f{0, 0, 0, 0} : s[kb][qb]);
    }
}

// p of key blocks [kSplit, 8) (the rest of the softmax step), then the P^T
// operands: pop[qb][j] holds p of keys 32j + 4g + i (elements 0..3) and
// 32j + 16 + 4g + i (elements 4..7) of query r16, rounded to bf16; l
// accumulates the fp32 p.
template <int kSplit, class W>
__device__ __forceinline__ void pack_tile(const W& w, v4f (&p)[8][kQB], int nk, bf16x8 (&pop)[kQB][4],
                                          float (&l)[kQB]) {
    exp_blocks<kSplit, 8>(w, p, nk);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v4f a = p[2 * j][qb], b = p[2 * j + 1][qb];
            pop[qb][j] = bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                                (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
            sum += ((a[0] + a[1]) + (a[2] + a[3])) + ((b[0] + b[1]) + (b[2] + b[3]));
        }
        l[qb] += sum;
    }
}

// V^T operand of O^T += V^T P^T for d block db and 32-key chunk j.
// Transpose read: in each 16-lane group, lane r receives element e from the
// address of lane 4e + (r >> 2), offset r & 3.  Lane 4e + c of group g
// points at key 32j + 16hh + 4g + e, dims 16db + 4c .. 16db + 4c + 3, so lane
// r gets keys 32j + 16hh + 4g + e (e = 0..3) of dim 16db + r: the key order
// of the P^T operand.
__device__ __forceinline__ bf16x8 read_vt(const unsigned char* vbase, uint32_t v_rd, int db, int j) {
    const unsigned char* base = vbase + (v_rd ^ (uint32_t)(db << 5)) + j * 32 * kRow;
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(lds_u8*)base);
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s*)(lds_u8*)(base + 16 * kRow));
    const bf16x4 x = __builtin_bit_cast(bf16x4, a), y = __builtin_bit_cast(bf16x4, b);
    return bf16x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// O^T += V^T P^T for one key tile, over the first kDB 16-dim blocks.
template <int kDB = 8>
__device__ __forceinline__ void pv_tile(const unsigned char* vbase, uint32_t v_rd, const bf16x8 (&pop)[kQB][4],
                                        v4f (&o)[8][kQB]) {
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 vop = read_vt(vbase, v_rd, db, j);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) o[db][qb] = mfma16(vop, pop[qb][j], o[db][qb]);
        }
    }
}

}  // namespace attn
}  // namespace qfa
