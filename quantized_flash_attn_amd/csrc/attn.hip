// Non-causal varlen FP8 flash attention for gfx950 (CDNA4).
//
// "FP8 vision encoder attention" (Requirements) runs FP8 attention with
// per-tensor scales over packed variable-length image batches; "FP8 ViT
// Encoder Attention" (intro) feeds it Q/K/V quantized on the fly.  Each
// query attends to every key of its own sequence [cu[b], cu[b+1]).
//
// Inputs are E4M3 codes in HBM (1 byte per element); the kernel works on the
// code values and folds the per-tensor scales into the softmax and epilogue.
// Code rows are always 128 dims wide: a head_dim D below 128 arrives
// zero-padded (the zeros add nothing to Q K^T and give zero output dims),
// the softmax scale is 1/sqrt(D), and only the D real output dims are
// written, to rows D wide.
//
// Work decomposition
//   * One workgroup = 8 waves = one (head, 256-query tile of one sequence);
//     one workgroup per CU (132 KiB of LDS), two waves per SIMD.  Query
//     tiles never cross a cu_seqlens boundary.  Workgroup ids are remapped
//     so that consecutive tiles (same head, same K/V) land on one XCD and
//     share its L2.
//   * Each wave owns 32 queries (two 16-query MFMA blocks) and streams all
//     keys of the sequence in 128-key tiles staged through LDS.
//   * K and V tiles are fetched with buffer_load_dwordx4 ... lds (L2 to LDS
//     without registers): V lands in its swizzled layout, K lands in a
//     staging buffer and is converted to bf16 the period before its use.
//     Rows past the end of the sequence are outside the buffer descriptor's
//     range and arrive as zeros; their scores are masked.
//
// Ping-pong schedule.  Waves 0-3 (group A) and 4-7 (group B) share the four
// SIMDs pairwise.  Each key tile takes four barrier-separated slots, and B
// runs two slots behind A, so on every SIMD one wave issues MFMAs while the
// other issues the softmax VALU work:
//            slot 1          slot 2          slot 3          slot 4
//   A    S_t = K_t Q^T    p_t = 2^(..)    split p_t       O += P_t V_t
//   B    split p_{t-1}    O += P V_{t-1}  S_t = K_t Q^T   p_t = 2^(..)
// (the last quarter of the exponentials of a tile runs with its split, which
// evens out the VALU work of the two groups).
//
//   S = K Q^T       bf16 MFMA on the exactly converted codes (every E4M3 value
//                   is a bf16 value).  gfx950's fp8 MFMAs add each group of
//                   products on a window of about 13 bits below the group's
//                   largest product and truncate the rest; with outlier-heavy
//                   Q/K that moves dominant logits by up to ~0.5 log2 units.
//                   The bf16 MFMA sums exactly.  The accumulator gives every
//                   lane 32 keys of ONE query, so the row max is in-lane plus
//                   two lane swaps.
//   online softmax  p = 2^(S c + 8 - m c), c = s_q s_k log2(e) / sqrt(D), m
//                   a running row max that only moves when a tile's max exceeds
//                   it by more than 0.5 log2 units, so p <= 2^8.5 = 362 < 448
//                   and most tiles skip the rescale.  The 2^8 shift keeps small
//                   p out of E4M3 subnormals.
//   P split         hi = E4M3(p), lo = E4M3(p - hi): two fp8 MFMAs give ~8
//                   significant bits of p.
//   O^T += V^T P^T  A = V^T read with ds_read_b64_tr_b8 from row-major fp8 V
//                   in LDS, B = P^T straight from the S accumulator layout.
//                   l sums the unquantized p in fp32.
//   epilogue        out = bf16(O * s_v / l).

#include <cmath>

#include "attn_common.h"

namespace qfa {
namespace {

using namespace attn;

constexpr int kKRow = 2 * kD + 16;  // bytes per bf16 K row in LDS (256 + 16 B of padding)

// LDS map (bytes): two fp8 K staging buffers | two bf16 K buffers | two fp8
// V buffers = 132 KiB.
constexpr int kK8Buf = kBN * kD;
constexpr int kKbBuf = kBN * kKRow;
constexpr int kVBuf = kBN * kD;
constexpr int kLdsK8 = 0;
constexpr int kLdsKb = kLdsK8 + 2 * kK8Buf;
constexpr int kLdsV = kLdsKb + 2 * kKbBuf;
constexpr int kLdsBytes = kLdsV + 2 * kVBuf;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kLdsV % 128 == 0 && kVBuf % 128 == 0, "V buffers must keep address bits 4..6 free for the swizzle");

__device__ inline v4f mfma_f8(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Four E4M3 codes (one dword) -> four bf16 values, exactly (scale 1).
__device__ inline bf16x4 codes_to_bf16(uint32_t w) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
    return bf16x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ inline bf16x8 codes_to_bf16x8(uint32_t w0, uint32_t w1) {
    const bf16x4 a = codes_to_bf16(w0), b = codes_to_bf16(w1);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// LDS layouts:
//   bf16 K: [key][128] rows padded to 272 B.  The K operand read has 16
//      consecutive rows read the same 16-byte column chunk; the 16-byte pad
//      puts row r's chunk c on banks 4(r + c) mod 64, so the 16 rows hit 16
//      distinct bank quads, and every address is a lane base plus immediates.
//   fp8 V: [key][128] rows of 128 B (8 chunks) as the async loads write
//      them; a transpose read touches rows {16a + 4g + b : a in 0..1,
//      b in 0..3}, so chunk c of row r is stored at chunk c ^ swz_v(r) with
//      swz_v(r) = (r & 3) | ((r >> 4) & 1) << 2.
//   fp8 K staging: unswizzled [key][128].
__device__ inline uint32_t swz_v(uint32_t row) { return (row & 3) | ((row >> 2) & 4); }

// Asynchronous fetch of one 128-key tile of K (fp8 staging) or V: wave w
// fills the 1 KiB segments 2w and 2w + 1 (tile rows [16w, 16w + 16)); lane
// l of a segment writes LDS bytes [16l, 16l + 16), so the V swizzle is
// applied by choosing which global chunk each lane reads.  Each segment's
// buffer descriptor starts at this head's slice of its first row and ends
// after the last row of the sequence: rows past it are out of range, which
// the hardware turns into zeros in LDS.
__device__ inline void issue_tile_load(const uint8_t* __restrict__ src, uint32_t row_stride, int h, int kt,
                                       int seq_hi, lds_u8* dst, int wave, uint32_t lane_off) {
    const int nrows = min(seq_hi - kt, kBN);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int seg = wave * 2 + r;
        const int rows_left = nrows - seg * 8;
        const int nrec = rows_left > 0 ? (rows_left - 1) * (int)row_stride + kD : 0;
        const size_t off = (size_t)(kt + seg * 8) * row_stride + (size_t)h * kD;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + off), 0, nrec, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + seg * 1024, 16, (int)lane_off, 0, 0, 0);
    }
}

// Everything one wave carries through the key loop.  Lane (r16, g) of a
// 16x16 accumulator holds rows 4g..4g+3 of column r16; every score and
// output block uses that layout (scores: rows = keys, columns = queries;
// output: rows = head dims, columns = queries).
struct Wave {
    const uint8_t* k8;
    const uint8_t* v8;
    uint32_t row_stride;   // bytes between tokens of one head (uniform)
    int h, seq_lo, seq_hi, nt, nk_last, wave;
    float cexp;            // s_q s_k log2(e) / sqrt(128)
    // per-lane offsets
    uint32_t k_rd;         // K operand: r16 * 272 + 64 g inside a bf16 K buffer
    uint32_t v_rd;         // V transpose read: key0 * 128 + 8 hh, swizzle in bits 4..6
    uint32_t g_k, g_v;     // async loads: row-in-segment * stride + 16-byte chunk (V: swizzled)
    uint32_t cv_src, cv_dst;  // K conversion inside a half tile: staging chunk / padded bf16 position
    int g4;                // 4 g: first key row of this lane inside a 16-key block
    bf16x8 q[kQB][4];      // Q operand (B of S = K Q^T)
    float m[kQB];          // running row max of the raw scores (lags by <= slack / c)
    v4f o[8][kQB];         // O^T blocks [d block][query block]
    float l[kQB];          // running sum of p over the keys this lane holds (reduced over the quad at the end)

    __device__ __forceinline__ void load_k(lds_u8* lds, int t, int buf) const {
        issue_tile_load(k8, row_stride, h, seq_lo + t * kBN, seq_hi, lds + kLdsK8 + buf * kK8Buf, wave, g_k);
    }
    __device__ __forceinline__ void load_v(lds_u8* lds, int t, int buf) const {
        issue_tile_load(v8, row_stride, h, seq_lo + t * kBN, seq_hi, lds + kLdsV + buf * kVBuf, wave, g_v);
    }
    // fp8 K staging -> bf16 K (exact) for half hf of a tile (rows 64hf..64hf+63),
    // by the 256 threads of one group: thread u converts the 16-byte staging
    // chunks 512hf + u and 512hf + u + 256 (rows 64hf + (u >> 3) + 32r, 16
    // codes each) into two adjacent 16-byte chunks of the padded bf16 row.
    __device__ __forceinline__ void convert_half(unsigned char* smem, int buf, int hf) const {
        const unsigned char* src = smem + kLdsK8 + buf * kK8Buf + hf * (kK8Buf / 2) + cv_src;
        unsigned char* dst = smem + kLdsKb + buf * kKbBuf + hf * 64 * kKRow + cv_dst;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const u32x4 w = *(const u32x4*)(src + r * kGroupThreads * 16);
            *(bf16x8*)(dst + r * 32 * kKRow) = codes_to_bf16x8(w[0], w[1]);
            *(bf16x8*)(dst + r * 32 * kKRow + 16) = codes_to_bf16x8(w[2], w[3]);
        }
    }
    // V^T operand of O^T += V^T P^T for d block db.  Transpose read: in each
    // 16-lane group, lane r receives byte j from the address of lane
    // 2j + (r >> 3), offset r & 7.  Lane 2j + hh of group g points at key
    // 32*rho + 16*(j>>2) + 4g + (j&3), column 16*db + 8*hh, so lane r gets 8
    // keys of column 16*db + r in the key order the P^T operand uses.
    __device__ __forceinline__ v8i read_v(const unsigned char* vbase, int db) const {
        const unsigned char* base = vbase + (v_rd ^ (uint32_t)(db << 4));
        v8i vop;
#pragma unroll
        for (int rho = 0; rho < 4; ++rho) {
            const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(lds_u8*)(base + rho * 32 * kD));
            vop[2 * rho] = t[0];
            vop[2 * rho + 1] = t[1];
        }
        return vop;
    }
};

// S = K Q^T for one key tile: s[kb][qb] holds keys 16kb + 4g + i of query r16.
__device__ __forceinline__ void qk_phase(const Wave& w, const unsigned char* smem, int buf, v4f (&s)[8][kQB]) {
    const unsigned char* kbase = smem + kLdsKb + buf * kKbBuf + w.k_rd;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) s[kb][qb] = v4f{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 kop = *(const bf16x8*)(kbase + kb * 16 * kKRow + c * 16);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) s[kb][qb] = mfma_bf16(kop, w.q[qb][c], s[kb][qb]);
        }
    }
}

// hi = E4M3(p), lo = E4M3(p - hi) for four probabilities: {hi dword, lo dword}.
__device__ __forceinline__ v2i split4(const v4f& p) {
    int h = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
    h = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], h, true);
    const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
    const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
    int l = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] - h01[0], p[1] - h01[1], 0, false);
    l = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] - h23[0], p[3] - h23[1], l, true);
    return v2i{h, l};
}

// The softmax step of a key tile is split over two slots to even out the
// VALU work of the two groups: softmax_head (mask, row max, rescale, and p
// of key blocks [0, kSplit)) and, in the next slot, the remaining key
// blocks followed by the hi/lo split.
constexpr int kSplit = 6;

// P^T operands: phi[qb] / plo[qb] hold the hi / lo codes of keys
// 16kb + 4g + i (dword kb, byte i) of query r16.  l accumulates the
// unquantized p in fp32: normalising by the quantized weights instead would
// drop the mass of the many p below E4M3's subnormal quantum (hi + lo rounds
// them to 0), a bias that would scale the whole output row.
__device__ __forceinline__ void split_phase(const Wave& w, v4f (&p)[8][kQB], int nk, v8i (&phi)[kQB], v8i (&plo)[kQB],
                                            float (&l)[kQB]) {
    exp_blocks<kSplit, 8>(w, p, nk);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        float sum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const v2i cd = split4(p[kb][qb]);
            phi[qb][kb] = cd[0];
            plo[qb][kb] = cd[1];
            sum += (p[kb][qb][0] + p[kb][qb][1]) + (p[kb][qb][2] + p[kb][qb][3]);
        }
        l[qb] += sum;
    }
}

// O^T += V^T P^T for one key tile; the running output accumulates in the
// MFMA accumulator.
__device__ __forceinline__ void pv_phase(Wave& w, const unsigned char* smem, int buf, const v8i (&phi)[kQB],
                                         const v8i (&plo)[kQB]) {
    const unsigned char* vbase = smem + kLdsV + buf * kVBuf;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        const v8i vop = w.read_v(vbase, db);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) w.o[db][qb] = mfma_f8(vop, phi[qb], w.o[db][qb]);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) w.o[db][qb] = mfma_f8(vop, plo[qb], w.o[db][qb]);
    }
}

// The key loop of one wave group.  Period t (t = 0..nt) has four slots
// separated by workgroup barriers:
//            slot 1             slot 2          slot 3             slot 4
//   A (kB=0) S_t = K_t Q^T      p_t (head)      p_t (tail), split, O += P_t V_t
//                                               K_{t+1} (half 1)
//   B (kB=1) p_{t-1} (tail),    O += P V_{t-1}  S_t = K_t Q^T       p_t (head)
//            split, K_{t+1}
//            (half 0)
// Loads: K8_{t+2} at slot 1 (lands by the end of slot 2), V_{t+1} at slot 3
// (lands by the end of slot 4).  Buffer lifetimes: Kb_t is read in slots 1
// (A) and 3 (B) of period t and rewritten with K_{t+2} during period t+1;
// V_t is read in slot 4 of period t (A) and slot 2 of period t+1 (B), and
// rewritten with V_{t+2} at slot 3 of period t+1.
template <bool kB>
__device__ __forceinline__ void key_loop(Wave& w, unsigned char* smem) {
    lds_u8* const lds = (lds_u8*)smem;
    const int nt = w.nt;
    v4f s[8][kQB];
    v8i phi[kQB], plo[kQB];
    for (int t = 0; t <= nt; ++t) {
        const int cur = t & 1, prev = cur ^ 1;
        const int nk_t = (t + 1 < nt) ? kBN : w.nk_last;   // valid keys of tile t (t < nt)
        const int nk_p = (t < nt) ? kBN : w.nk_last;       // valid keys of tile t - 1 (t >= 1)
        // slot 1
        if (t + 2 < nt) w.load_k(lds, t + 2, cur);
        if constexpr (!kB) {
            if (t < nt) qk_phase(w, smem, cur, s);
        } else {
            if (t >= 1) split_phase(w, s, nk_p, phi, plo, w.l);
            if (t + 1 < nt) w.convert_half(smem, prev, 0);
        }
        __syncthreads();
        // slot 2
        if constexpr (!kB) {
            if (t < nt) softmax_head<kSplit>(w, s, nk_t);
        } else {
            if (t >= 1) pv_phase(w, smem, prev, phi, plo);
        }
        wait_async_loads();
        __syncthreads();
        // slot 3
        if (t + 1 < nt) w.load_v(lds, t + 1, prev);
        if constexpr (!kB) {
            if (t < nt) split_phase(w, s, nk_t, phi, plo, w.l);
            if (t + 1 < nt) w.convert_half(smem, prev, 1);
        } else {
            if (t < nt) qk_phase(w, smem, cur, s);
        }
        __syncthreads();
        // slot 4
        if constexpr (!kB) {
            if (t < nt) pv_phase(w, smem, cur, phi, plo);
        } else {
            if (t < nt) softmax_head<kSplit>(w, s, nk_t);
        }
        wait_async_loads();
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8,
    const float* __restrict__ scales, const int32_t* __restrict__ cu, int num_seqs, int num_heads,
    int tiles_per_head, int head_dim, float log2e_rsqrt_d, __bf16* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
    lds_u8* const lds = (lds_u8*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int h = logical / tiles_per_head;
    const int vt = logical - h * tiles_per_head;
    const int b = find_sequence(cu, num_seqs, vt);
    const int seq_lo = cu[b], seq_hi = cu[b + 1];
    const int q0 = seq_lo + (vt - (seq_lo / kBM + b)) * kBM;
    if (q0 >= seq_hi) return;  // spare tile (uniform over the workgroup)

    Wave w;
    w.k8 = k8;
    w.v8 = v8;
    w.row_stride = (uint32_t)num_heads * kD;
    w.h = h;
    w.seq_lo = seq_lo;
    w.seq_hi = seq_hi;
    w.nt = (seq_hi - seq_lo + kBN - 1) / kBN;
    w.nk_last = seq_hi - seq_lo - (w.nt - 1) * kBN;
    w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const bool group_b = w.wave >= kWaves / 2;          // wave-uniform
    {
        // K operand: row 16kb + r16, 16-byte chunk 4g + c.
        w.k_rd = (uint32_t)(r16 * kKRow + 64 * g);
        // V transpose read: key 32rho + 16(j>>2) + 4g + (j&3); its swizzle
        // depends on j only (bit 4 of the key is bit 2 of j).
        const uint32_t j = r16 >> 1, hh = r16 & 1;
        const uint32_t key0 = 16 * (j >> 2) + 4 * g + (j & 3);
        w.v_rd = (key0 * kD + 8 * hh) | (swz_v(key0) << 4);
        // Async loads: lane covers row (lane >> 3) of each 8-row segment and
        // physical chunk lane & 7.  This wave's segments hold rows
        // 16w..16w+15, whose swizzle bit 2 (row bit 4) is w & 1.
        const uint32_t rr = (uint32_t)lane >> 3, pc = (uint32_t)lane & 7;
        const uint32_t row = rr * w.row_stride;
        w.g_k = row + pc * 16;
        w.g_v = row + ((pc ^ swz_v(rr + 16 * ((uint32_t)w.wave & 1))) << 4);
        // K conversion: thread u of its group.
        const uint32_t u = (uint32_t)tid & (kGroupThreads - 1);
        w.cv_src = u * 16;
        w.cv_dst = (u >> 3) * kKRow + (u & 7) * 32;
        w.g4 = 4 * g;
    }
    const int nt = w.nt;

    // ---- prologue: K8_0, K8_1, V_0 in flight; Q operand; K_0 converted ----
    w.load_k(lds, 0, 0);
    if (nt > 1) w.load_k(lds, 1, 1);
    w.load_v(lds, 0, 0);

    // Q operand (B of S = K Q^T, bf16 16x16x32): lane holds query r16 of the
    // block and the 32 head dims [32g, 32g + 32) as four 8-element chunks; the
    // K operand uses the same (lane group, chunk, element) -> dim mapping.
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = q0 + w.wave * (16 * kQB) + qb * 16 + r16;
        u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (qi < seq_hi) {
            const u32x4* src = (const u32x4*)(q8 + (size_t)qi * w.row_stride + (size_t)h * kD + 32 * g);
            a = src[0];
            c = src[1];
        }
        w.q[qb][0] = codes_to_bf16x8(a[0], a[1]);
        w.q[qb][1] = codes_to_bf16x8(a[2], a[3]);
        w.q[qb][2] = codes_to_bf16x8(c[0], c[1]);
        w.q[qb][3] = codes_to_bf16x8(c[2], c[3]);
    }
    const float s_q = scales[0], s_k = scales[1], s_v = scales[2];
    w.cexp = s_q * s_k * log2e_rsqrt_d;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) w.o[db][qb] = v4f{0, 0, 0, 0};
        w.l[qb] = 0.0f;
        w.m[qb] = kMInit;
    }

    wait_async_loads();
    __syncthreads();
    w.convert_half(smem, 0, group_b ? 0 : 1);   // both groups: K_0 complete
    wait_async_loads();
    __syncthreads();

    // ---- key loop: group A runs tile t in period t, group B runs its slots
    // 1-2 on tile t-1 and 3-4 on tile t.  Each group has its own copy of the
    // loop, so its registers are allocated for its own live ranges; both
    // copies execute the same sequence of barriers.
    if (group_b)
        key_loop<true>(w, smem);
    else
        key_loop<false>(w, smem);

    // ---- epilogue: lane holds O^T[d = 16db + 4g + i][query r16]; the output
    // rows hold head_dim dims (a multiple of 8, so a lane's 4 dims are all
    // inside or all past it) ----
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = q0 + w.wave * (16 * kQB) + qb * 16 + r16;
        if (qi < seq_hi) {
            const float f = s_v / quad_sum(w.l[qb]);
            __bf16* dst = out + ((size_t)qi * num_heads + h) * head_dim + 4 * g;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                if (16 * db + 4 * g < head_dim) {
                    bf16x4 r;
                    r[0] = (__bf16)(w.o[db][qb][0] * f);
                    r[1] = (__bf16)(w.o[db][qb][1] * f);
                    r[2] = (__bf16)(w.o[db][qb][2] * f);
                    r[3] = (__bf16)(w.o[db][qb][3] * f);
                    *(bf16x4*)(dst + 16 * db) = r;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_attention(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                            const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads, int head_dim,
                            void* out, hipStream_t s) {
    const int tph = tiles_per_head(total_tokens, num_seqs);
    const long long nwg = (long long)tph * num_heads;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    // log2(e) / sqrt(head_dim) in float32: for head_dim 128 this is the
    // product of the two float32 constants, as before.
    const float rsqrt_d = head_dim == kD ? kRsqrtD : (float)(1.0 / std::sqrt((double)head_dim));
    attn_fwd_kernel<<<(unsigned)nwg, kThreads, 0, s>>>(q8, k8, v8, scales, cu_seqlens, num_seqs, num_heads,
                                                       tph, head_dim, kLog2e * rsqrt_d, (__bf16*)out);
    return hipGetLastError();
}

}  // namespace qfa
