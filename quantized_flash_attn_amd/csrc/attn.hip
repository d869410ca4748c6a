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
// zero-padded.  The kernel is instantiated for the number of 32-dim chunks
// (kDC) and 16-dim output blocks (kDB) that cover D, so the padding beyond
// them costs no matrix work (D = 80 or 72: 3 chunks, 5 blocks); the rest of
// the padding adds nothing to Q K^T.  The softmax scale is 1/sqrt(D), and
// only the D real output dims are written, to rows D wide.
//
// Work decomposition
//   * One workgroup = 8 waves = one (head, 256-query tile of one sequence);
//     one workgroup per CU (160 KiB of LDS), two waves per SIMD.  Query
//     tiles never cross a cu_seqlens boundary.  Workgroup ids are remapped
//     so that consecutive tiles (same head, same K/V) land on one XCD and
//     share its L2.
//   * Each wave owns 32 queries and streams all keys of the sequence in
//     128-key tiles staged through LDS.
//   * K and V tiles of codes are fetched with buffer_load_dwordx4 ... lds (L2
//     to LDS without registers) into one staging buffer each; rows past the
//     end of the sequence are outside the buffer descriptor's range and
//     arrive as zeros (their scores are masked).  Once per tile, a wave group
//     converts the codes exactly to fp16 (every E4M3 value is an fp16 value)
//     into double-buffered fp16 tiles:
//     K in the layout of the BF16 baseline kernel (attn_common.h), V
//     transposed (V^T, read by transposed 8-bit LDS reads of the staged
//     codes), so that both products read their LDS operands with
//     ds_read_b128.
//
// Ping-pong schedule.  Waves 0-3 (group A) and 4-7 (group B) share the four
// SIMDs pairwise.  Each key tile takes four barrier-separated slots, and B
// runs two slots behind A, so on every SIMD one wave issues MFMAs while the
// other issues the softmax VALU work:
//            slot 1          slot 2            slot 3          slot 4
//   A    S_t = K_t Q^T    p_t (head)        p_t (tail)      O += P_t V_t
//   B    p_{t-1} (tail)   O += P V_{t-1}    S_t = K_t Q^T   p_t (head)
// plus one code conversion of K and one of V per tile (key_loop says where).
//
// Two register layouts (the Wave and WaveWide structs below):
//   16x16   v_mfma_f32_16x16x32_f16, each wave two 16-query blocks; the
//           conversions follow the P V products.
//   32x32   v_mfma_f32_32x32x16_f16, each wave one 32-query block: half the
//           MFMA instructions and waits for the same LDS bytes, and one lane
//           swap for a row max; the conversions follow the softmax tails.
// The 32x32 layout needs 4-6 % fewer GPU cycles per tile but about 4 % more
// energy per call.  A launch that fills the chip holds the board at its
// power limit, where time is energy over the limit, so it runs the 16x16
// layout; a launch of at most 3/4 as many workgroups as CUs stays below the
// limit at full clock, so it runs the 32x32 layout (head dims above 96; the
// 16x16 layout covers all head dims).
//
//   S = K Q^T       fp16 MFMA on the exactly converted codes.  gfx950's fp8
//                   MFMAs add each group of 8 products on a window of about
//                   13 bits below the group's largest product and truncate
//                   the rest; with outlier-heavy Q/K that moves dominant
//                   logits by up to ~0.5 log2 units.  The fp16 MFMA sums
//                   products of two E4M3 values (at most 8 significant bits)
//                   in fp32.  The 16x16 accumulator gives every lane 32 keys
//                   of ONE query, so the row max is in-lane plus two lane
//                   swaps (32x32: 64 keys, one swap).
//                   qfa_fp8_varlen_attn_fp8qk instead runs S on
//                   v_mfma_f32_16x16x128_f8f6f4 straight from the codes (16x16
//                   layout, head dims above 64): no K conversion and half
//                   the matrix cycles of S, at the price of that truncation,
//                   for inputs without isolated large elements.
//   online softmax  p = 2^(S c + 8 - mc), c = s_q s_k log2(e) / sqrt(D), mc
//                   a running row max (log2 units) that may lag a tile's
//                   max by 7.5 units and, when it must move, moves 4 units
//                   above it; the decision is taken per MFMA query block
//                   (16 or 32 queries), so most blocks skip the O and l
//                   rescale on most tiles.
//   O^T += V^T P^T  fp16 MFMA: A = V^T read with ds_read_b128 from the
//                   converted V^T, B = P^T straight from the S accumulator
//                   layout, rounded to fp16 (11 significant bits; bf16's 8
//                   cost up to 2^-9 of each weight).  Two E4M3 terms of p (hi + lo)
//                   on the fp8 MFMA would cost the same matrix time plus two
//                   slow conversions per pair of p; one E4M3 term is too
//                   coarse.  l is the row sum of the same fp16 p, taken by
//                   16x16x32 MFMAs with a ones (or selector) A operand (8 per
//                   tile, in the P V slot, instead of 64 fp32 adds in the VALU
//                   slot), so O / l is a convex combination of V rows.
//   epilogue        out = bf16(O * s_v / l).

#include <atomic>
#include <cmath>
#include <mutex>

#include "attn_common.h"

namespace qfa {
namespace {

using namespace attn;

// LDS map (bytes): two fp16 K tiles | two fp16 V^T tiles | K code staging |
// V code staging = 160 KiB.  With S on the fp8 MFMA the K codes are read
// as staged, so they are staged twice (double-buffered), at the starts of
// the two fp16 K tiles' space, and the K code staging area is unused.
constexpr int kCodeTile = kBN * kD;   // 16 KiB of E4M3 codes
constexpr int kLdsK = 0;
constexpr int kLdsV = 2 * kTileBytes;
constexpr int kLdsK8 = 4 * kTileBytes;
constexpr int kLdsV8 = kLdsK8 + kCodeTile;
constexpr int kLdsBytes = kLdsV8 + kCodeTile;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// The softmax step of a key tile is split over two slots to even out the
// VALU work of the slots: softmax_head (mask, row max, rescale, and p of key
// blocks [0, kSplit)) and, in the next slot, the remaining key blocks and
// the P^T operands.
constexpr int kSplit = 4;

// Four E4M3 codes (one dword) -> four fp16 values, exactly (scale 1): every
// E4M3 value (3 mantissa bits, magnitudes 2^-9 .. 448) is an fp16 normal.
__device__ inline f16x4 codes_to_f16(uint32_t w) {
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ inline f16x8 codes_to_f16x8(uint32_t w0, uint32_t w1) {
    const f16x4 a = codes_to_f16(w0), b = codes_to_f16(w1);
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Asynchronous fetch of one 128-key tile of codes into a staging buffer
// ([key][128] rows of 128 B, 16-byte chunks permuted within each row by the
// lane offsets): wave w fills the 1 KiB segments 2w and 2w + 1 (tile rows
// [16w, 16w + 16)); lane l of a segment writes LDS bytes [16l, 16l + 16),
// i.e. row l >> 3 of the segment, chunk l & 7.  Each
// segment's buffer descriptor starts at this head's slice of its first row
// and ends after the last row of the sequence: rows past it are out of
// range, which the hardware turns into zeros in LDS.
__device__ inline void issue_code_tile_load(const uint8_t* __restrict__ src, uint32_t row_stride, int h, int kt,
                                            int seq_hi, lds_u8* dst, int wave, uint32_t lane_off0,
                                            uint32_t lane_off1) {
    const int nrows = min(seq_hi - kt, kBN);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int seg = wave * 2 + r;
        const int rows_left = nrows - seg * 8;
        const int nrec = rows_left > 0 ? (rows_left - 1) * (int)row_stride + kD : 0;
        const size_t off = (size_t)(kt + seg * 8) * row_stride + (size_t)h * kD;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + off), 0, nrec, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + seg * 1024, 16, (int)(r == 0 ? lane_off0 : lane_off1), 0,
                                                 0, 0);
    }
}

// Staged K codes -> one fp16 K tile, by the 256 threads of one wave group.
// Each 16-lane group converts the rows 2m and 2m + 1 (m = (u >> 4) + 16r,
// r = 0..3): lanes 0..3 take 16-code chunks j = 0..3 of row 2m, lanes 4..7
// the same chunks of row 2m + 1, lanes 8..15 chunks 4..7 of both, and each
// chunk becomes logical fp16 chunks 2j and 2j + 1 of its row, stored at
// chunk ^ swz_k(row).  The K staging holds chunk q of row k at q ^ 4 (k & 1)
// (async-load lane offsets), so every 16-lane group reads 16 distinct
// 16-byte slots of the 256 bytes of rows 2m and 2m + 1 and stores to 16
// distinct chunks (the LDS bank layout is described at swz_vt).
__device__ __forceinline__ void convert_k_tile(const unsigned char* src, unsigned char* dst, uint32_t u) {
    const uint32_t q = u & 15, j = (q & 3) + 4 * (q >> 3);
    const uint32_t row0 = 2 * (u >> 4) + ((q >> 2) & 1);   // row of r = 0; r adds 32 rows
    const uint32_t rd = row0 * kD + 16 * (j ^ (4 * (row0 & 1)));
    const uint32_t swz = swz_k(row0);                       // the same for row0 + 32r
    unsigned char* d = dst + row0 * kRow;
    u32x4 w[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w[r] = *(const u32x4*)(src + rd + r * 32 * kD);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        *(f16x8*)(d + r * 32 * kRow + 16 * ((2 * j) ^ swz)) = codes_to_f16x8(w[r][0], w[r][1]);
        *(f16x8*)(d + r * 32 * kRow + 16 * ((2 * j + 1) ^ swz)) = codes_to_f16x8(w[r][2], w[r][3]);
    }
}

// ---- V^T tiles ----
// The converted V is stored transposed, as V^T [128 dims][128 keys] fp16 in
// 256-byte rows, so that P V reads its A operand with ds_read_b128 like
// Q K^T does (half the LDS instructions of transposed 8-byte reads).  Within
// each 32-key chunk j the keys are permuted into the order of the P^T
// operand: logical 16-byte chunk 4j + g of row d holds, at element 4hh + i,
// key 32j + 16hh + 4g + i of dim d.  Chunk c of row d sits at c ^ swz_vt(d).
//
// LDS banks, as the bank-conflict counter shows them for 16-byte accesses:
// 64 banks of 4 bytes (256 bytes), served 16 lanes at a time, so an access
// is conflict-free when 16 consecutive lanes touch distinct 16-byte slots
// modulo 256 bytes.  Rows are 256 bytes: swz_vt(d) = d & 15 (the K layout)
// gives the 16 rows of an operand read, and of a conversion store, 16
// distinct chunks.
__device__ inline uint32_t swz_vt(uint32_t d) { return d & 15; }

// V code staging is swizzled at 16-byte granularity: logical chunk q of tile
// row k sits at chunk q ^ swz_v8(k).  A transposed read takes one 16-byte
// column chunk of the 8 rows {32j + 16hh + 4g + i}; swz_v8 maps their bits
// 0, 1 and 4 to distinct chunks, and row bit 2 (g's low bit) flips chunk bit
// 0 so that neighbouring lane groups use the other chunks as well.
__device__ inline uint32_t swz_v8(uint32_t k) { return ((k & 3) | ((k >> 2) & 4)) ^ ((k >> 2) & 1); }

// Staged V codes -> one V^T tile, by the 256 threads of one wave group.
// ds_read_b64_tr_b8: in each 16-lane group, lane r receives byte e (e = 0..7)
// from the address of lane 2e + (r >> 3), at offset r & 7 (measured).  Read n
// (0..7) of 16-lane group G of wave gw converts dims 16n .. 16n + 15 of
// 32-key chunk j = gw for g = G: source lane s points at key row
// 32j + 16(s >> 3) + 4g + ((s >> 1) & 3), at the low (s even) or high (s odd)
// 8 bytes of the row's 16-byte chunk n, so that lane r receives, for dim
// 16n + r, keys 32j + 16hh + 4g + i at element 4hh + i: logical V^T chunk
// 4j + g of row 16n + r, stored with one ds_write_b128.
__device__ __forceinline__ void convert_vt(const unsigned char* src, unsigned char* dst, uint32_t u) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const uint32_t j = u >> 6, g = (u >> 4) & 3, r = u & 15;
    const uint32_t krow = 32 * j + 16 * (r >> 3) + 4 * g + ((r >> 1) & 3);
    const uint32_t src_off = krow * kD + 16 * swz_v8(krow) + 8 * (r & 1);
    const uint32_t dst_off = r * kRow + 16 * ((4 * j + g) ^ swz_vt(r));
    v2i x[8];
#pragma unroll
    for (int n = 0; n < 8; ++n)
        x[n] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(lds_u8*)(src + (src_off ^ (uint32_t)(n << 4))));
#pragma unroll
    for (int n = 0; n < 8; ++n)
        *(f16x8*)(dst + dst_off + n * 16 * kRow) = codes_to_f16x8((uint32_t)x[n][0], (uint32_t)x[n][1]);
}

// Half of the same conversion, by the 256 threads of one wave group: the
// 32-key chunks 2 half and 2 half + 1, each thread 4 of the 8 reads (dims
// 16n .. 16n + 15 for n in 4nh .. 4nh + 3); every 16-lane group keeps the
// lane pattern of convert_vt.
__device__ __forceinline__ void convert_vt_half(const unsigned char* src, unsigned char* dst, uint32_t u,
                                                uint32_t half) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const uint32_t j = 2 * half + (u >> 7), nh = (u >> 6) & 1, g = (u >> 4) & 3, r = u & 15;
    const uint32_t krow = 32 * j + 16 * (r >> 3) + 4 * g + ((r >> 1) & 3);
    const uint32_t src_off = krow * kD + 16 * swz_v8(krow) + 8 * (r & 1);
    const uint32_t dst_off = r * kRow + 16 * ((4 * j + g) ^ swz_vt(r));
    v2i x[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
        x[n] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(lds_u8*)(src + (src_off ^ (uint32_t)((4 * nh + n) << 4))));
#pragma unroll
    for (int n = 0; n < 4; ++n)
        *(f16x8*)(dst + dst_off + (4 * nh + n) * 16 * kRow) = codes_to_f16x8((uint32_t)x[n][0], (uint32_t)x[n][1]);
}

// O^T += V^T P^T for one key tile over the first kDB 16-dim blocks, V^T read
// from a converted V^T tile: the A operand of dim block db and key chunk j
// is row 16db + r16, logical chunk 4j + g, at vt_rd ^ (j << 6) (+ 16 rows per
// block).  Each operand is requested three steps before its MFMAs issue (the
// scheduling fence keeps it there), so LDS latency overlaps the matrix work.
template <int kDB>
__device__ __forceinline__ void pv_tile_t(const unsigned char* vtbase, uint32_t vt_rd, const f16x8 (&pop)[kQB][4],
                                          v4f (&o)[8][kQB]) {
    constexpr int kSteps = 4 * kDB;   // step n: dim block n >> 2, key chunk n & 3
    constexpr int kAhead = 3;
    auto operand = [&](int n) {
        return *(const f16x8*)(vtbase + (vt_rd ^ (uint32_t)((n & 3) << 6)) + (n >> 2) * 16 * kRow);
    };
    f16x8 vop[4];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) vop[n] = operand(n);
#pragma unroll
    for (int n = 0; n < kSteps; ++n) {
        if (n + kAhead < kSteps) vop[(n + kAhead) & 3] = operand(n + kAhead);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) o[n >> 2][qb] = mfma16(vop[n & 3], pop[qb][n & 3], o[n >> 2][qb]);
    }
}

// P^T operands from p, rounded to fp16 (nearest even, v_cvt_pk_f16_f32):
// pop[qb][j] holds p of keys 32j + 4g + i (elements 0..3) and
// 32j + 16 + 4g + i (elements 4..7) of query r16.  p <= 2^(8 + slack) fits
// fp16's range; 11 significant bits against bf16's 8.
__device__ __forceinline__ void pack_f16(const v4f (&p)[8][kQB], f16x8 (&pop)[kQB][4]) {
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v4f a = p[2 * j][qb], b = p[2 * j + 1][qb];
            pop[qb][j] = f16x8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
                               (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
        }
}

// l += the tile's row sums of the fp16 p: with every A entry 1, each output
// entry of a 16x16x32 product is the sum of its query's 32 p, already
// reduced over the lanes.
__device__ __forceinline__ void row_sums(const f16x8 (&pop)[kQB][4], v4f (&l)[kQB]) {
    const _Float16 one = (_Float16)1.0f;
    const f16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) l[qb] = mfma16(ones, pop[qb][j], l[qb]);
}

// S = K Q^T for one key tile on the fp8 MFMA (v_mfma_f32_16x16x128_f8f6f4,
// E4M3 x E4M3, float32 accumulation; each product in a group of 8 is
// truncated below the group's largest, see the header comment): one
// instruction per (16-key block, query block) covers all 128 dims.  The A
// operand is read straight from the double-buffered K code staging (rows of
// 128 bytes), whose logical 16-byte chunk c of key row k sits at chunk
// c ^ swz_k8(k): lane (r16, g) holds key 16kb + r16, dims 32g .. 32g + 31
// (chunks 2g and 2g + 1, at rd and rd ^ 16), and the Q operand holds the
// same dims of query r16, so each lane pairs like dims with like.  A 16-byte
// LDS read is served 16 lanes at a time from 64 banks of 4 bytes (256
// bytes), so it is conflict-free when 16 consecutive lanes touch distinct
// 16-byte slots modulo 256 bytes (the bank-conflict counter shows two-way
// conflicts, 4 cycles per read, with the swizzle k & 7 alone).  Lanes
// r16 = 0..15 read rows of both parities, i.e. both halves of a 256-byte
// window, and within each parity swz_k8 takes 8 distinct values.  Each
// operand is requested three key blocks before its MFMAs issue.
__device__ inline uint32_t swz_k8(uint32_t k) { return (k & 7) ^ ((k >> 3) & 1); }

__device__ __forceinline__ void qk_tile_f8(const unsigned char* kbase, uint32_t rd, const v8i (&q)[kQB],
                                           v4f (&s)[8][kQB]) {
    constexpr int kAhead = 3;
    auto operand = [&](int kb) {
        const u32x4 a = *(const u32x4*)(kbase + rd + kb * 16 * kD);
        const u32x4 b = *(const u32x4*)(kbase + (rd ^ 16u) + kb * 16 * kD);
        return v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    };
    v8i kop[4];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) kop[n] = operand(n);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        if (kb + kAhead < 8) kop[(kb + kAhead) & 3] = operand(kb + kAhead);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
            s[kb][qb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop[kb & 3], q[qb], v4f{0, 0, 0, 0}, 0, 0, 0,
                                                                          0, 0, 0);
    }
}

// Everything one wave carries through the key loop, in the 16x16 layout
// (every head dim).  Lane (r16, g) of a 16x16 accumulator holds rows
// 4g..4g+3 of column r16; every score and output block uses that layout
// (scores: rows = keys, columns = queries; output: rows = head dims,
// columns = queries).  kDC_: live 32-dim chunks of Q K^T; kDB_: live 16-dim
// output blocks (o[db] for db >= kDB_ is never touched).
template <int kDC_, int kDB_>
struct Wave {
    static constexpr int kDC = kDC_;
    static constexpr int kDB = kDB_;
    static constexpr bool kBlockRescale = true;   // rescale decisions per 16-query block
    static constexpr bool kConvertInTail = false;  // code conversions after P V (see key_loop)
    static constexpr bool kSplitV = false;          // V converted by one group (see key_loop)
    typedef v4f Scores[8][kQB];   // s[kb][qb]: keys 16kb + 4g + i of query r16
    typedef f16x8 POps[kQB][4];   // P^T operands of one key tile (pack_f16)
    const uint8_t* k8;
    const uint8_t* v8;
    uint32_t row_stride;   // bytes between tokens of one head (uniform)
    int h, seq_hi, k0, nt, nk_last, wave;   // keys [k0, k0 + 128 nt) of the sequence ending at seq_hi
    float cexp;            // s_q s_k log2(e) / sqrt(D)
    uint32_t k_rd, vt_rd;  // operand offsets inside an fp16 K / V^T tile
    uint32_t g_ld, g_ldv;  // async loads of K / V codes: row-in-segment * stride + 16-byte chunk
    uint32_t cv;           // conversion: thread index inside its group
    int g4;                // 4 g: first key row of this lane inside a 16-key block
    f16x8 q[kQB][4];       // Q operand (B of S = K Q^T)
    float mc[kQB];         // running row max in log2 units (S c), within the rescale slack of the true max
    v4f o[8][kQB];         // O^T blocks [d block][query block]
    v4f l[kQB];            // running row sums of the fp16 p per query (the 4 entries are equal)

    // Lane offsets (after wave and row_stride are set).  Async loads: lane
    // covers row lane >> 3 of each 8-row segment, LDS chunk lane & 7, and
    // fetches the logical chunk that the staging swizzle puts there:
    // (lane & 7) ^ 4 (row & 1) for K; (lane & 7) ^ swz_v8(row) for V, where
    // the tile row 16 wave + 8r + (lane >> 3) has bit 4 = wave & 1 for both of
    // the wave's segments.
    __device__ __forceinline__ void setup(int tid) {
        const uint32_t lane = (uint32_t)tid & 63, r16 = lane & 15, g = lane >> 4;
        k_rd = k_operand_offset((int)r16, (int)g);
        vt_rd = r16 * kRow + 16 * (g ^ swz_vt(r16));
        g_ld = (lane >> 3) * row_stride + 16 * ((lane & 7) ^ (4 * ((lane >> 3) & 1)));
        g_ldv = (lane >> 3) * row_stride + 16 * ((lane & 7) ^ swz_v8((lane >> 3) + 16 * ((uint32_t)wave & 1)));
        cv = (uint32_t)tid & (kGroupThreads - 1);
        g4 = 4 * (int)g;
    }
    // Q operand (B of S = K Q^T, fp16 16x16x32): for the c-th MFMA, lane
    // holds query r16 of the block and head dims 32c + 8g .. + 7, the
    // mapping the K operand uses.
    __device__ __forceinline__ void load_q(const uint8_t* __restrict__ q8, int q0, int lane) {
        const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int qi = q0 + wave * (16 * kQB) + qb * 16 + r16;
#pragma unroll
            for (int c = 0; c < kDC; ++c) {
                u32x2 a = {0, 0};
                if (qi < seq_hi) a = *(const u32x2*)(q8 + (size_t)qi * row_stride + (size_t)h * kD + 32 * c + 8 * g);
                q[qb][c] = codes_to_f16x8(a[0], a[1]);
            }
        }
    }
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
            for (int db = 0; db < kDB; ++db) o[db][qb] = v4f{0, 0, 0, 0};
            l[qb] = v4f{0, 0, 0, 0};
            mc[qb] = kMInit;
        }
    }

    __device__ __forceinline__ void load_k8(lds_u8* lds, int t) const {
        issue_code_tile_load(k8, row_stride, h, k0 + t * kBN, seq_hi, lds + kLdsK8, wave, g_ld, g_ld);
    }
    __device__ __forceinline__ void load_v8(lds_u8* lds, int t) const {
        issue_code_tile_load(v8, row_stride, h, k0 + t * kBN, seq_hi, lds + kLdsV8, wave, g_ldv, g_ldv);
    }
    __device__ __forceinline__ void convert_k(unsigned char* smem, int buf) const {
        convert_k_tile(smem + kLdsK8, smem + kLdsK + buf * kTileBytes, cv);
    }
    __device__ __forceinline__ void convert_v(unsigned char* smem, int buf) const {
        convert_vt(smem + kLdsV8, smem + kLdsV + buf * kTileBytes, cv);
    }

    // The four phases of a key tile (see key_loop).
    __device__ __forceinline__ void qk(const unsigned char* ktile, Scores& s) const { qk_tile<kDC>(ktile, k_rd, q, s); }
    __device__ __forceinline__ void head(Scores& s, int nk) { softmax_head<kSplit>(*this, s, nk); }
    __device__ __forceinline__ void tail(Scores& s, int nk, POps& pop) const {
        exp_blocks<kSplit, 8>(*this, s, nk);
        pack_f16(s, pop);
    }
    __device__ __forceinline__ void pv(const unsigned char* vttile, const POps& pop) {
        pv_tile_t<kDB>(vttile, vt_rd, pop, o);
        row_sums(pop, l);
    }

    // Epilogue: lane holds O^T[d = 16db + 4g + i][query r16]; the output rows
    // hold head_dim dims (a multiple of 8, so a lane's 4 dims are all inside
    // or all past it).  out = bf16(O * s_v / l).
    __device__ __forceinline__ void store(__bf16* __restrict__ out, int q0, int num_heads, int head_dim, float s_v,
                                          int lane) const {
        const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int qi = q0 + wave * (16 * kQB) + qb * 16 + r16;
            if (qi < seq_hi) {
                const float f = s_v / l[qb][0];
                __bf16* dst = out + ((size_t)qi * num_heads + h) * head_dim + 4 * g;
#pragma unroll
                for (int db = 0; db < kDB; ++db) {
                    if (16 * db + 4 * g < head_dim) {
                        bf16x4 r;
                        r[0] = (__bf16)(o[db][qb][0] * f);
                        r[1] = (__bf16)(o[db][qb][1] * f);
                        r[2] = (__bf16)(o[db][qb][2] * f);
                        r[3] = (__bf16)(o[db][qb][3] * f);
                        *(bf16x4*)(dst + 16 * db) = r;
                    }
                }
            }
        }
    }
    // Split-key partial: O / l in code units as fp16, and (mc, l).
    __device__ __forceinline__ void store_partial(_Float16* __restrict__ part_o, v2f* __restrict__ part_ml,
                                                  size_t prow0, int q0, int lane) const {
        const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int qt = wave * (16 * kQB) + qb * 16 + r16;   // query in tile
            if (q0 + qt < seq_hi) {
                const float il = 1.0f / l[qb][0];
                _Float16* dst = part_o + (prow0 + qt) * kD + 4 * g;
#pragma unroll
                for (int db = 0; db < kDB; ++db) {
                    f16x4 r;
                    r[0] = (_Float16)(o[db][qb][0] * il);
                    r[1] = (_Float16)(o[db][qb][1] * il);
                    r[2] = (_Float16)(o[db][qb][2] * il);
                    r[3] = (_Float16)(o[db][qb][3] * il);
                    *(f16x4*)(dst + 16 * db) = r;
                }
                if (g == 0) part_ml[prow0 + qt] = v2f{mc[qb], l[qb][0]};
            }
        }
    }
};

// The 16x16 layout with S on the fp8 MFMA (qk_tile_f8): the Q operand holds
// the codes of all 128 dims, K tile t's codes are staged into buffer t & 1
// (the key loop's K tile t & 1) and read as they are, and there is no K
// conversion.  Everything else is Wave's (its fp16 Q operand is never
// loaded or read, so it takes no registers).  The staging swizzle puts
// logical chunk c of tile row k at chunk c ^ swz_k8(k): an async-load lane
// covers row (lane >> 3) of an 8-row segment, LDS chunk lane & 7, and a
// wave's two segments are tile rows 16 wave + (lane >> 3) and that + 8
// (bit 3 of the row 0 and 1), so it fetches logical chunk
// (lane & 7) ^ (lane >> 3) in the first and (lane & 7) ^ (lane >> 3) ^ 1 in
// the second.
template <int kDC_, int kDB_>
struct WaveF8 : Wave<kDC_, kDB_> {
    v8i qc[kQB];     // Q operand (B of S = K Q^T): codes of dims 32g .. 32g + 31 of query r16
    uint32_t g_ld1;  // async K load of the wave's second segment (the first is g_ld)

    __device__ __forceinline__ void setup(int tid) {
        Wave<kDC_, kDB_>::setup(tid);
        const uint32_t lane = (uint32_t)tid & 63, r16 = lane & 15, g = lane >> 4;
        this->k_rd = r16 * kD + 16 * ((2 * g) ^ swz_k8(r16));
        this->g_ld = (lane >> 3) * this->row_stride + 16 * ((lane & 7) ^ swz_k8(lane >> 3));
        g_ld1 = (lane >> 3) * this->row_stride + 16 * ((lane & 7) ^ swz_k8((lane >> 3) + 8));
    }
    __device__ __forceinline__ void load_q(const uint8_t* __restrict__ q8, int q0, int lane) {
        const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const int qi = q0 + this->wave * (16 * kQB) + qb * 16 + r16;
            u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
            if (qi < this->seq_hi) {
                const uint8_t* src = q8 + (size_t)qi * this->row_stride + (size_t)this->h * kD + 32 * g;
                a = *(const u32x4*)src;
                b = *(const u32x4*)(src + 16);
            }
            qc[qb] = v8i{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        }
    }
    __device__ __forceinline__ void load_k8(lds_u8* lds, int t) const {
        issue_code_tile_load(this->k8, this->row_stride, this->h, this->k0 + t * kBN, this->seq_hi,
                             lds + kLdsK + (t & 1) * kTileBytes, this->wave, this->g_ld, g_ld1);
    }
    __device__ __forceinline__ void convert_k(unsigned char*, int) const {}
    // V^T: key chunks 0-1 by group A (convert_v_first), 2-3 by group B (convert_v); see key_loop
    static constexpr bool kSplitV = true;
    __device__ __forceinline__ void convert_v_first(unsigned char* smem, int buf) const {
        convert_vt_half(smem + kLdsV8, smem + kLdsV + buf * kTileBytes, this->cv, 0);
    }
    __device__ __forceinline__ void convert_v(unsigned char* smem, int buf) const {
        convert_vt_half(smem + kLdsV8, smem + kLdsV + buf * kTileBytes, this->cv, 1);
    }
    __device__ __forceinline__ void qk(const unsigned char* ktile, typename Wave<kDC_, kDB_>::Scores& s) const {
        qk_tile_f8(ktile, this->k_rd, qc, s);
    }
};

// ---- The 32x32 layout (head dims above 96) ----
//
// Both products run on v_mfma_f32_32x32x16_f16.  An operand read (1 KiB
// per wave) then feeds one 32x32x16 product instead of two 16x16x32 ones:
// the same LDS bytes per multiply-add, half the MFMA instructions and the
// waits that go with them, which leaves more issue cycles to the wave that
// runs the softmax on the same SIMD.  Lane l = (c32, hh), c32 = l & 31,
// hh = l >> 5.
//   Operands (A of both products, 16 B per lane): row c32 of a 32-row block,
//     logical 16-byte chunk 2c + hh of the 16-element k-step c.  K and V^T
//     tiles both place logical chunk j of row r at j ^ (r & 15), so one lane
//     offset rd = c32 * kRow + 16 (hh ^ (c32 & 15)) serves both, at rd ^ 32c
//     (+ 32 rows per block).
//   Q (B of S = K Q^T): query c32 of the wave's 32, head dims 16c + 8hh + e.
//   Accumulators: register r of 32x32 block b holds row
//     32b + 8(r >> 2) + 4hh + (r & 3) of column c32.  In S the rows are
//     keys, in O^T head dims, and the column is the lane's query: a lane
//     holds 64 of its query's 128 scores of a tile, the lane l ^ 32 the
//     rest.
//   P^T (B of O^T += V^T P^T) for the 16-key step m: registers
//     8(m & 1) .. 8(m & 1) + 7 of S block m >> 1, whose element e is key
//     16m + 8(e >> 2) + 4hh + (e & 3).  The V^T tile holds the same keys in
//     the same order in logical chunk 2m + hh of each row (convert_vt32).
typedef float v16f __attribute__((ext_vector_type(16)));
__device__ inline v16f mfma32(f16x8 a, f16x8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// V code staging of the 32x32 layout, swizzled at 16-byte granularity like
// swz_v8: a transposed read takes one 16-byte column chunk of the 8 rows
// {16m + 4hh + 8a + i : a < 2, i < 4}, which differ in row bits 0, 1 and 3;
// swz_v8w maps those to distinct chunks, and row bit 2 flips chunk bit 0.
__device__ inline uint32_t swz_v8w(uint32_t k) { return ((k & 3) | ((k >> 1) & 4)) ^ ((k >> 2) & 1); }

// Staged V codes -> one V^T tile of the 32x32 layout, by the 256 threads of
// one wave group.  With the lane mapping of ds_read_b64_tr_b8 (convert_vt),
// 16-lane group G of wave gw takes the 16-key step m = 2gw + (G >> 1) and
// half hh = G & 1: source lane s points at key row
// 16m + 4hh + 8(s >> 3) + ((s >> 1) & 3), low (s even) or high (s odd) 8
// bytes of its 16-byte chunk n, so that lane r receives, for dim 16n + r,
// key 16m + 8(e >> 2) + 4hh + (e & 3) at element e: logical chunk 2m + hh
// of V^T row 16n + r, stored with one ds_write_b128.
__device__ __forceinline__ void convert_vt32(const unsigned char* src, unsigned char* dst, uint32_t u) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const uint32_t grp = (u >> 4) & 3, r = u & 15;
    const uint32_t m = 2 * (u >> 6) + (grp >> 1), hh = grp & 1;
    const uint32_t krow = 16 * m + 4 * hh + 8 * (r >> 3) + ((r >> 1) & 3);
    const uint32_t src_off = krow * kD + 16 * swz_v8w(krow) + 8 * (r & 1);
    const uint32_t dst_off = r * kRow + 16 * ((2 * m + hh) ^ swz_vt(r));
    v2i x[8];
#pragma unroll
    for (int n = 0; n < 8; ++n)
        x[n] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(lds_u8*)(src + (src_off ^ (uint32_t)(n << 4))));
#pragma unroll
    for (int n = 0; n < 8; ++n)
        *(f16x8*)(dst + dst_off + n * 16 * kRow) = codes_to_f16x8((uint32_t)x[n][0], (uint32_t)x[n][1]);
}

// S = K Q^T for one key tile: step n multiplies K operand (32-key block
// n & 3, 16-dim step n >> 2) into S block n & 3, so products into one
// accumulator are four steps apart.  Operands are requested kAhead steps
// before their product issues.
__device__ __forceinline__ void qk_tile32(const unsigned char* kbase, uint32_t rd, const f16x8 (&q)[8],
                                          v16f (&s)[4]) {
    constexpr int kSteps = 32;
    constexpr int kAhead = 4;
    auto operand = [&](int n) {
        return *(const f16x8*)(kbase + (rd ^ (uint32_t)((n >> 2) << 5)) + (n & 3) * 32 * kRow);
    };
    f16x8 kop[8];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) kop[n] = operand(n);
#pragma unroll
    for (int n = 0; n < kSteps; ++n) {
        if (n + kAhead < kSteps) kop[(n + kAhead) & 7] = operand(n + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = n & 3, c = n >> 2;
        s[kb] = mfma32(kop[n & 7], q[c], c == 0 ? v16f{} : s[kb]);
    }
}

// l += the row sums of the fp16 p, on the 16x16x32 MFMA.  Fed as its B
// operand, pop[m] of lane l = c + 16g (c < 16) lands in column c, k-group g;
// lanes c and c + 32 (g = 0, 2) hold the 16 keys of query c, lanes c + 16 and
// c + 48 (g = 1, 3) those of query c + 16.  The selector A (WaveWide::sel)
// has ones in row 4g' (g' < 4) over the k-groups of parity g' & 1, so output
// row 4g' of column c, which lane c + 16g' holds in entry 0, is the row sum
// of that lane's own query; the other rows are zero.
//
// O^T += V^T P^T for one key tile: step n multiplies the V^T operand (32-dim
// block n & 3, 16-key step n >> 2) with P^T of that key step.  The row sums
// of each key step (above) are interleaved after its last product, so
// that consecutive row-sum products, which share one accumulator, issue
// five products apart.
__device__ __forceinline__ void pv_tile32(const unsigned char* vtbase, uint32_t rd, const f16x8 (&pop)[8],
                                          f16x8 sel, v16f (&o)[4], v4f& l) {
    constexpr int kSteps = 32;
    constexpr int kAhead = 3;
    auto operand = [&](int n) {
        return *(const f16x8*)(vtbase + (rd ^ (uint32_t)((n >> 2) << 5)) + (n & 3) * 32 * kRow);
    };
    f16x8 vop[4];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) vop[n] = operand(n);
#pragma unroll
    for (int n = 0; n < kSteps; ++n) {
        if (n + kAhead < kSteps) vop[(n + kAhead) & 3] = operand(n + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        o[n & 3] = mfma32(vop[n & 3], pop[n >> 2], o[n & 3]);
        if ((n & 3) == 3) l = mfma16(sel, pop[n >> 2], l);
    }
}

// P^T operands from p, rounded to fp16 (nearest even): pop[m] = registers
// 8(m & 1) .. + 7 of S block m >> 1.
__device__ __forceinline__ void pack_f16_32(const v16f (&p)[4], f16x8 (&pop)[8]) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const v16f& a = p[m >> 1];
        const int r = 8 * (m & 1);
        pop[m] = f16x8{(_Float16)a[r], (_Float16)a[r + 1], (_Float16)a[r + 2], (_Float16)a[r + 3],
                       (_Float16)a[r + 4], (_Float16)a[r + 5], (_Float16)a[r + 6], (_Float16)a[r + 7]};
    }
}

struct WaveWide {
    static constexpr int kDB = 4;   // 32-dim output blocks
    static constexpr bool kConvertInTail = true;   // code conversions after the softmax tails (see key_loop)
    static constexpr bool kSplitV = false;         // V converted by one group (see key_loop)
    typedef v16f Scores[4];         // s[kb]: 32-key block kb (layout above)
    typedef f16x8 POps[8];          // P^T operands of the tile's 8 16-key steps
    const uint8_t* k8;
    const uint8_t* v8;
    uint32_t row_stride;
    int h, seq_hi, k0, nt, nk_last, wave;
    float cexp;
    uint32_t rd;                     // operand offset inside an fp16 K or V^T tile
    uint32_t g_ld, g_ldv0, g_ldv1;   // async loads: K segments; V segments 0 and 1
    uint32_t cv;
    int hh4;                         // 4 hh: first key row of this lane inside an 8-key group
    f16x8 sel;                       // A operand of the row-sum products (pv_tile32)
    f16x8 q[8];                      // Q operand, one per 16-dim step
    float mc;                        // running row max of the lane's query (log2 units)
    v16f o[4];                       // O^T blocks of the lane's query
    v4f l;                           // entry 0: row sum of the lane's query

    // Lane offsets (after wave and row_stride are set).  Async V loads: the
    // tile row 16 wave + 8r + (lane >> 3) of segment r has swz_v8w of its
    // low four bits, 8r + (lane >> 3), so the two segments differ.
    __device__ __forceinline__ void setup(int tid) {
        const uint32_t lane = (uint32_t)tid & 63, c32 = lane & 31, hh = lane >> 5;
        const uint32_t r16 = lane & 15, g = lane >> 4;
        rd = c32 * kRow + 16 * (hh ^ (c32 & 15));
        g_ld = (lane >> 3) * row_stride + 16 * ((lane & 7) ^ (4 * ((lane >> 3) & 1)));
        g_ldv0 = (lane >> 3) * row_stride + 16 * ((lane & 7) ^ swz_v8w(lane >> 3));
        g_ldv1 = (lane >> 3) * row_stride + 16 * ((lane & 7) ^ swz_v8w(8 + (lane >> 3)));
        cv = (uint32_t)tid & (kGroupThreads - 1);
        hh4 = 4 * (int)hh;
        const _Float16 one = (_Float16)(((r16 & 3) == 0 && (g & 1) == ((r16 >> 2) & 1)) ? 1.0f : 0.0f);
        sel = f16x8{one, one, one, one, one, one, one, one};
    }
    __device__ __forceinline__ void load_q(const uint8_t* __restrict__ q8, int q0, int lane) {
        const int c32 = lane & 31, hh = lane >> 5;
        const int qi = q0 + wave * 32 + c32;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            u32x2 a = {0, 0};
            if (qi < seq_hi) a = *(const u32x2*)(q8 + (size_t)qi * row_stride + (size_t)h * kD + 16 * c + 8 * hh);
            q[c] = codes_to_f16x8(a[0], a[1]);
        }
    }
    __device__ __forceinline__ void reset() {
#pragma unroll
        for (int db = 0; db < kDB; ++db) o[db] = v16f{};
        l = v4f{0, 0, 0, 0};
        mc = kMInit;
    }

    __device__ __forceinline__ void load_k8(lds_u8* lds, int t) const {
        issue_code_tile_load(k8, row_stride, h, k0 + t * kBN, seq_hi, lds + kLdsK8, wave, g_ld, g_ld);
    }
    __device__ __forceinline__ void load_v8(lds_u8* lds, int t) const {
        issue_code_tile_load(v8, row_stride, h, k0 + t * kBN, seq_hi, lds + kLdsV8, wave, g_ldv0, g_ldv1);
    }
    __device__ __forceinline__ void convert_k(unsigned char* smem, int buf) const {
        convert_k_tile(smem + kLdsK8, smem + kLdsK + buf * kTileBytes, cv);
    }
    __device__ __forceinline__ void convert_v(unsigned char* smem, int buf) const {
        convert_vt32(smem + kLdsV8, smem + kLdsV + buf * kTileBytes, cv);
    }

    // Keys past nk (the last tile) get `dead`: -inf before the max, 0 after
    // the exponentials (also where c = 0 made -inf * c a NaN).
    template <int kLo, int kHi>
    __device__ __forceinline__ void mask(Scores& s, int nk, float dead) const {
#pragma unroll
        for (int kb = kLo; kb < kHi; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = hh4 >= nk - (32 * kb + 8 * (r >> 2) + (r & 3)) ? dead : s[kb][r];
    }
    template <int kLo, int kHi>
    __device__ __forceinline__ void exponentials(Scores& s, int nk) const {
        const float bias = 8.0f - mc;
#pragma unroll
        for (int kb = kLo; kb < kHi; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], cexp, bias));
        if (nk < kBN) mask<kLo, kHi>(s, nk, 0.0f);
    }

    // The four phases of a key tile (see key_loop).  head: mask, the query's
    // tile max tm (its 64 scores here, then the other half-wave's), and when
    // tm outgrew mc by more than the slack for any query of the wave, mc
    // moves to max(mc, tm + headroom) and O and l are rescaled; then p of S
    // blocks 0 and 1.  tail: p of blocks 2 and 3, and the P^T operands.
    __device__ __forceinline__ void qk(const unsigned char* ktile, Scores& s) const { qk_tile32(ktile, rd, q, s); }
    __device__ __forceinline__ void head(Scores& s, int nk) {
        if (nk < kBN) mask<0, 4>(s, nk, -INFINITY);
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        const v2i a = __builtin_amdgcn_permlane32_swap(__float_as_int(mx), __float_as_int(mx), false, false);
        const float tm = fmaxf(__int_as_float(a[0]), __int_as_float(a[1])) * cexp;
        if (__any(tm - mc > kRescaleSlack)) {
            const float mnew = fmaxf(mc, tm + kRescaleHeadroom);
            const float alpha = __builtin_amdgcn_exp2f(mc - mnew);
            mc = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < kDB; ++db) o[db] *= alpha;
        }
        exponentials<0, 2>(s, nk);
    }
    __device__ __forceinline__ void tail(Scores& s, int nk, POps& pop) const {
        exponentials<2, 4>(s, nk);
        pack_f16_32(s, pop);
    }
    __device__ __forceinline__ void pv(const unsigned char* vttile, const POps& pop) {
        pv_tile32(vttile, rd, pop, sel, o, l);
    }

    // Epilogue: register 4j + i of block db holds dim 32db + 8j + 4hh + i of
    // the lane's query.
    __device__ __forceinline__ void store(__bf16* __restrict__ out, int q0, int num_heads, int head_dim, float s_v,
                                          int lane) const {
        const int c32 = lane & 31, hh = lane >> 5;
        const int qi = q0 + wave * 32 + c32;
        if (qi >= seq_hi) return;
        const float f = s_v / l[0];
        __bf16* dst = out + ((size_t)qi * num_heads + h) * head_dim + 4 * hh;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (32 * db + 8 * j + 4 * hh < head_dim) {
                    bf16x4 r;
#pragma unroll
                    for (int i = 0; i < 4; ++i) r[i] = (__bf16)(o[db][4 * j + i] * f);
                    *(bf16x4*)(dst + 32 * db + 8 * j) = r;
                }
            }
    }
    __device__ __forceinline__ void store_partial(_Float16* __restrict__ part_o, v2f* __restrict__ part_ml,
                                                  size_t prow0, int q0, int lane) const {
        const int c32 = lane & 31, hh = lane >> 5;
        const int qt = wave * 32 + c32;   // query in tile
        if (q0 + qt >= seq_hi) return;
        const float il = 1.0f / l[0];
        _Float16* dst = part_o + (prow0 + qt) * kD + 4 * hh;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                f16x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = (_Float16)(o[db][4 * j + i] * il);
                *(f16x4*)(dst + 32 * db + 8 * j) = r;
            }
        if (hh == 0) part_ml[prow0 + qt] = v2f{mc, l[0]};
    }
};

// The key loop of one wave group.  Period t (t = 0..nt) has four slots
// separated by workgroup barriers (see the table at the top).  Loads: codes
// of K_{t+1} into the K staging buffer at slot 1 (landing by the end of
// slot 2), codes of V_{t+1} into the V staging buffer at slot 3 (landing by
// the end of slot 4).  W is the wave's layout (Wave or WaveWide), which
// supplies the phases and says where the code conversions go:
//   after P V (W::kConvertInTail false): K_{t+1} by A at slot 4 of period t,
//     V_{t+1} by B at slot 2 of period t+1, in the slot of the other group's
//     softmax head;
//   after the softmax tails (true): K_{t+1} by A at slot 3 of period t,
//     V_{t+1} by B at slot 1 of period t+1, next to the other group's Q K^T.
// With S on the fp8 MFMA (WaveF8) K is not converted (its codes are read as
// staged, double-buffered: K_{t+1} lands in the buffer that held K_{t-1},
// last read at slot 3 of period t-1) and V_t is converted in two halves
// (W::kSplitV): by A at slot 1 of period t, after its Q K^T, which is half
// as long as on the fp16 MFMA, and by B at slot 2 of period t, after its
// P V.
// Either way: fp16 K_t is read in slots 1 (A) and 3 (B) of period t and
// rewritten with K_{t+2} in period t+1; fp16 V^T_t is written in slot 1 or 2
// of period t, read in slot 4 of period t (A) and slot 2 of period t+1 (B),
// and rewritten with V^T_{t+2} in period t+2 (the other buffer holds
// V^T_{t+1}); each staging buffer is converted before the next load into it
// is issued.
template <bool kB, class W>
__device__ __forceinline__ void key_loop(W& w, unsigned char* smem) {
    lds_u8* const lds = (lds_u8*)smem;
    const int nt = w.nt;
    typename W::Scores s;
    typename W::POps pop;
    for (int t = 0; t <= nt; ++t) {
        const int cur = t & 1, prev = cur ^ 1;
        const int nk_t = (t + 1 < nt) ? kBN : w.nk_last;   // valid keys of tile t (t < nt)
        const int nk_p = (t < nt) ? kBN : w.nk_last;       // valid keys of tile t - 1 (t >= 1)
        // slot 1
        if (t + 1 < nt) w.load_k8(lds, t + 1);
        if constexpr (!kB) {
            if (t < nt) {
                mfma_phase_begin();
                w.qk(smem + kLdsK + cur * kTileBytes, s);
                if constexpr (W::kSplitV) {
                    if (t >= 1) w.convert_v_first(smem, cur);
                }
                mfma_phase_end();
            }
        } else {
            if (t >= 1) w.tail(s, nk_p, pop);
            if constexpr (W::kConvertInTail) {
                if (t >= 1 && t < nt) w.convert_v(smem, cur);
            }
        }
        __syncthreads();
        // slot 2
        if constexpr (!kB) {
            if (t < nt) w.head(s, nk_t);
        } else {
            if (t >= 1) {
                mfma_phase_begin();
                w.pv(smem + kLdsV + prev * kTileBytes, pop);
            }
            if constexpr (!W::kConvertInTail) {
                if (t >= 1 && t < nt) w.convert_v(smem, cur);
            }
            mfma_phase_end();
        }
        wait_async_loads();
        __syncthreads();
        // slot 3
        if (t + 1 < nt) w.load_v8(lds, t + 1);
        if constexpr (!kB) {
            if (t < nt) w.tail(s, nk_t, pop);
            if constexpr (W::kConvertInTail) {
                if (t + 1 < nt) w.convert_k(smem, prev);
            }
        } else {
            if (t < nt) {
                mfma_phase_begin();
                w.qk(smem + kLdsK + cur * kTileBytes, s);
                mfma_phase_end();
            }
        }
        __syncthreads();
        // slot 4
        if constexpr (!kB) {
            if (t < nt) {
                mfma_phase_begin();
                w.pv(smem + kLdsV + cur * kTileBytes, pop);
            }
            if constexpr (!W::kConvertInTail) {
                if (t + 1 < nt) w.convert_k(smem, prev);
            }
            mfma_phase_end();
        } else {
            if (t < nt) w.head(s, nk_t);
        }
        wait_async_loads();
        __syncthreads();
    }
}

// kPartial: the keys of each sequence are split into num_splits ranges of
// whole key tiles, one workgroup per (head, query tile, range); instead of the
// output, a workgroup writes for each of its queries the partial result over
// its range, normalised by its own row sum and kept in code units (a convex
// combination of V codes, so |value| <= 448 fits fp16), and (mc, l): its
// running max in log2 units and its row sum.  attn_combine_kernel merges the
// ranges.  Partial rows are indexed [split][head][virtual tile][query in
// tile] and hold 128 fp16 dims (those past the live blocks unwritten).
template <class W, bool kPartial>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8,
    const float* __restrict__ scales, const int32_t* __restrict__ cu, int num_seqs, int num_heads,
    int tiles_per_head, int num_splits, int head_dim, float log2e_rsqrt_d, __bf16* __restrict__ out,
    _Float16* __restrict__ part_o, v2f* __restrict__ part_ml) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
    lds_u8* const lds = (lds_u8*)smem;

    const int tid = threadIdx.x, lane = tid & 63;

    // logical id = (head, key range, virtual query tile): consecutive ids
    // share one head's K/V range and land on one XCD
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int per_head = tiles_per_head * num_splits;
    const int h = logical / per_head;
    const int rem = logical - h * per_head;
    const int split = rem / tiles_per_head;
    const int vt = rem - split * tiles_per_head;
    const int b = find_sequence(cu, num_seqs, vt);
    const int seq_lo = cu[b], seq_hi = cu[b + 1];
    const int q0 = seq_lo + (vt - (seq_lo / kBM + b)) * kBM;
    if (q0 >= seq_hi) return;  // spare tile (uniform over the workgroup)

    // key tiles [t0, t0 + nt) of the sequence's nt_seq
    const int nt_seq = (seq_hi - seq_lo + kBN - 1) / kBN;
    const int per = (nt_seq + num_splits - 1) / num_splits;
    const int t0 = min(nt_seq, split * per);
    const int nt = min(nt_seq, t0 + per) - t0;
    const size_t prow0 = ((size_t)(split * num_heads + h) * tiles_per_head + vt) * kBM;
    if constexpr (kPartial) {
        if (nt == 0) {   // a range past the sequence's last key tile: an empty partial (l = 0)
            if (tid < kBM && q0 + tid < seq_hi) part_ml[prow0 + tid] = v2f{kMInit, 0.0f};
            return;
        }
    }

    W w;
    w.k8 = k8;
    w.v8 = v8;
    w.row_stride = (uint32_t)num_heads * kD;
    w.h = h;
    w.seq_hi = seq_hi;
    w.k0 = seq_lo + t0 * kBN;
    w.nt = nt;
    w.nk_last = min(kBN, seq_hi - (w.k0 + (nt - 1) * kBN));
    w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const bool group_b = w.wave >= kWaves / 2;          // wave-uniform
    w.setup(tid);

    // ---- prologue: codes of K_0 and V_0 in flight; Q operand; K_0 and V_0
    // converted (A: K, B: V; with S on the fp8 MFMA only V, all of it by B) ----
    w.load_k8(lds, 0);
    w.load_v8(lds, 0);
    w.load_q(q8, q0, lane);
    const float s_q = scales[0], s_k = scales[1], s_v = scales[2];
    w.cexp = s_q * s_k * log2e_rsqrt_d;
    w.reset();

    wait_async_loads();
    __syncthreads();
    if (group_b) {
        w.convert_v(smem, 0);
        if constexpr (W::kSplitV) w.convert_v_first(smem, 0);
    } else {
        w.convert_k(smem, 0);
    }
    __syncthreads();

    // ---- key loop: group A runs tile t in period t, group B runs its slots
    // 1-2 on tile t-1 and 3-4 on tile t.  Each group has its own copy of the
    // loop, so its registers are allocated for its own live ranges; both
    // copies execute the same sequence of barriers.
    if (group_b)
        key_loop<true>(w, smem);
    else
        key_loop<false>(w, smem);

    if constexpr (kPartial)
        w.store_partial(part_o, part_ml, prow0, q0, lane);
    else
        w.store(out, q0, num_heads, head_dim, s_v, lane);
}

// Merge the key ranges of attn_fwd_kernel<.., true>.  Workgroup = 16
// queries of one (head, virtual query tile), 16 threads per query, thread c
// covering dims 8c .. 8c + 7, so a wave reads and writes whole rows.  With M
// the largest range max and w_s = 2^(mc_s - M) l_s, out = bf16(s_v *
// sum_s w_s O_s / sum_s w_s): the softmax normalisation over the whole
// sequence.  Empty ranges (l = 0) are skipped, so their unwritten rows are
// never read.
constexpr int kCombineQueries = 16;   // queries per combine workgroup
__global__ __launch_bounds__(256) void attn_combine_kernel(const _Float16* __restrict__ part_o,
                                                           const v2f* __restrict__ part_ml,
                                                           const float* __restrict__ scales,
                                                           const int32_t* __restrict__ cu, int num_seqs,
                                                           int num_heads, int tiles_per_head, int num_splits,
                                                           int head_dim, __bf16* __restrict__ out) {
    constexpr int kGroups = kBM / kCombineQueries;   // workgroups per query tile
    const int tile = blockIdx.x / kGroups;
    const int h = tile / tiles_per_head;
    const int vt = tile - h * tiles_per_head;
    const int b = find_sequence(cu, num_seqs, vt);
    const int seq_lo = cu[b], seq_hi = cu[b + 1];
    const int q0 = seq_lo + (vt - (seq_lo / kBM + b)) * kBM;
    const int qt = (blockIdx.x - tile * kGroups) * kCombineQueries + (int)(threadIdx.x >> 4);   // query in tile
    const int c = threadIdx.x & 15;                                                             // 8-dim chunk
    if (q0 + qt >= seq_hi || 8 * c >= head_dim) return;
    const size_t split_rows = (size_t)num_heads * tiles_per_head * kBM;
    const size_t row0 = ((size_t)h * tiles_per_head + vt) * kBM + qt;
    // loops over kMaxSplits are unrolled, so the weights stay in registers
    v2f ml[kMaxSplits];
    float mmax = kMInit;
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
        ml[sp] = sp < num_splits ? part_ml[row0 + sp * split_rows] : v2f{kMInit, 0.0f};
        if (ml[sp][1] > 0.0f) mmax = fmaxf(mmax, ml[sp][0]);
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplits; ++sp) {
        if (!(ml[sp][1] > 0.0f)) continue;
        const float wt = __builtin_amdgcn_exp2f(ml[sp][0] - mmax) * ml[sp][1];
        wsum += wt;
        const f16x8 x = *(const f16x8*)(part_o + (row0 + sp * split_rows) * kD + 8 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wt * (float)x[i];
    }
    const float f = scales[2] / wsum;
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)(acc[i] * f);
    *(bf16x8*)(out + ((size_t)(q0 + qt) * num_heads + h) * head_dim + 8 * c) = r;
}

// Largest launch (in workgroups) that runs the 32x32 layout on the current
// device: 3/4 of its CUs, which leaves the board below its power limit (see
// the top of the file); 0 if the device cannot be queried.
long long wide_layout_max_workgroups() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
        v = 3 * cus / 4;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// The kernel for a launch of `workgroups` at head_dim: above 96 dims the
// 32x32 layout for launches below the power limit, else the 16x16 one; the
// 16x16 instantiation is the smallest whose 32-dim chunks and 16-dim blocks
// cover head_dim.
template <bool kPartial>
auto* attention_kernel_for(int head_dim, long long workgroups) {
    auto* kernel = workgroups <= wide_layout_max_workgroups() ? attn_fwd_kernel<WaveWide, kPartial>
                                                              : attn_fwd_kernel<Wave<4, 8>, kPartial>;
    if (head_dim <= 32) kernel = attn_fwd_kernel<Wave<1, 2>, kPartial>;
    else if (head_dim <= 64) kernel = attn_fwd_kernel<Wave<2, 4>, kPartial>;
    else if (head_dim <= 80) kernel = attn_fwd_kernel<Wave<3, 5>, kPartial>;
    else if (head_dim <= 96) kernel = attn_fwd_kernel<Wave<3, 6>, kPartial>;
    return kernel;
}

// The same with S on the fp8 MFMA where that costs fewer matrix cycles
// (head dims above 64: one 128-dim fp8 product against three or four 32-dim
// fp16 ones), in the 16x16 layout for every launch size; up to 64 dims the
// exact kernel.
auto* attention_kernel_fp8qk_for(int head_dim, long long workgroups) {
    if (head_dim <= 64) return attention_kernel_for<false>(head_dim, workgroups);
    if (head_dim <= 80) return attn_fwd_kernel<WaveF8<3, 5>, false>;
    if (head_dim <= 96) return attn_fwd_kernel<WaveF8<3, 6>, false>;
    return attn_fwd_kernel<WaveF8<4, 8>, false>;
}

// log2(e) / sqrt(head_dim) in float32: for head_dim 128 this is the product
// of the two float32 constants.
float softmax_log2_factor(int head_dim) {
    const float rsqrt_d = head_dim == kD ? kRsqrtD : (float)(1.0 / std::sqrt((double)head_dim));
    return kLog2e * rsqrt_d;
}

// Workspace of qfa_fp8_varlen_attn_split_noalloc, for callers that cannot
// allocate device memory.  Each GPU the library runs on holds its own copy
// until the process ends; its size covers every split count the automatic
// rule picks (at most 512 virtual query tiles x 256 rows of 264 bytes, about
// 33 MiB).  Host code never passes the array's name to a kernel (on the host
// it is a stand-in, not a device address): it passes the address
// hipGetSymbolAddress returns for the current device.
__device__ __attribute__((aligned(256))) unsigned char scratch[kAttnScratchBytes];

}  // namespace

hipError_t attention_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

size_t attention_workspace_bytes(int num_seqs, int total_tokens, int num_heads, int num_splits) {
    if (num_splits <= 1) return 0;
    const size_t rows = (size_t)num_splits * num_heads * tiles_per_head(total_tokens, num_seqs) * kBM;
    const size_t o_bytes = (rows * kD * sizeof(_Float16) + 255) & ~(size_t)255;
    return o_bytes + rows * 2 * sizeof(float);
}

hipError_t launch_attention(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                            const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads, int head_dim,
                            void* out, hipStream_t s) {
    return launch_attention_split(q8, k8, v8, scales, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim, 1,
                                  nullptr, out, s);
}

hipError_t launch_attention_fp8qk(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                                  const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads,
                                  int head_dim, void* out, hipStream_t s) {
    const int tph = tiles_per_head(total_tokens, num_seqs);
    const long long nwg = (long long)tph * num_heads;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    attention_kernel_fp8qk_for(head_dim, nwg)<<<(unsigned)nwg, kThreads, 0, s>>>(
        q8, k8, v8, scales, cu_seqlens, num_seqs, num_heads, tph, 1, head_dim, softmax_log2_factor(head_dim),
        (__bf16*)out, nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_attention_split(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                                  const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads,
                                  int head_dim, int num_splits, void* workspace, void* out, hipStream_t s) {
    const int tph = tiles_per_head(total_tokens, num_seqs);
    const long long nwg = (long long)tph * num_heads;
    if (nwg <= 0) return hipSuccess;
    if (nwg * num_splits > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    const float c = softmax_log2_factor(head_dim);
    if (num_splits <= 1) {
        attention_kernel_for<false>(head_dim, nwg)<<<(unsigned)nwg, kThreads, 0, s>>>(
            q8, k8, v8, scales, cu_seqlens, num_seqs, num_heads, tph, 1, head_dim, c, (__bf16*)out, nullptr, nullptr);
        return hipGetLastError();
    }
    const size_t rows = (size_t)num_splits * nwg * kBM;
    _Float16* part_o = (_Float16*)workspace;
    v2f* part_ml = (v2f*)((char*)workspace + ((rows * kD * sizeof(_Float16) + 255) & ~(size_t)255));
    attention_kernel_for<true>(head_dim, nwg * num_splits)<<<(unsigned)(nwg * num_splits), kThreads, 0, s>>>(
        q8, k8, v8, scales, cu_seqlens, num_seqs, num_heads, tph, num_splits, head_dim, c, nullptr, part_o, part_ml);
    attn_combine_kernel<<<(unsigned)(nwg * (kBM / kCombineQueries)), 256, 0, s>>>(
        part_o, part_ml, scales, cu_seqlens, num_seqs, num_heads, tph, num_splits, head_dim, (__bf16*)out);
    return hipGetLastError();
}

}  // namespace qfa
