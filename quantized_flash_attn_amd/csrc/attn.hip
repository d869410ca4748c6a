// Non-causal varlen FP8 flash attention for gfx950 (CDNA4).
//
// "FP8 vision encoder attention" (Requirements) runs FP8 attention with
// per-tensor scales over packed variable-length image batches; "FP8 ViT
// Encoder Attention" (intro) feeds it Q/K/V quantized on the fly.  Each
// query attends to every key of its own sequence [cu[b], cu[b+1]).
//
// Inputs are E4M3 codes in HBM (1 byte per element); the kernel works on the
// code values and folds the per-tensor scales into the softmax and epilogue.
//
// Work decomposition
//   * One workgroup = 4 waves = one (head, 128-query tile of one sequence).
//     Query tiles never cross a cu_seqlens boundary.  Workgroup ids are
//     remapped so that consecutive tiles (same head, same K/V) land on the
//     same XCD and share its L2.
//   * Each wave owns 32 queries (two 16-query MFMA blocks) and streams all
//     keys of the sequence in 128-key tiles staged through LDS.
//   * The next tile's K and V are fetched with buffer_load_dwordx4 ... lds
//     while the current tile computes: V lands directly in its swizzled
//     layout, K lands in a staging buffer and is converted to bf16 between
//     two barriers.  Rows past the end of the sequence are out of the buffer
//     descriptor's range and arrive as zeros; their scores are masked.
//
// Per key tile:
//   S^T = K Q^T     v_mfma_f32_16x16x32_bf16 on the exactly converted codes
//                   (every E4M3 value is a bf16 value).  gfx950's fp8 MFMAs
//                   sum each group of 8 products on a 14-bit window below the
//                   group's largest product, truncating the rest; with
//                   outlier-heavy Q/K that moves large logits by up to ~0.4
//                   and flips near-ties.  The bf16 MFMA sums exactly.  The
//                   accumulator gives every lane 32 keys of ONE query, so the
//                   row max / row sum are in-lane plus two lane swaps.
//   online softmax  p = 2^(S*c + 8 - m*c), c = s_q*s_k*log2(e)/sqrt(128), m a
//                   running row max.  The 2^8 shift keeps small p out of E4M3
//                   subnormals.  m (and with it O and l) is only moved when the
//                   tile's max exceeds it by more than 0.5 in log2 units, so p
//                   stays below 2^8.5 = 362 < 448 and most tiles skip the
//                   rescale.
//   P split         hi = E4M3(p), lo = E4M3(p - hi): two fp8 MFMAs
//                   (v_mfma_f32_16x16x128_f8f6f4) give ~8 significant bits of p.
//   O^T += V^T P^T  A = V^T read with ds_read_b64_tr_b8 from row-major fp8 V
//                   in LDS, B = P^T straight from the S^T accumulator layout.
//                   The O^T accumulator again gives each lane one query.
//   epilogue        out = bf16(O * s_v / l).

#include "qfa_internal.h"

namespace qfa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kD = 128;        // head_dim
constexpr int kBM = 128;       // queries per workgroup
constexpr int kBN = 128;       // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKRow = 2 * kD;  // bytes per bf16 K row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRsqrtD = 0.08838834764831845f;  // 1/sqrt(128)
constexpr float kRescaleSlack = 0.5f;            // log2 units the running max may lag

// LDS map (bytes): fp8 K staging | bf16 K | two fp8 V buffers.  80 KiB, so
// two workgroups fit one CU's 160 KiB.
constexpr int kLdsK8 = 0;
constexpr int kLdsKb = kBN * kD;
constexpr int kLdsV = kLdsKb + kBN * kKRow;
constexpr int kVBuf = kBN * kD;
constexpr int kLdsBytes = kLdsV + 2 * kVBuf;

__device__ inline v4f mfma_f8(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ inline v4f mfma_bf16(bf16x8 a, bf16x8 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
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

// Reductions over the four lanes {l, l^16, l^32, l^48} that hold one query.
__device__ inline float quad_max(float x) {
    const v2i a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
    const v2i b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}
__device__ inline float quad_sum(float x) {
    const v2i a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    const v2i b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// LDS layouts (16-byte chunks XOR-swizzled so operand reads hit distinct banks):
//   bf16 K: [key][128] rows of 256 B (16 chunks); 16 consecutive rows read the
//      same chunk -> swizzle by row & 15.
//   fp8 V: [key][128] rows of 128 B (8 chunks); a transpose read touches rows
//      {16a + 4g + b : a in 0..1, b in 0..3} -> swizzle by (row & 3) | ((row >> 4) & 1) << 2.
//   fp8 K staging: unswizzled [key][128].
__device__ inline int swz_k(int row) { return row & 15; }
__device__ inline int swz_v(int row) { return (row & 3) | ((row >> 2) & 4); }

// Per-lane byte offsets, computed once per workgroup so the hot loop only
// adds compile-time immediates (the swizzles reduce to lane constants).
struct LaneOffsets {
    int k_read[4];    // bf16 K operand, chunk c of key block 0 (+ kb * 16 rows)
    int v_read[8];    // fp8 V transpose read, column block db of key group 0 (+ rho * 32 rows)
    uint32_t g_row;   // async load: this lane's row inside a segment times the token stride
    int g_chunk;      // async load: 16-byte chunk of K (unswizzled staging)
    int g_vchunk[2];  // async load: 16-byte chunk of V for segments with (seg >> 1) even / odd
};

// Buffer descriptor word 3 for raw byte addressing on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;

// Asynchronous fetch of one key tile: each wave fills four 1 KiB segments of
// the K staging buffer and of V buffer `vbuf`; lane l of a segment writes
// LDS bytes [16l, 16l + 16), so the V swizzle is applied by choosing which
// global chunk each lane reads.  Segment s holds tile rows [8s, 8s + 8).
// The buffer descriptors start at this head's slice of row kt and end after
// the last row of the sequence: rows past it are out of range, which the
// hardware turns into zeros in LDS.
__device__ inline void issue_tile_loads(const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8,
                                        size_t row_stride, int h, int kt, int seq_hi, unsigned char* smem,
                                        int vbuf, int wave, const LaneOffsets& lo) {
    // Everything but the lane offsets is wave-uniform and lives in SGPRs:
    // each segment gets its own descriptor starting at its first row.
    const int nrows = min(seq_hi - kt, kBN);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int seg = wave * 4 + r;
        const int rows_left = nrows - seg * 8;
        const int nrec = rows_left > 0 ? (rows_left - 1) * (int)row_stride + kD : 0;
        const size_t off = (size_t)(kt + seg * 8) * row_stride + (size_t)h * kD;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k8 + off), 0, nrec, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v8 + off), 0, nrec, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_u8*)(smem + kLdsK8 + seg * 1024), 16,
                                                 (int)(lo.g_row + lo.g_chunk), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_u8*)(smem + kLdsV + vbuf * kVBuf + seg * 1024), 16,
                                                 (int)(lo.g_row + lo.g_vchunk[(r >> 1) & 1]), 0, 0, 0);
    }
}

// fp8 K staging -> bf16 K (exact), by all threads.  Thread t converts
// positions t + 256r: rows (t >> 3) + 32r, whose swizzle (row & 15) is the
// same for every r.
__device__ inline void convert_k_tile(unsigned char* smem, int tid) {
    const int row0 = tid >> 3, c16 = tid & 7;
    const unsigned char* src = smem + kLdsK8 + tid * 16;
    unsigned char* dst0 = smem + kLdsKb + row0 * kKRow + (((2 * c16) ^ swz_k(row0)) << 4);
    unsigned char* dst1 = smem + kLdsKb + row0 * kKRow + (((2 * c16 + 1) ^ swz_k(row0)) << 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const u32x4 w = *(const u32x4*)(src + r * kThreads * 16);
        *(bf16x8*)(dst0 + r * 32 * kKRow) = codes_to_bf16x8(w[0], w[1]);
        *(bf16x8*)(dst1 + r * 32 * kKRow) = codes_to_bf16x8(w[2], w[3]);
    }
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

// Workgroups are dispatched round-robin over the 8 XCDs; give each XCD a
// contiguous range of logical tiles so tiles sharing K/V share an L2.
__device__ inline int xcd_remap(int bid, int nwg) {
    const int q = nwg / 8, r = nwg % 8;
    const int x = bid % 8, k = bid / 8;
    return x * q + min(x, r) + k;
}

struct WaveState {
    float m_run[2];
    float l_run[2];
    v4f o[8][2];
};

// One key tile for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
// kRagged: keys >= nk are past the sequence and masked.
template <bool kRagged>
__device__ __forceinline__ void tile_step(const unsigned char* sKb, const unsigned char* sVt, int nk,
                                          const bf16x8 (&qop)[2][4], float cexp, WaveState& ws, int g,
                                          const LaneOffsets& lo) {
    // ---- S^T = K Q^T (bf16 MFMA on the exact code values) ----
    v4f s[8][2];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        s[kb][0] = s[kb][1] = v4f{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const bf16x8 kop = *(const bf16x8*)(sKb + lo.k_read[c] + kb * 16 * kKRow);
            s[kb][0] = mfma_bf16(kop, qop[0][c], s[kb][0]);
            s[kb][1] = mfma_bf16(kop, qop[1][c], s[kb][1]);
        }
    }
    // lane's scores s[kb][qb][i] belong to key 16kb + 4g + i of the tile
    if constexpr (kRagged) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * kb + 4 * g + i >= nk) s[kb][0][i] = s[kb][1][i] = -INFINITY;
    }

    // ---- running max; rescale O and l only when the max moved far ----
    float m_new[2];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float mx = s[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        m_new[qb] = fmaxf(ws.m_run[qb], quad_max(mx));
        grow |= (m_new[qb] - ws.m_run[qb]) * cexp > kRescaleSlack;
    }
    if (__any(grow)) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float alpha = __builtin_amdgcn_exp2f((ws.m_run[qb] - m_new[qb]) * cexp);
            ws.m_run[qb] = m_new[qb];
            ws.l_run[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < 8; ++db) ws.o[db][qb] *= alpha;
        }
    }

    // ---- p = 2^(S c + 8 - m c), split into E4M3 hi + lo ----
    v8i phi[2], plo[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float bias = 8.0f - ws.m_run[qb] * cexp;
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], cexp, bias));
                if constexpr (kRagged) {
                    if (16 * kb + 4 * g + i >= nk) p[i] = 0.0f;
                }
                lsum += p[i];
            }
            int hw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            hw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hw, true);
            const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
            const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
            int lw = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] - h01[0], p[1] - h01[1], 0, false);
            lw = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] - h23[0], p[3] - h23[1], lw, true);
            phi[qb][kb] = hw;
            plo[qb][kb] = lw;
        }
        ws.l_run[qb] += lsum;
    }

    // ---- O^T += V^T P^T ----
    // Transpose read: in each 16-lane group, lane r receives byte j from the
    // address of lane 2j + (r >> 3), offset r & 7.  Lane 2j + hh of group g
    // points at key 32*rho + 16*(j>>2) + 4g + (j&3), column 16*db + 8*hh, so
    // lane r gets 8 keys of column 16*db + r in the key order the P^T operand
    // uses.  The accumulator input of an MFMA is added exactly, so the running
    // output accumulates in place.
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        v8i vop;
#pragma unroll
        for (int rho = 0; rho < 4; ++rho) {
            const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i*)(lds_u8*)(sVt + lo.v_read[db] + rho * 32 * kD));
            vop[2 * rho] = t[0];
            vop[2 * rho + 1] = t[1];
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            ws.o[db][qb] = mfma_f8(vop, phi[qb], ws.o[db][qb]);
            ws.o[db][qb] = mfma_f8(vop, plo[qb], ws.o[db][qb]);
        }
    }
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8, const uint8_t* __restrict__ v8,
    const float* __restrict__ scales, const int32_t* __restrict__ cu, int num_seqs, int num_heads,
    int tiles_per_head, __bf16* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const int r16 = lane & 15, g = lane >> 4;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int h = logical / tiles_per_head;
    const int vt = logical - h * tiles_per_head;
    const int b = find_sequence(cu, num_seqs, vt);
    const int seq_lo = cu[b], seq_hi = cu[b + 1];
    const int q0 = seq_lo + (vt - (seq_lo / kBM + b)) * kBM;
    if (q0 >= seq_hi) return;  // spare tile (uniform over the workgroup)

    const size_t row_stride = (size_t)num_heads * kD;  // elements between tokens of one head

    LaneOffsets lo;
    {
        // K operand: row 16kb + r16, so row & 15 = r16 for every kb.
#pragma unroll
        for (int c = 0; c < 4; ++c) lo.k_read[c] = r16 * kKRow + (((4 * g + c) ^ swz_k(r16)) << 4);
        // V transpose read: key 32rho + 16(j>>2) + 4g + (j&3); its swizzle
        // depends on j only (bit 4 of the key is bit 2 of j).
        const int j = r16 >> 1, hh = r16 & 1;
        const int key0 = 16 * (j >> 2) + 4 * g + (j & 3);
#pragma unroll
        for (int db = 0; db < 8; ++db) lo.v_read[db] = key0 * kD + ((db ^ swz_v(key0)) << 4) + 8 * hh;
        // Async loads: lane covers row (lane >> 3) of each 8-row segment,
        // physical chunk lane & 7; for V, segment rows 8s..8s+7 have
        // swizzle bit 2 equal to (s >> 1) & 1.
        lo.g_row = (uint32_t)(lane >> 3) * (uint32_t)row_stride;
        const int pc = lane & 7;
        lo.g_chunk = pc * 16;
        lo.g_vchunk[0] = (pc ^ swz_v(lane >> 3)) << 4;
        lo.g_vchunk[1] = (pc ^ swz_v((lane >> 3) + 16)) << 4;
    }

    issue_tile_loads(k8, v8, row_stride, h, seq_lo, seq_hi, smem, 0, wave, lo);

    // Q operand (B of S^T = K Q^T, bf16 16x16x32): lane holds query r16 of the
    // block and the 32 head dims [32g, 32g + 32) as four 8-element chunks; the
    // K operand uses the same (lane group, chunk, element) -> dim mapping.
    bf16x8 qop[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qi = q0 + wave * 32 + qb * 16 + r16;
        u32x4 a = {0, 0, 0, 0}, c = {0, 0, 0, 0};
        if (qi < seq_hi) {
            const u32x4* p = (const u32x4*)(q8 + (size_t)qi * row_stride + (size_t)h * kD + 32 * g);
            a = p[0];
            c = p[1];
        }
        qop[qb][0] = codes_to_bf16x8(a[0], a[1]);
        qop[qb][1] = codes_to_bf16x8(a[2], a[3]);
        qop[qb][2] = codes_to_bf16x8(c[0], c[1]);
        qop[qb][3] = codes_to_bf16x8(c[2], c[3]);
    }

    const float s_q = scales[0], s_k = scales[1], s_v = scales[2];
    const float cexp = s_q * s_k * (kLog2e * kRsqrtD);

    WaveState ws;
    ws.m_run[0] = ws.m_run[1] = -1e30f;
    ws.l_run[0] = ws.l_run[1] = 0.0f;
#pragma unroll
    for (int db = 0; db < 8; ++db) ws.o[db][0] = ws.o[db][1] = v4f{0, 0, 0, 0};

    wait_async_loads();
    __syncthreads();
    convert_k_tile(smem, tid);
    __syncthreads();

    int vbuf = 0;
    for (int kt = seq_lo; kt < seq_hi; kt += kBN) {
        const int nk = min(kBN, seq_hi - kt);
        const bool more = kt + kBN < seq_hi;
        if (more) issue_tile_loads(k8, v8, row_stride, h, kt + kBN, seq_hi, smem, vbuf ^ 1, wave, lo);
        const unsigned char* sVt = smem + kLdsV + vbuf * kVBuf;
        if (nk == kBN)
            tile_step<false>(smem + kLdsKb, sVt, nk, qop, cexp, ws, g, lo);
        else
            tile_step<true>(smem + kLdsKb, sVt, nk, qop, cexp, ws, g, lo);
        wait_async_loads();
        __syncthreads();  // all waves are done with this tile's K and V; the next tile has landed
        if (more) {
            convert_k_tile(smem, tid);
            __syncthreads();
        }
        vbuf ^= 1;
    }

    // ---- epilogue: lane holds O^T[d = 16db + 4g + i][query r16] ----
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float l = quad_sum(ws.l_run[qb]);
        const int qi = q0 + wave * 32 + qb * 16 + r16;
        if (qi < seq_hi) {
            const float f = s_v / l;
            __bf16* dst = out + (size_t)qi * row_stride + (size_t)h * kD + 4 * g;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                bf16x4 r;
                r[0] = (__bf16)(ws.o[db][qb][0] * f);
                r[1] = (__bf16)(ws.o[db][qb][1] * f);
                r[2] = (__bf16)(ws.o[db][qb][2] * f);
                r[3] = (__bf16)(ws.o[db][qb][3] * f);
                *(bf16x4*)(dst + 16 * db) = r;
            }
        }
    }
}

}  // namespace

hipError_t launch_attention(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                            const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads, void* out,
                            hipStream_t s) {
    const int tiles_per_head = total_tokens / kBM + num_seqs;
    const long long nwg = (long long)tiles_per_head * num_heads;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    attn_fwd_kernel<<<(unsigned)nwg, kThreads, 0, s>>>(q8, k8, v8, scales, cu_seqlens, num_seqs, num_heads,
                                                       tiles_per_head, (__bf16*)out);
    return hipGetLastError();
}

}  // namespace qfa
