// Non-causal varlen BF16 flash attention for gfx950 (CDNA4): the baseline
// the FP8 path is weighed against.  "FP8 ViT Encoder Attention"
// (Performance) and "FP8 vision encoder attention" (Expected performance)
// state every gain of FP8 encoder attention as a BF16 -> FP8 pair on the same
// shapes; this kernel gives the BF16 side of that pair on MI355X.
//
//   out[i,h,:] = sum_j softmax_j(<q_i, k_j> / sqrt(128)) v_j
// over the keys j of the sequence [cu[b], cu[b+1]) that holds query i.
//
// It keeps the E4M3 kernel's workgroup shape (8 waves, 256 queries, 128-key
// tiles), tile mapping, XCD order, ping-pong schedule and online softmax
// (attn_common.h).  What differs:
//   * K and V are bf16 in HBM and land in LDS directly (buffer_load ... lds,
//     no registers, no staging, no conversion) in 256-byte rows whose 16-byte
//     chunks are XOR-swizzled per row, so both operand reads are free of bank
//     conflicts.  Two K and two V buffers: 128 KiB of LDS.
//   * S = K Q^T and O^T += V^T P^T are both v_mfma_f32_16x16x32_bf16; P is
//     rounded to bf16 (nearest even) from the fp32 probabilities, and l sums
//     the fp32 probabilities.
//   * The V^T operand is read with ds_read_b64_tr_b16 from row-major V.
//   * The softmax scale is 1/sqrt(128) alone; there are no per-tensor scales.

#include "attn_common.h"

namespace qfa {
namespace {

using namespace attn;

constexpr int kLdsK = 0;
constexpr int kLdsV = 2 * kTileBytes;
constexpr int kLdsBytes = 4 * kTileBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// LDS layouts: the K and V tiles of attn_common.h (swz_k, swz_v).

// Asynchronous fetch of one 128-key tile of K or V: wave w fills the 1 KiB
// segments 4w .. 4w + 3 (tile rows [16w, 16w + 16)); lane l of a segment
// writes LDS bytes [16l, 16l + 16), i.e. row l >> 4 of the segment, physical
// chunk l & 15, so the swizzle is applied by choosing which global chunk
// each lane reads.  `lane_off[r]` is that choice for segment 4w + r.  Each
// segment's buffer descriptor starts at this head's slice of its first row
// and ends after the last row of the sequence: rows past it are out of
// range, which the hardware turns into zeros in LDS.
__device__ inline void issue_tile_load(const unsigned char* __restrict__ src, uint32_t row_stride, int h, int kt,
                                       int seq_hi, lds_u8* dst, int wave, const uint32_t (&lane_off)[4]) {
    const int nrows = min(seq_hi - kt, kBN);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int seg = wave * 4 + r;
        const int rows_left = nrows - seg * 4;
        const int nrec = rows_left > 0 ? (rows_left - 1) * (int)row_stride + kRow : 0;
        const size_t off = (size_t)(kt + seg * 4) * row_stride + (size_t)h * kRow;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)(src + off), 0, nrec, kRsrcWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + seg * 1024, 16, (int)lane_off[r], 0, 0, 0);
    }
}

// Everything one wave carries through the key loop.  Lane (r16, g) of a
// 16x16 accumulator holds rows 4g..4g+3 of column r16 (scores: rows = keys,
// columns = queries; output: rows = head dims, columns = queries).
struct Wave {
    static constexpr int kDB = 8;   // live 16-dim output blocks
    static constexpr bool kBlockRescale = false;   // one rescale decision per wave (fewer registers)
    const unsigned char* k;
    const unsigned char* v;
    uint32_t row_stride;   // bytes between tokens of one head (uniform)
    int h, seq_lo, seq_hi, nt, nk_last, wave;
    float cexp;            // log2(e) / sqrt(128)
    uint32_t k_rd;         // K operand: row r16, chunk (4g ^ r16); chunk c of the operand at k_rd ^ (c << 4)
    uint32_t v_rd;         // V^T read: row 4g + e, byte 8c + 32 (4(g & 1) + e); d block db at v_rd ^ (db << 5)
    uint32_t g_k[4], g_v[4];  // async loads: row-in-segment * stride + swizzled 16-byte chunk, per segment
    int g4;                // 4 g: first key row of this lane inside a 16-key block
    bf16x8 q[kQB][4];      // Q operand (B of S = K Q^T)
    float mc[kQB];         // running row max in log2 units (S c), within the rescale slack of the true max
    v4f o[8][kQB];         // O^T blocks [d block][query block]
    float l[kQB];          // running sum of p over the keys this lane holds (reduced over the quad at the end)

    __device__ __forceinline__ void load_k(lds_u8* lds, int t, int buf) const {
        issue_tile_load(k, row_stride, h, seq_lo + t * kBN, seq_hi, lds + kLdsK + buf * kTileBytes, wave, g_k);
    }
    __device__ __forceinline__ void load_v(lds_u8* lds, int t, int buf) const {
        issue_tile_load(v, row_stride, h, seq_lo + t * kBN, seq_hi, lds + kLdsV + buf * kTileBytes, wave, g_v);
    }
};

// The softmax step of a key tile is split over two slots to even out the
// VALU work of the two groups: softmax_head (mask, row max, rescale, and p
// of key blocks [0, kSplit)) and, in the next slot, the remaining key
// blocks followed by the P^T operands.
constexpr int kSplit = 5;

// The key loop of one wave group.  Period t (t = 0..nt) has four slots
// separated by workgroup barriers:
//            slot 1             slot 2          slot 3             slot 4
//   A (kB=0) S_t = K_t Q^T      p_t (head)      p_t (tail), pack   O += P_t V_t
//   B (kB=1) p_{t-1} (tail),    O += P V_{t-1}  S_t = K_t Q^T       p_t (head)
//            pack
// Loads: K_{t+1} at slot 1 (lands by the end of slot 2), V_{t+1} at slot 3
// (lands by the end of slot 4).  Buffer lifetimes: K_t is read in slots 1
// (A) and 3 (B) of period t and rewritten with K_{t+2} at slot 1 of period
// t+1; V_t is read in slot 4 of period t (A) and slot 2 of period t+1 (B),
// and rewritten with V_{t+2} at slot 3 of period t+1.
template <bool kB>
__device__ __forceinline__ void key_loop(Wave& w, unsigned char* smem) {
    lds_u8* const lds = (lds_u8*)smem;
    const int nt = w.nt;
    v4f s[8][kQB];
    bf16x8 pop[kQB][4];
    for (int t = 0; t <= nt; ++t) {
        const int cur = t & 1, prev = cur ^ 1;
        const int nk_t = (t + 1 < nt) ? kBN : w.nk_last;   // valid keys of tile t (t < nt)
        const int nk_p = (t < nt) ? kBN : w.nk_last;       // valid keys of tile t - 1 (t >= 1)
        // slot 1
        if (t + 1 < nt) w.load_k(lds, t + 1, prev);
        if constexpr (!kB) {
            if (t < nt) {
                mfma_phase_begin();
                qk_tile(smem + kLdsK + cur * kTileBytes, w.k_rd, w.q, s);
                mfma_phase_end();
            }
        } else {
            if (t >= 1) pack_tile<kSplit>(w, s, nk_p, pop, w.l);
        }
        __syncthreads();
        // slot 2
        if constexpr (!kB) {
            if (t < nt) softmax_head<kSplit>(w, s, nk_t);
        } else {
            if (t >= 1) {
                mfma_phase_begin();
                pv_tile(smem + kLdsV + prev * kTileBytes, w.v_rd, pop, w.o);
                mfma_phase_end();
            }
        }
        wait_async_loads();
        __syncthreads();
        // slot 3
        if (t + 1 < nt) w.load_v(lds, t + 1, prev);
        if constexpr (!kB) {
            if (t < nt) pack_tile<kSplit>(w, s, nk_t, pop, w.l);
        } else {
            if (t < nt) {
                mfma_phase_begin();
                qk_tile(smem + kLdsK + cur * kTileBytes, w.k_rd, w.q, s);
                mfma_phase_end();
            }
        }
        __syncthreads();
        // slot 4
        if constexpr (!kB) {
            if (t < nt) {
                mfma_phase_begin();
                pv_tile(smem + kLdsV + cur * kTileBytes, w.v_rd, pop, w.o);
                mfma_phase_end();
            }
        } else {
            if (t < nt) softmax_head<kSplit>(w, s, nk_t);
        }
        wait_async_loads();
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads, 1) void attn_bf16_fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ cu, int num_seqs, int num_heads, int tph, __bf16* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];
    lds_u8* const lds = (lds_u8*)smem;

    const int tid = threadIdx.x, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;

    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int h = logical / tph;
    const int vt = logical - h * tph;
    const int b = find_sequence(cu, num_seqs, vt);
    const int seq_lo = cu[b], seq_hi = cu[b + 1];
    const int q0 = seq_lo + (vt - (seq_lo / kBM + b)) * kBM;
    if (q0 >= seq_hi) return;  // spare tile (uniform over the workgroup)

    Wave w;
    w.k = (const unsigned char*)k;
    w.v = (const unsigned char*)v;
    w.row_stride = (uint32_t)num_heads * kRow;
    w.h = h;
    w.seq_lo = seq_lo;
    w.seq_hi = seq_hi;
    w.nt = (seq_hi - seq_lo + kBN - 1) / kBN;
    w.nk_last = seq_hi - seq_lo - (w.nt - 1) * kBN;
    w.wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const bool group_b = w.wave >= kWaves / 2;          // wave-uniform
    {
        w.k_rd = k_operand_offset(r16, g);
        w.v_rd = v_operand_offset(r16, g);
        // Async loads: lane covers row rr = lane >> 4 of each 4-row segment
        // and physical chunk pc = lane & 15; segment 4w + r holds tile rows
        // 16w + 4r + rr, whose swizzles are 4r + rr (K) and 2(4(r & 1) + rr) (V).
        const uint32_t rr = (uint32_t)lane >> 4, pc = (uint32_t)lane & 15;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            w.g_k[r] = rr * w.row_stride + 16 * (pc ^ swz_k(4 * r + rr));
            w.g_v[r] = rr * w.row_stride + 16 * (pc ^ swz_v(4 * r + rr));
        }
        w.g4 = 4 * g;
    }

    // ---- prologue: K_0 and V_0 in flight; Q operand ----
    w.load_k(lds, 0, 0);
    w.load_v(lds, 0, 0);

    // Q operand (B of S = K Q^T, bf16 16x16x32): for the c-th MFMA, lane
    // holds query r16 of the block and head dims 32c + 8g .. + 7, the
    // mapping the K operand uses.
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = q0 + w.wave * (16 * kQB) + qb * 16 + r16;
        u32x4 a[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
        if (qi < seq_hi) {
            const unsigned char* src = (const unsigned char*)q + (size_t)qi * w.row_stride + (size_t)h * kRow + 16 * g;
#pragma unroll
            for (int c = 0; c < 4; ++c) a[c] = *(const u32x4*)(src + 64 * c);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) w.q[qb][c] = __builtin_bit_cast(bf16x8, a[c]);
    }
    w.cexp = kLog2e * kRsqrtD;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) w.o[db][qb] = v4f{0, 0, 0, 0};
        w.l[qb] = 0.0f;
        w.mc[qb] = kMInit;
    }

    wait_async_loads();
    __syncthreads();

    // ---- key loop: group A runs tile t in period t, group B runs its slots
    // 1-2 on tile t-1 and 3-4 on tile t; both copies of the loop execute the
    // same sequence of barriers.
    if (group_b)
        key_loop<true>(w, smem);
    else
        key_loop<false>(w, smem);

    // ---- epilogue: lane holds O^T[d = 16db + 4g + i][query r16] ----
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int qi = q0 + w.wave * (16 * kQB) + qb * 16 + r16;
        if (qi < seq_hi) {
            const float f = 1.0f / quad_sum(w.l[qb]);
            __bf16* dst = out + (size_t)qi * num_heads * kD + (size_t)h * kD + 4 * g;
#pragma unroll
            for (int db = 0; db < 8; ++db) {
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

}  // namespace

hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                 int num_seqs, int total_tokens, int num_heads, void* out, hipStream_t s) {
    const int tph = tiles_per_head(total_tokens, num_seqs);
    const long long nwg = (long long)tph * num_heads;
    if (nwg <= 0) return hipSuccess;
    if (nwg > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    attn_bf16_fwd_kernel<<<(unsigned)nwg, kThreads, 0, s>>>((const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                                                            cu_seqlens, num_seqs, num_heads, tph, (__bf16*)out);
    return hipGetLastError();
}

}  // namespace qfa
