// Scale state, per-tensor amax and bf16 -> E4M3 quantization for gfx950.
//
// Dynamic scaling ("FP8 ViT Encoder Attention", Usage; "FP8 vision encoder
// attention", Enable FP8 attention): each forward observes the amax of Q, K
// and V, records it in a 16-entry circular buffer per tensor and derives the
// forward's scale from the buffer's maximum.  Static scaling ("FP8 ViT
// Encoder Attention", Calibrate-Once, Reuse Workflow): loaded amax values
// times a margin.  Quantization ("FP8 ViT Encoder Attention", intro) turns
// Q/K/V into FP8 before the attention call.
//
// Kernels (both HBM-streaming):
//   amax_partial_kernel    grid (P, 3): max of |x| as bf16 bit patterns,
//                          one partial per workgroup, no atomics; workgroup
//                          (0, 0) also snapshots the ring cursor.  Its loads
//                          allocate in the caches (unlike quantize's
//                          streaming loads), so that quantize, which reads
//                          the same tensors right after, finds part of them
//                          in the 256 MB Infinity Cache.
//   quantize_kernel        grid (G, 3): x * inv -> clamp +-448 -> E4M3 (RNE).
//                          Dynamic mode: every workgroup first reduces its
//                          tensor's partials and derives the forward's scale
//                          from the ring itself (all workgroups compute the
//                          same value); workgroup (0, t) is the only writer of
//                          ring slot, cursor and scales.  No atomics.
//   amax_packed_kernel,    the same two steps reading Q, K and V straight out
//   quantize_packed_kernel of a fused QKV projection output [T, 3, H, D]
//                          (D <= 128) and writing codes [T, H, 128] whose dims
//                          past D are zero, the layout the attention kernel
//                          reads.  This replaces the split into three tensors
//                          and the head-dim padding that "FP8 ViT Encoder
//                          Attention" (Performance) counts among the costs of
//                          small images.

#include "qfa_internal.h"

// Every float operation here must round exactly as written (bit-exact codes).
#pragma clang fp contract(off)

namespace qfa {
namespace {

constexpr int kThreads = 256;
constexpr float kFp8Max = 448.0f;
constexpr float kAmaxFloor = 0x1p-100f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// a = max(amax_eff, 2^-100); descale = fp32(a / 448); inv = fp32(448 / a).
// Both divisions are IEEE float32 (correctly rounded; no fast-math).
__device__ inline void scales_from_amax(float amax_eff, float* descale, float* inv) {
    const float a = fmaxf(amax_eff, kAmaxFloor);
    *descale = a / kFp8Max;
    *inv = kFp8Max / a;
}

__global__ void init_state_kernel(DeviceState* st, int history_len, float e0, float e1, float e2) {
    const int t = threadIdx.x;
    if (t < 3 * QFA_MAX_HISTORY) (&st->ring[0][0])[t] = 0.0f;
    if (t < 3) {
        st->amax_observed[t] = 0.0f;
        st->amax_eff[t] = 0.0f;
        float d, i;
        scales_from_amax(0.0f, &d, &i);
        st->descale[t] = d;
        st->inv[t] = i;
        st->static_eff[t] = t == 0 ? e0 : (t == 1 ? e1 : e2);
    }
    if (t == 0) {
        st->cursor = 0;
        st->history_len = history_len;
    }
}

__device__ inline uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    return m;
}

// |x| of a bf16 is its bit pattern with the sign cleared; for finite values
// the integer order of those patterns is the order of the magnitudes, so the
// integer maximum is exact and independent of reduction order.
__device__ inline uint32_t max_abs_bits(u32x4 w, uint32_t m) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m = max(m, w[j] & 0x7FFFu);
        m = max(m, (w[j] >> 16) & 0x7FFFu);
    }
    return m;
}

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const u32x4* __restrict__ q, const u32x4* __restrict__ k,
                                                                const u32x4* __restrict__ v, int64_t n_chunks,
                                                                DeviceState* st) {
    const int t = blockIdx.y;
    uint32_t* __restrict__ partial = &st->partial[0][0];
    // The ring cursor as this forward finds it; the quantize kernel reads the
    // snapshot while its workgroup (0, 0) advances the cursor itself.
    if (blockIdx.x == 0 && t == 0 && threadIdx.x == 0) st->cursor_snap = st->cursor;
    const u32x4* __restrict__ src = t == 0 ? q : (t == 1 ? k : v);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t m = 0;
    for (; i + 3 * stride < n_chunks; i += 4 * stride) {
        const u32x4 a = src[i];
        const u32x4 b = src[i + stride];
        const u32x4 c = src[i + 2 * stride];
        const u32x4 d = src[i + 3 * stride];
        m = max_abs_bits(a, m);
        m = max_abs_bits(b, m);
        m = max_abs_bits(c, m);
        m = max_abs_bits(d, m);
    }
    for (; i < n_chunks; i += stride) m = max_abs_bits(src[i], m);
    m = wave_max_u32(m);
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
        partial[t * kMaxPartials + blockIdx.x] = r;
    }
}

// The forward's scale for tensor t, derived inside every quantize workgroup
// from state written before this kernel started (the amax partials, the
// ring and the cursor snapshot), so all workgroups agree without
// synchronising.  amax_t = max of the partials; the ring's slot
// cursor % history_len receives amax_t, so the effective amax is the maximum
// of amax_t and the other slots (the slot being replaced is excluded: its
// old value leaves the window).  Workgroup (0, t) writes the slot, the
// scales and (t = 0) the incremented cursor; nobody else reads those fields
// during this kernel, and its readers exclude the slot, so there is no race.
__device__ float dynamic_inv(DeviceState* st, int t, int n_partials) {
    __shared__ uint32_t red[kThreads / 64];
    __shared__ float sh_inv;
    const int lane = threadIdx.x & 63;
    // This thread's partials (indices past the last are clamped to it: a
    // repeated value does not change the maximum), all loaded before use.
    constexpr int kPerThread = kMaxPartials / kThreads;
    uint32_t v[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) v[r] = st->partial[t][min((int)threadIdx.x + kThreads * r, n_partials - 1)];
    // Ring slots other than the one being replaced, one per lane.
    const int cursor = st->cursor_snap;
    const int hist = st->history_len;
    const int slot = cursor % hist;
    const float rv = (lane < hist && lane != slot) ? st->ring[t][lane] : 0.0f;
    uint32_t m = 0;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) m = max(m, v[r]);
    m = wave_max_u32(m);
    if (lane == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x < 64) {
        uint32_t bits = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) bits = max(bits, red[w]);
        const float amax = __uint_as_float(bits << 16);
        float eff = fmaxf(amax, rv);
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) eff = fmaxf(eff, __shfl_xor(eff, off));  // max over lanes 0..15
        if (lane == 0) {
            float d, i;
            scales_from_amax(eff, &d, &i);
            sh_inv = i;
            if (blockIdx.x == 0) {
                st->ring[t][slot] = amax;
                st->amax_observed[t] = amax;
                st->amax_eff[t] = eff;
                st->descale[t] = d;
                st->inv[t] = i;
                if (t == 0) st->cursor = cursor + 1;
            }
        }
    }
    __syncthreads();
    return sh_inv;
}

// 8 bf16 values -> 8 E4M3 codes: fp32 multiply (RNE), clamp to +-448 (the
// conversion instruction alone turns values beyond the format into NaN),
// then v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950, RNE, sign of zero kept).
__device__ inline u32x2 quantize8(u32x4 w, float inv) {
    u32x2 out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const uint32_t w0 = w[2 * j], w1 = w[2 * j + 1];
        float y0 = __uint_as_float(w0 << 16) * inv;
        float y1 = __uint_as_float(w0 & 0xFFFF0000u) * inv;
        float y2 = __uint_as_float(w1 << 16) * inv;
        float y3 = __uint_as_float(w1 & 0xFFFF0000u) * inv;
        y0 = __builtin_amdgcn_fmed3f(y0, -kFp8Max, kFp8Max);
        y1 = __builtin_amdgcn_fmed3f(y1, -kFp8Max, kFp8Max);
        y2 = __builtin_amdgcn_fmed3f(y2, -kFp8Max, kFp8Max);
        y3 = __builtin_amdgcn_fmed3f(y3, -kFp8Max, kFp8Max);
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, r, true);
        out[j] = (uint32_t)r;
    }
    return out;
}

template <bool kStatic>
__global__ __launch_bounds__(kThreads) void quantize_kernel(DeviceState* st, const u32x4* __restrict__ q,
                                                            const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                            int64_t n_chunks, u32x2* __restrict__ q8,
                                                            u32x2* __restrict__ k8, u32x2* __restrict__ v8,
                                                            int n_partials) {
    const int t = blockIdx.y;
    float inv;
    if constexpr (kStatic) {
        const float eff = st->static_eff[t];
        float d;
        scales_from_amax(eff, &d, &inv);
        // The static factors do not depend on the data: workgroup 0 records
        // them; every workgroup derives the same value from static_eff.
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            st->amax_eff[t] = eff;
            st->descale[t] = d;
            st->inv[t] = inv;
        }
    } else {
        inv = dynamic_inv(st, t, n_partials);
    }
    const u32x4* __restrict__ src = t == 0 ? q : (t == 1 ? k : v);
    u32x2* __restrict__ dst = t == 0 ? q8 : (t == 1 ? k8 : v8);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    for (; i + 3 * stride < n_chunks; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(quantize8(a, inv), dst + i);
        __builtin_nontemporal_store(quantize8(b, inv), dst + i + stride);
        __builtin_nontemporal_store(quantize8(c, inv), dst + i + 2 * stride);
        __builtin_nontemporal_store(quantize8(d, inv), dst + i + 3 * stride);
    }
    for (; i < n_chunks; i += stride) __builtin_nontemporal_store(quantize8(__builtin_nontemporal_load(src + i), inv), dst + i);
}

// Packed input: tensor t's chunk i (8 consecutive bf16 of one head row) is
// chunk (token * 3 + t) * cpr + w of the [T, 3, H, D] array, with
// token = i / cpr, w = i % cpr and cpr = H * D / 8 chunks per (token, tensor).
__global__ __launch_bounds__(kThreads) void amax_packed_kernel(const u32x4* __restrict__ qkv, uint32_t n_chunks,
                                                               uint32_t cpr, DeviceState* st) {
    const int t = blockIdx.y;
    uint32_t* __restrict__ partial = &st->partial[0][0];
    if (blockIdx.x == 0 && t == 0 && threadIdx.x == 0) st->cursor_snap = st->cursor;
    const uint32_t stride = gridDim.x * kThreads;
    auto src = [&](uint32_t i) {
        const uint32_t token = i / cpr, w = i - token * cpr;
        return qkv + ((size_t)token * 3 + t) * cpr + w;
    };
    uint32_t m = 0;
    uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    // four independent loads in flight per thread (i + 3 stride < n_chunks < 2^31: no overflow)
    for (; i + 3 * stride < n_chunks; i += 4 * stride) {
        const u32x4 a = *src(i);
        const u32x4 b = *src(i + stride);
        const u32x4 c = *src(i + 2 * stride);
        const u32x4 d = *src(i + 3 * stride);
        m = max_abs_bits(a, m);
        m = max_abs_bits(b, m);
        m = max_abs_bits(c, m);
        m = max_abs_bits(d, m);
    }
    for (; i < n_chunks; i += stride) m = max_abs_bits(*src(i), m);
    m = wave_max_u32(m);
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
        partial[t * kMaxPartials + blockIdx.x] = r;
    }
}

// Output chunk o of tensor t (8 codes) is dims 8 (o & 15) .. + 7 of head row
// o >> 4 = token * H + h of the [T, H, 128] codes; the first cph = D / 8
// chunks of a row come from the packed input, the rest are zero.
template <bool kStatic>
__global__ __launch_bounds__(kThreads) void quantize_packed_kernel(DeviceState* st, const u32x4* __restrict__ qkv,
                                                                   uint32_t n_out_chunks, uint32_t num_heads,
                                                                   uint32_t cph, u32x2* __restrict__ q8,
                                                                   u32x2* __restrict__ k8, u32x2* __restrict__ v8,
                                                                   int n_partials) {
    const int t = blockIdx.y;
    float inv;
    if constexpr (kStatic) {
        const float eff = st->static_eff[t];
        float d;
        scales_from_amax(eff, &d, &inv);
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            st->amax_eff[t] = eff;
            st->descale[t] = d;
            st->inv[t] = inv;
        }
    } else {
        inv = dynamic_inv(st, t, n_partials);
    }
    u32x2* __restrict__ dst = t == 0 ? q8 : (t == 1 ? k8 : v8);
    const uint32_t cpr = num_heads * cph;
    const uint32_t stride = gridDim.x * kThreads;
    // Input chunk of output chunk o (valid when (o & 15) < cph).
    auto src = [&](uint32_t o) {
        const uint32_t row = o >> 4, dc = o & 15;
        const uint32_t token = row / num_heads, h = row - token * num_heads;
        return qkv + ((size_t)token * 3 + t) * cpr + h * cph + dc;
    };
    const u32x4 zero = {0u, 0u, 0u, 0u};
    uint32_t o = blockIdx.x * kThreads + threadIdx.x;
    // four independent chunks in flight per thread (o + 3 stride < n_out_chunks < 2^31: no overflow)
    for (; o + 3 * stride < n_out_chunks; o += 4 * stride) {
        u32x4 x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t oo = o + r * stride;
            x[r] = (oo & 15) < cph ? __builtin_nontemporal_load(src(oo)) : zero;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) __builtin_nontemporal_store(quantize8(x[r], inv), dst + o + r * stride);
    }
    for (; o < n_out_chunks; o += stride) {
        const u32x4 x = (o & 15) < cph ? __builtin_nontemporal_load(src(o)) : zero;
        __builtin_nontemporal_store(quantize8(x, inv), dst + o);
    }
}

int grid_for(int64_t n_chunks, int64_t chunks_per_thread, int cap) {
    int64_t g = (n_chunks + kThreads * chunks_per_thread - 1) / (kThreads * chunks_per_thread);
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

}  // namespace

hipError_t launch_init_state(DeviceState* st, int history_len, const float static_eff[3], hipStream_t s) {
    init_state_kernel<<<1, 64, 0, s>>>(st, history_len, static_eff[0], static_eff[1], static_eff[2]);
    return hipGetLastError();
}

// n: elements per tensor (a multiple of 128, so of 8).
hipError_t launch_quantize_dynamic(DeviceState* st, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   int64_t n, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s) {
    const int64_t chunks = n / 8;
    // Grid shapes from a sweep at 1 x 8192 tokens, 16 heads (amax: 256
    // workgroups per tensor, each thread streaming >= 8 chunks; quantize: 16
    // chunks per thread): 74 % of HBM peak for the pair, against 66 % with
    // 4x more, thinner workgroups (whose scale prologue then dominates).
    const int ga = grid_for(chunks, 8, kMaxPartials);
    amax_partial_kernel<<<dim3(ga, 3), kThreads, 0, s>>>((const u32x4*)q, (const u32x4*)k, (const u32x4*)v, chunks, st);
    const int gq = grid_for(chunks, 16, 2048);
    quantize_kernel<false><<<dim3(gq, 3), kThreads, 0, s>>>(st, (const u32x4*)q, (const u32x4*)k, (const u32x4*)v,
                                                           chunks, (u32x2*)q8, (u32x2*)k8, (u32x2*)v8, ga);
    return hipGetLastError();
}

// qkv: [total_tokens, 3, num_heads, head_dim] bf16 (head_dim a multiple of
// 8, at most 128); outputs [total_tokens, num_heads, 128] codes.  The caller
// guarantees total_tokens * num_heads * 16 < 2^31.
hipError_t launch_quantize_packed(DeviceState* st, bool dynamic, const uint16_t* qkv, int64_t total_tokens,
                                  int num_heads, int head_dim, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s) {
    const uint32_t cph = (uint32_t)head_dim / 8;
    const uint32_t cpr = (uint32_t)num_heads * cph;
    const uint32_t in_chunks = (uint32_t)total_tokens * cpr;            // per tensor
    const uint32_t out_chunks = (uint32_t)total_tokens * (uint32_t)num_heads * 16;
    int ga = 1;
    if (dynamic) {
        ga = grid_for(in_chunks, 8, kMaxPartials);
        amax_packed_kernel<<<dim3(ga, 3), kThreads, 0, s>>>((const u32x4*)qkv, in_chunks, cpr, st);
    }
    const int gq = grid_for(out_chunks, 16, 2048);
    if (dynamic)
        quantize_packed_kernel<false><<<dim3(gq, 3), kThreads, 0, s>>>(st, (const u32x4*)qkv, out_chunks,
                                                                       (uint32_t)num_heads, cph, (u32x2*)q8,
                                                                       (u32x2*)k8, (u32x2*)v8, ga);
    else
        quantize_packed_kernel<true><<<dim3(gq, 3), kThreads, 0, s>>>(st, (const u32x4*)qkv, out_chunks,
                                                                      (uint32_t)num_heads, cph, (u32x2*)q8,
                                                                      (u32x2*)k8, (u32x2*)v8, 1);
    return hipGetLastError();
}

hipError_t launch_quantize_static(DeviceState* st, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  int64_t n, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s) {
    const int64_t chunks = n / 8;
    const int gq = grid_for(chunks, 16, 2048);
    quantize_kernel<true><<<dim3(gq, 3), kThreads, 0, s>>>(st, (const u32x4*)q, (const u32x4*)k, (const u32x4*)v,
                                                          chunks, (u32x2*)q8, (u32x2*)k8, (u32x2*)v8, 1);
    return hipGetLastError();
}

}  // namespace qfa
