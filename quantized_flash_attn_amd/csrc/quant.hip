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
// Dynamic mode makes one pass over the data in the usual case.  The
// forward's effective amax is max(amax_t, the ring slots other than the one
// being replaced), and the second operand is known before the pass.  So:
//   amax_quantize_kernel   grid (P, 3): streams tensor t once, quantizing
//                          with the scale of that speculative amax (the
//                          other slots' maximum) while taking max|x| as bf16
//                          bit patterns; one partial per workgroup, no
//                          atomics; workgroup (0, 0) snapshots the cursor.
//   requantize_kernel      grid (R, 3): every workgroup reduces the partials
//                          and derives the forward's scale from the ring
//                          (all agree); workgroup (0, t) is the only writer
//                          of ring slot, cursor and scales.  If amax_t did
//                          not exceed the speculative amax, the scale is the
//                          one already used and the codes stand (bit for bit
//                          the codes of a separate amax pass); otherwise the
//                          tensor is quantized again with the new scale.
//                          The second pass runs on the first forwards and
//                          when a tensor sets a new maximum over the window.
//   quantize_kernel<true>  grid (G, 3): static mode, x * inv -> clamp +-448
//                          -> E4M3 (RNE) with the loaded scales.
//   amax_packed_kernel,    amax, then quantize, reading Q, K and V straight out
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
        st->requantized[t] = 0;
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

// Ring maximum over the slots other than the one this forward replaces
// (slot cursor % history_len): the effective amax of the forward is the
// maximum of this and amax_t.  Uniform over the workgroup.
__device__ inline float ring_max_others(const DeviceState* st, int t, int cursor) {
    const int hist = st->history_len;
    const int slot = cursor % hist;
    float r[QFA_MAX_HISTORY];   // every slot at once: one load, no chain of dependent loads
#pragma unroll
    for (int j = 0; j < QFA_MAX_HISTORY; ++j) r[j] = st->ring[t][j];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < QFA_MAX_HISTORY; ++j)
        if (j < hist && j != slot) m = fmaxf(m, r[j]);
    return m;
}

// The forward's scale for tensor t, derived inside every workgroup of the
// second kernel from state written before it started (the amax partials,
// the ring and the cursor snapshot), so all workgroups agree without
// synchronising.  amax_t = max of the partials; the ring's slot
// cursor % history_len receives amax_t, so the effective amax is the maximum
// of amax_t and the other slots (the slot being replaced is excluded: its
// old value leaves the window).  *again is set when amax_t exceeds the other
// slots' maximum, i.e. when the scale differs from the one the first pass
// used.  Workgroup (0, t) writes the slot, the scales, the requantized flag
// and (t = 0) the incremented cursor; nobody else reads those fields during
// this kernel, and its readers exclude the slot, so there is no race.
__device__ float dynamic_inv(DeviceState* st, int t, int n_partials, bool* again) {
    __shared__ uint32_t red[kThreads / 64];
    __shared__ float sh_inv;
    __shared__ int sh_again;
    const int lane = threadIdx.x & 63;
    // This thread's partials (indices past the last are clamped to it: a
    // repeated value does not change the maximum), all loaded before use.
    constexpr int kPerThread = kMaxPartials / kThreads;
    uint32_t v[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) v[r] = st->partial[t][min((int)threadIdx.x + kThreads * r, n_partials - 1)];
    // Ring slots other than the one being replaced, one per lane.
    const float ring_lane = st->ring[t][lane & (QFA_MAX_HISTORY - 1)];   // loaded alongside cursor and history
    const int cursor = st->cursor_snap;
    const int hist = st->history_len;
    const int slot = cursor % hist;
    const float rv = (lane < hist && lane != slot) ? ring_lane : 0.0f;
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
        float others = rv;
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) others = fmaxf(others, __shfl_xor(others, off));  // lanes 0..15
        const float eff = fmaxf(amax, others);
        if (lane == 0) {
            float d, i;
            scales_from_amax(eff, &d, &i);
            sh_inv = i;
            sh_again = amax > others;
            if (blockIdx.x == 0) {
                st->ring[t][slot] = amax;
                st->amax_observed[t] = amax;
                st->amax_eff[t] = eff;
                st->descale[t] = d;
                st->inv[t] = i;
                st->requantized[t] = amax > others;
                if (t == 0) st->cursor = cursor + 1;
            }
        }
    }
    __syncthreads();
    *again = sh_again != 0;
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

// Where tensor t's chunks come from and go to.  A chunk is 8 bf16 in and 8
// codes out; n() chunks per tensor.
//   Split: three [T, H, D] tensors, chunk i of tensor t at src_t + i.
//   Packed: a fused [T, 3, H, D] projection output (D <= 128) into codes
//   [T, H, 128]: output chunk o is dims 8 (o & 15) .. + 7 of head row o >> 4
//   = token * H + h; the first cph = D / 8 chunks of a row come from input
//   chunk (token * 3 + t) * cpr + h * cph + (o & 15), cpr = H * cph, the rest
//   are zero.
struct SplitIO {
    const u32x4* src;
    u32x2* dst;
    int64_t count;
    __device__ int64_t n() const { return count; }
    __device__ u32x4 load(int64_t i) const { return __builtin_nontemporal_load(src + i); }
    __device__ void store(int64_t i, u32x2 c) const { __builtin_nontemporal_store(c, dst + i); }
};

struct PackedIO {
    const u32x4* qkv;
    u32x2* dst;
    uint32_t out_chunks, num_heads, cph, cpr, t;
    __device__ int64_t n() const { return out_chunks; }
    __device__ u32x4 load(int64_t i) const {
        const uint32_t o = (uint32_t)i, row = o >> 4, dc = o & 15;
        if (dc >= cph) return u32x4{0u, 0u, 0u, 0u};
        const uint32_t token = row / num_heads, h = row - token * num_heads;
        return __builtin_nontemporal_load(qkv + ((size_t)token * 3 + t) * cpr + h * cph + dc);
    }
    __device__ void store(int64_t i, u32x2 c) const { __builtin_nontemporal_store(c, dst + i); }
};

// Grid-stride pass over this workgroup's chunks with four chunks in flight
// per thread: codes with factor get_inv() and, if kMax, the running max|x|
// bits.  The first four loads are issued before get_inv() runs, so a scale
// derived from the state overlaps the first memory round trip.
template <bool kMax, class IO, class InvFn>
__device__ inline uint32_t stream_pass(const IO& io, InvFn get_inv) {
    const int64_t n = io.n();
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint32_t m = 0;
    const bool first_full = i + 3 * stride < n;
    u32x4 x0[4];
    if (first_full) {
#pragma unroll
        for (int r = 0; r < 4; ++r) x0[r] = io.load(i + r * stride);
    }
    const float inv = get_inv();
    if (first_full) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (kMax) m = max_abs_bits(x0[r], m);
            io.store(i + r * stride, quantize8(x0[r], inv));
        }
        i += 4 * stride;
    }
    for (; i + 3 * stride < n; i += 4 * stride) {
        u32x4 x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = io.load(i + r * stride);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (kMax) m = max_abs_bits(x[r], m);
            io.store(i + r * stride, quantize8(x[r], inv));
        }
    }
    for (; i < n; i += stride) {
        const u32x4 x = io.load(i);
        if constexpr (kMax) m = max_abs_bits(x, m);
        io.store(i, quantize8(x, inv));
    }
    return m;
}

// Workgroup maximum of m -> partial[t][blockIdx.x].
__device__ inline void store_partial(DeviceState* st, int t, uint32_t m) {
    m = wave_max_u32(m);
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = red[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) r = max(r, red[w]);
        st->partial[t][blockIdx.x] = r;
    }
}

// First pass: codes with the scale of the other slots' maximum, and the
// amax partial.  Workgroup (0, 0) snapshots the ring cursor, which the
// second kernel reads while its workgroup (0, 0) advances the cursor.
template <class IO>
__device__ inline void amax_quantize(DeviceState* st, const IO& io) {
    const int t = blockIdx.y;
    const int cursor = st->cursor;
    const uint32_t m = stream_pass<true>(io, [&] {
        float d, inv;
        scales_from_amax(ring_max_others(st, t, cursor), &d, &inv);
        return inv;
    });
    if (blockIdx.x == 0 && t == 0 && threadIdx.x == 0) st->cursor_snap = cursor;
    store_partial(st, t, m);
}

// Second pass: the forward's scale; quantize tensor t again only if it
// differs from the first pass's.
template <class IO>
__device__ inline void requantize(DeviceState* st, const IO& io, int n_partials) {
    bool again;
    const float inv = dynamic_inv(st, blockIdx.y, n_partials, &again);
    if (again) stream_pass<false>(io, [=] { return inv; });
}

// The static factors do not depend on the data: workgroup 0 records them;
// every workgroup derives the same value from static_eff.
__device__ inline float static_inv(DeviceState* st, int t) {
    const float eff = st->static_eff[t];
    float d, inv;
    scales_from_amax(eff, &d, &inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        st->amax_eff[t] = eff;
        st->descale[t] = d;
        st->inv[t] = inv;
    }
    return inv;
}

__device__ inline SplitIO split_io(const u32x4* q, const u32x4* k, const u32x4* v, u32x2* q8, u32x2* k8, u32x2* v8,
                                   int64_t n_chunks) {
    const int t = blockIdx.y;
    return SplitIO{t == 0 ? q : (t == 1 ? k : v), t == 0 ? q8 : (t == 1 ? k8 : v8), n_chunks};
}

__device__ inline PackedIO packed_io(const u32x4* qkv, u32x2* q8, u32x2* k8, u32x2* v8, uint32_t out_chunks,
                                     uint32_t num_heads, uint32_t cph) {
    const uint32_t t = blockIdx.y;
    return PackedIO{qkv, t == 0 ? q8 : (t == 1 ? k8 : v8), out_chunks, num_heads, cph, num_heads * cph, t};
}

__global__ __launch_bounds__(kThreads) void amax_quantize_kernel(DeviceState* st, const u32x4* __restrict__ q,
                                                                 const u32x4* __restrict__ k,
                                                                 const u32x4* __restrict__ v, int64_t n_chunks,
                                                                 u32x2* __restrict__ q8, u32x2* __restrict__ k8,
                                                                 u32x2* __restrict__ v8) {
    amax_quantize(st, split_io(q, k, v, q8, k8, v8, n_chunks));
}

__global__ __launch_bounds__(kThreads) void requantize_kernel(DeviceState* st, const u32x4* __restrict__ q,
                                                              const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                                              int64_t n_chunks, u32x2* __restrict__ q8,
                                                              u32x2* __restrict__ k8, u32x2* __restrict__ v8,
                                                              int n_partials) {
    requantize(st, split_io(q, k, v, q8, k8, v8, n_chunks), n_partials);
}

__global__ __launch_bounds__(kThreads) void quantize_static_kernel(DeviceState* st, const u32x4* __restrict__ q,
                                                                   const u32x4* __restrict__ k,
                                                                   const u32x4* __restrict__ v, int64_t n_chunks,
                                                                   u32x2* __restrict__ q8, u32x2* __restrict__ k8,
                                                                   u32x2* __restrict__ v8) {
    stream_pass<false>(split_io(q, k, v, q8, k8, v8, n_chunks), [&] { return static_inv(st, blockIdx.y); });
}

__global__ __launch_bounds__(kThreads) void amax_quantize_packed_kernel(DeviceState* st, const u32x4* __restrict__ qkv,
                                                                        uint32_t out_chunks, uint32_t num_heads,
                                                                        uint32_t cph, u32x2* __restrict__ q8,
                                                                        u32x2* __restrict__ k8,
                                                                        u32x2* __restrict__ v8) {
    amax_quantize(st, packed_io(qkv, q8, k8, v8, out_chunks, num_heads, cph));
}

__global__ __launch_bounds__(kThreads) void requantize_packed_kernel(DeviceState* st, const u32x4* __restrict__ qkv,
                                                                     uint32_t out_chunks, uint32_t num_heads,
                                                                     uint32_t cph, u32x2* __restrict__ q8,
                                                                     u32x2* __restrict__ k8, u32x2* __restrict__ v8,
                                                                     int n_partials) {
    requantize(st, packed_io(qkv, q8, k8, v8, out_chunks, num_heads, cph), n_partials);
}

__global__ __launch_bounds__(kThreads) void quantize_static_packed_kernel(DeviceState* st,
                                                                          const u32x4* __restrict__ qkv,
                                                                          uint32_t out_chunks, uint32_t num_heads,
                                                                          uint32_t cph, u32x2* __restrict__ q8,
                                                                          u32x2* __restrict__ k8,
                                                                          u32x2* __restrict__ v8) {
    stream_pass<false>(packed_io(qkv, q8, k8, v8, out_chunks, num_heads, cph),
                       [&] { return static_inv(st, blockIdx.y); });
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
    // One partial per first-pass workgroup (at most kMaxPartials per tensor,
    // each thread streaming >= 8 chunks).  The second pass uses the same grid:
    // a smaller one costs the same when it only derives the scale (about 4 us
    // at 1 x 8192 tokens, 16 heads, most of it the launch and one round trip
    // to the partials) and streams slower when it quantizes again (53 us with
    // 256 workgroups per tensor, 60 with 64, 83 with 32).
    const int g = grid_for(chunks, 8, kMaxPartials);
    amax_quantize_kernel<<<dim3(g, 3), kThreads, 0, s>>>(st, (const u32x4*)q, (const u32x4*)k, (const u32x4*)v, chunks,
                                                         (u32x2*)q8, (u32x2*)k8, (u32x2*)v8);
    requantize_kernel<<<dim3(g, 3), kThreads, 0, s>>>(st, (const u32x4*)q, (const u32x4*)k,
                                                                         (const u32x4*)v, chunks, (u32x2*)q8,
                                                                         (u32x2*)k8, (u32x2*)v8, g);
    return hipGetLastError();
}

// qkv: [total_tokens, 3, num_heads, head_dim] bf16 (head_dim a multiple of
// 8, at most 128); outputs [total_tokens, num_heads, 128] codes.  The caller
// guarantees total_tokens * num_heads * 16 < 2^31.
hipError_t launch_quantize_packed(DeviceState* st, bool dynamic, const uint16_t* qkv, int64_t total_tokens,
                                  int num_heads, int head_dim, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s) {
    const uint32_t cph = (uint32_t)head_dim / 8;
    const uint32_t out_chunks = (uint32_t)total_tokens * (uint32_t)num_heads * 16;
    if (dynamic) {
        const int g = grid_for(out_chunks, 8, kMaxPartials);
        amax_quantize_packed_kernel<<<dim3(g, 3), kThreads, 0, s>>>(st, (const u32x4*)qkv, out_chunks,
                                                                    (uint32_t)num_heads, cph, (u32x2*)q8, (u32x2*)k8,
                                                                    (u32x2*)v8);
        requantize_packed_kernel<<<dim3(g, 3), kThreads, 0, s>>>(
            st, (const u32x4*)qkv, out_chunks, (uint32_t)num_heads, cph, (u32x2*)q8, (u32x2*)k8, (u32x2*)v8, g);
    } else {
        const int g = grid_for(out_chunks, 16, 2048);
        quantize_static_packed_kernel<<<dim3(g, 3), kThreads, 0, s>>>(st, (const u32x4*)qkv, out_chunks,
                                                                      (uint32_t)num_heads, cph, (u32x2*)q8,
                                                                      (u32x2*)k8, (u32x2*)v8);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_static(DeviceState* st, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  int64_t n, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s) {
    const int64_t chunks = n / 8;
    // 4 chunks per thread: small tensors get enough workgroups to cover the memory latency (a 2304-token, 16-head
    // static forward: 8.1 us against 8.9 us with 16); large ones reach the 2048 cap either way
    const int g = grid_for(chunks, 4, 2048);
    quantize_static_kernel<<<dim3(g, 3), kThreads, 0, s>>>(st, (const u32x4*)q, (const u32x4*)k, (const u32x4*)v,
                                                           chunks, (u32x2*)q8, (u32x2*)k8, (u32x2*)v8);
    return hipGetLastError();
}

}  // namespace qfa
