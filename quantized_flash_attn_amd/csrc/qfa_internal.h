// Internal declarations shared by the C ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "qfa.h"

namespace qfa {

// Partial amax results one forward may write per tensor (the amax grid is
// capped to this many workgroups per tensor).
constexpr int kMaxPartials = 256;

// Device-resident scale state of one attention layer (the caller's buffer).
// Tensor index t: 0 = Q, 1 = K, 2 = V.
struct DeviceState {
    float ring[3][QFA_MAX_HISTORY];   // observed amax values; unfilled slots are 0
    float amax_observed[3];           // amax seen by the last dynamic forward
    float amax_eff[3];                // effective amax of the last forward
    float descale[3];                 // dequantization factors s_t (read by attention)
    float inv[3];                     // quantization factors
    float static_eff[3];              // fp32(static_amax * margin)
    int32_t cursor;                   // dynamic forwards so far
    int32_t history_len;              // 1..16
    int32_t requantized[3];           // 1 if the last dynamic forward needed the second pass for tensor t
    int32_t cursor_snap;              // cursor as the current forward's first pass found it
    alignas(16) uint32_t partial[3][kMaxPartials];  // per-workgroup max of |bf16| bit patterns
};
static_assert(offsetof(DeviceState, partial) % 16 == 0, "partials must be 16-byte aligned");

// Launchers (enqueue only; return the HIP launch error).
hipError_t launch_init_state(DeviceState* st, int history_len, const float static_eff[3], hipStream_t s);
hipError_t launch_quantize_dynamic(DeviceState* st, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   int64_t n, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s);
hipError_t launch_quantize_static(DeviceState* st, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  int64_t n, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s);
hipError_t launch_quantize_packed(DeviceState* st, bool dynamic, const uint16_t* qkv, int64_t total_tokens,
                                  int num_heads, int head_dim, uint8_t* q8, uint8_t* k8, uint8_t* v8, hipStream_t s);
// q8, k8, v8: [total_tokens, num_heads, 128] codes, zero past head_dim;
// out: [total_tokens, num_heads, head_dim] bf16.
hipError_t launch_attention(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                            const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads, int head_dim,
                            void* out, hipStream_t s);
// The same with S = K Q^T on the fp8 MFMA for head dims above 64 (the
// exact kernel up to 64).
hipError_t launch_attention_fp8qk(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                                  const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads,
                                  int head_dim, void* out, hipStream_t s);
// Split-key variant: num_splits key ranges per (head, query tile), partial
// results in `workspace` (attention_workspace_bytes), merged by a second
// kernel; num_splits <= 1 is launch_attention.
size_t attention_workspace_bytes(int num_seqs, int total_tokens, int num_heads, int num_splits);
// The library's own split workspace on the current device (a file-scope
// device array of kAttnScratchBytes; its address is looked up once per
// device).  No allocation.
constexpr size_t kAttnScratchBytes = (size_t)36 << 20;
hipError_t attention_scratch(void** ptr);
hipError_t launch_attention_split(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                                  const int32_t* cu_seqlens, int num_seqs, int total_tokens, int num_heads,
                                  int head_dim, int num_splits, void* workspace, void* out, hipStream_t s);
hipError_t launch_attention_bf16(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                 int num_seqs, int total_tokens, int num_heads, void* out, hipStream_t s);

}  // namespace qfa
