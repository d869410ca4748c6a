/*
 * qfa.h -- C ABI of the MI355X (gfx950) FP8 varlen ViT-attention library.
 *
 * The library implements one path: per-tensor amax of bf16 Q, K, V feeding a
 * 16-entry circular buffer of observed amax values per tensor (dynamic
 * scaling) or loaded amax values times a margin (static scaling); saturating
 * bf16 -> OCP E4M3 quantization of Q, K, V; and non-causal flash attention
 * over packed variable-length sequences on the E4M3 codes with bf16 output.
 *
 * Sources (web pages, cited by title and section):
 *   [P2] "FP8 ViT Encoder Attention" (vLLM documentation)
 *   [P4] "FP8 vision encoder attention" (Sonar documentation)
 *
 * Conventions for every entry point:
 *   - Tensors are contiguous, token-major [total_tokens, num_heads, head_dim];
 *     head_dim is 128, except where an entry point says otherwise (the
 *     packed quantize path and the FP8 attention take head dims 8..128 in
 *     steps of 8 on codes zero-padded to 128).  Q, K and V share num_heads
 *     and cu_seqlens.
 *   - Device pointers must be 16-byte aligned.  The caller owns all device
 *     memory; the library never allocates device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Kernels are enqueued on it; hot-path entry points never synchronise.
 *   - Every argument is validated on the host before any HIP call, so a
 *     non-OK status means nothing was enqueued.  A HIP launch error, or an
 *     asynchronous error left by earlier work, is returned as QFA_ERR_HIP.
 *     qfa_last_error() gives a thread-local message for the last failure.
 *   - Device data is trusted: cu_seqlens contents must satisfy the rules of
 *     qfa_fp8_varlen_attn (check with qfa_check_cu_seqlens when unsure).
 */
#ifndef QFA_H
#define QFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qfa_status {
    QFA_OK = 0,
    QFA_ERR_NULL = 1,        /* a required pointer is NULL */
    QFA_ERR_SHAPE = 2,       /* negative/zero/overflowing sizes, bad num_seqs */
    QFA_ERR_UNSUPPORTED = 3, /* head_dim not accepted by the entry point */
    QFA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
    QFA_ERR_MODE = 5,        /* mode is neither QFA_DYNAMIC nor QFA_STATIC */
    QFA_ERR_NO_STATIC = 6,   /* QFA_STATIC on a state initialised without static amax */
    QFA_ERR_VALUE = 7,       /* history_len not in 1..16; static amax, margin or their product not finite and > 0 */
    QFA_ERR_STATE = 8,       /* the handle was not initialised by qfa_init_scale_state */
    QFA_ERR_HIP = 9,         /* a HIP runtime error */
    QFA_ERR_DATA = 10,       /* qfa_check_cu_seqlens found invalid cu_seqlens contents */
    QFA_ERR_WORKSPACE = 11   /* a split launch's workspace is missing or smaller than it needs */
} qfa_status;

typedef enum qfa_mode {
    QFA_DYNAMIC = 0, /* observe amax, push it into the ring, scale from the ring maximum */
    QFA_STATIC = 1   /* scale from the loaded amax times margin; no amax pass */
} qfa_mode;

#define QFA_HEAD_DIM 128
#define QFA_MAX_HISTORY 16
#define QFA_MAX_SPLITS 16   /* key ranges per query tile in qfa_fp8_varlen_attn_split */
#define QFA_NOALLOC_SCRATCH_BYTES ((size_t)36 << 20) /* workspace of qfa_fp8_varlen_attn_split_noalloc */

/*
 * Host handle of one attention layer's scale state.  Filled by
 * qfa_init_scale_state; the caller keeps it (by value or pointer) next to
 * the device buffer it names.  Fields are read-only for the caller.
 */
typedef struct qfa_scale_state {
    uint32_t magic;          /* QFA_STATE_MAGIC once initialised */
    int32_t history_len;     /* ring length, 1..16 ([P2] Usage uses 16) */
    int32_t has_static;      /* 1 if static amax values were given */
    float static_amax[3];    /* loaded amax of Q, K, V (amax domain) */
    float margin;            /* static multiplier ([P2] Calibrate-Once: default 1.5) */
    void* device;            /* caller-owned device buffer, qfa_scale_state_bytes() bytes */
} qfa_scale_state;

#define QFA_STATE_MAGIC 0x31414651u /* "QFA1" */

/*
 * Host copy of the device-resident scale state (qfa_read_scale_state).
 * Tensor index t: 0 = Q, 1 = K, 2 = V.
 */
typedef struct qfa_scale_snapshot {
    float ring[3][QFA_MAX_HISTORY]; /* observed amax values; unused slots are 0 */
    float amax_observed[3];         /* amax seen by the last dynamic forward */
    float amax_eff[3];              /* effective amax of the last forward */
    float descale[3];               /* s_t = fp32(max(amax_eff, 2^-100) / 448) */
    float inv[3];                   /* fp32(448 / max(amax_eff, 2^-100)) */
    int32_t cursor;                 /* dynamic forwards so far */
    int32_t history_len;
    int32_t requantized[3];         /* 1 if the last dynamic forward quantized tensor t a second time */
} qfa_scale_snapshot;

/* Bytes of device memory a scale state needs (a few KiB). */
size_t qfa_scale_state_bytes(void);

/*
 * Initialise a scale state ([P2] Usage: dynamic scaling from a 16-entry
 * circular buffer of observed amax values; [P2] Calibrate-Once, Reuse
 * Workflow and [P4] Create static scales: loaded scales times a save margin,
 * default 1.5).
 *   st           host handle to fill (out)
 *   device_buf   device buffer of qfa_scale_state_bytes() bytes, 16-B aligned
 *   history_len  ring length, 1..16 (16 for the pages' behaviour)
 *   static_amax  host float[3] amax values of Q, K, V for static mode, or NULL
 *                (then QFA_STATIC is refused with QFA_ERR_NO_STATIC)
 *   margin       static multiplier, finite and > 0 (1.5 is the pages' default;
 *                pass 1.0 for values that already include the margin);
 *                ignored when static_amax is NULL
 * Enqueues one small kernel that zeroes the ring and cursor and stores the
 * static effective amax fp32(static_amax * margin).  Re-initialising a state
 * resets it.
 */
qfa_status qfa_init_scale_state(qfa_scale_state* st, void* device_buf, int history_len,
                                const float* static_amax, float margin, void* stream);

/*
 * One forward of the quantizer ([P2] intro: Q/K/V quantized on the fly to FP8
 * before the attention call).
 *   QFA_DYNAMIC: amax_t = max|x| over tensor t; ring[t][cursor % history_len]
 *     = amax_t; cursor += 1; amax_eff[t] = max(ring[t][:]).
 *   QFA_STATIC:  amax_eff[t] = fp32(static_amax[t] * margin); ring untouched.
 *   Both: a = max(amax_eff, 2^-100); descale = fp32(a / 448); inv =
 *     fp32(448 / a); code = E4M3(fp32(x * inv[t])) rounded to nearest even,
 *     saturated to +-448, sign of zero kept.
 *   q, k, v      device bf16 [total_tokens, num_heads, head_dim]
 *   q8, k8, v8   device uint8 E4M3 codes, same shape (out)
 * Dynamic mode reads each tensor once when amax_t does not exceed the ring
 * maximum over the slots other than the one being replaced: it quantizes with
 * that maximum's scale while taking amax_t, and the result is then exactly the
 * one defined above.  Otherwise (the first forwards, or a new maximum over the
 * window) it quantizes tensor t a second time with the new scale;
 * qfa_scale_snapshot.requantized[t] says which happened.
 * total_tokens may be 0 (the forward still records amax 0 in dynamic mode).
 * Forwards on one state must be ordered on one stream (single-writer ring);
 * distinct states are independent.
 */
qfa_status qfa_quantize_qkv(const qfa_scale_state* st, int mode, const void* q, const void* k,
                            const void* v, int64_t total_tokens, int num_heads, int head_dim,
                            uint8_t* q8, uint8_t* k8, uint8_t* v8, void* stream);

/*
 * One forward of the quantizer straight from a fused QKV projection output
 * ([P2] Performance counts the three quantization launches and the head-dim
 * un-padding among the overheads of small images): same scale-state rules
 * as qfa_quantize_qkv, with
 *   qkv          device bf16 [total_tokens, 3, num_heads, head_dim]
 *                (Q = qkv[:, 0], K = qkv[:, 1], V = qkv[:, 2])
 *   head_dim     8..128 in steps of 8 (e.g. 80 or 72 for ViT encoders
 *                whose hidden size is not 128 * num_heads)
 *   q8, k8, v8   device uint8 E4M3 codes [total_tokens, num_heads, 128]
 *                (out): dims [0, head_dim) are the codes, dims past it 0 --
 *                the layout qfa_fp8_varlen_attn reads for any head_dim
 * amax is taken over the head_dim real dims only.  Two launches (dynamic)
 * or one (static).  total_tokens * num_heads * 16 must be below 2^31.
 */
qfa_status qfa_quantize_qkv_packed(const qfa_scale_state* st, int mode, const void* qkv, int64_t total_tokens,
                                   int num_heads, int head_dim, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                                   void* stream);

/* Device pointer to float[3] {s_q, s_k, s_v} inside the state (valid after a forward). */
const float* qfa_descale_ptr(const qfa_scale_state* st);

/*
 * Varlen FP8 attention with per-tensor scales ([P4] Requirements: a
 * per-tensor FP8 varlen attention over packed variable-length image batches).
 *   out[i,h,:] = sum_j softmax_j(s_q*s_k*<q_i,k_j>/sqrt(head_dim)) * s_v * v_j
 * over the keys j of the sequence that contains token i, non-causal.
 *   q8, k8, v8     device E4M3 codes [total_tokens, num_heads, 128]; for
 *                  head_dim < 128 the dims past head_dim must hold code 0
 *                  (as qfa_quantize_qkv_packed writes them)
 *   scales         device float[3] {s_q, s_k, s_v} (e.g. qfa_descale_ptr)
 *   cu_seqlens     device int32[num_seqs + 1]: cu[0] = 0, non-decreasing,
 *                  cu[num_seqs] = total_tokens; empty sequences are allowed
 *   head_dim       8..128 in steps of 8 (128 for qfa_quantize_qkv's codes)
 *   out            device bf16 [total_tokens, num_heads, head_dim] (out)
 * total_tokens must be below 2^31, num_seqs at most 2^30 and num_heads at
 * most 65536, and (total_tokens / 256 + num_seqs) * num_heads workgroups
 * must fit an int (QFA_ERR_SHAPE otherwise).  The kernel converts the codes exactly to
 * fp16 and runs both products on fp16 MFMAs with float32 accumulation; the
 * probabilities are rounded to fp16 for the P*V product.
 */
qfa_status qfa_fp8_varlen_attn(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                               const float* scales, const int32_t* cu_seqlens, int num_seqs,
                               int64_t total_tokens, int num_heads, int head_dim, void* out,
                               void* stream);

/*
 * The same attention with S = Q K^T on the fp8 matrix cores, like the
 * per-tensor FP8 attention kernel that [P4] Requirements names for
 * gfx942/gfx950, for inputs known to hold no isolated large elements.
 * Arguments, layouts, limits and errors as qfa_fp8_varlen_attn.  For
 * head_dim above 64, S is taken by v_mfma_f32_16x16x128_f8f6f4 on the codes
 * themselves: no conversion of K and half the matrix cycles of S.  That
 * instruction truncates every product in a group of 8 consecutive dims to a
 * multiple of 2^(E - 13), E the exponent of the group's largest product, so
 * a product of two outliers (say 20x the typical magnitude) wipes out the
 * low bits of its 7 neighbours: the result can then miss the tolerance
 * qfa_fp8_varlen_attn holds.  On Gaussian Q and K without outliers it stays
 * as accurate as qfa_fp8_varlen_attn.  The error grows with the logits'
 * scale times the outliers' size: in an emulation of the instruction,
 * Gaussian Q and K of standard deviation 1 keep 0.1 % of elements 20x larger
 * inside the tolerance, standard deviation 3 does not keep 10x ones.  For
 * head_dim <= 64 it runs
 * qfa_fp8_varlen_attn's kernel (exact products).
 */
qfa_status qfa_fp8_varlen_attn_fp8qk(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                     const float* scales, const int32_t* cu_seqlens, int num_seqs,
                                     int64_t total_tokens, int num_heads, int head_dim, void* out,
                                     void* stream);

/*
 * The same attention with the keys of each (head, 256-query tile) split into
 * up to QFA_MAX_SPLITS ranges of whole 128-key tiles, one workgroup per
 * range, for launches that would leave compute units idle (small images:
 * "FP8 ViT Encoder Attention", Performance, finds no FP8 gain there; "FP8
 * vision encoder attention", Expected performance, measures 2304 tokens).
 * Each range writes, per query, its partial output normalised by its own
 * softmax sum (fp16, in code units) plus its running max and sum (float32)
 * to `workspace`; a second kernel merges the ranges with the usual
 * max-shifted weights and writes `out`.  Arguments as qfa_fp8_varlen_attn,
 * plus:
 *   num_splits       0 = qfa_fp8_varlen_attn_auto_splits(...), else 1..16;
 *                    1 runs qfa_fp8_varlen_attn (no workspace used).
 *                    Ranges past a sequence's last key tile are empty.
 *   workspace        caller-owned device memory, 16-byte aligned, of at least
 *                    qfa_fp8_varlen_attn_workspace_bytes(...) bytes; may be
 *                    NULL when the split count resolves to 1.  Its contents
 *                    on entry do not matter and are garbage on return.
 *   workspace_bytes  its size (QFA_ERR_WORKSPACE if too small or missing)
 * QFA_ERR_VALUE for num_splits outside 0..16; QFA_ERR_SHAPE when the
 * workgroups times the ranges, or 16 merge workgroups per query tile, exceed
 * an int.  Calls sharing one workspace must be ordered on one stream.
 */
qfa_status qfa_fp8_varlen_attn_split(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                     const float* scales, const int32_t* cu_seqlens, int num_seqs,
                                     int64_t total_tokens, int num_heads, int head_dim, int num_splits,
                                     void* workspace, size_t workspace_bytes, void* out, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP-graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * qfa_fp8_varlen_attn_split with the library's own workspace instead of a
 * caller-owned one.  That workspace is a fixed device array of
 * QFA_NOALLOC_SCRATCH_BYTES (36 MiB) that each GPU the library runs on holds
 * until the process ends; it covers every split count the automatic rule
 * (num_splits = 0) picks.  A request needing more (an explicit num_splits on
 * a large launch) returns QFA_ERR_WORKSPACE before anything is enqueued.
 * The call enqueues kernels only: no hipMalloc, hipFree or other allocating
 * routine; the array's address on the current device (which must be the
 * stream's) is looked up once per device.  All calls on one GPU share that
 * GPU's array, which keeps the last call's contents: calls that overlap on
 * one GPU (other streams, other threads) race and must be ordered by the
 * caller.  Nothing in the array needs to start at zero.  Other arguments and
 * results as qfa_fp8_varlen_attn_split.
 */
qfa_status qfa_fp8_varlen_attn_split_noalloc(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                             const float* scales, const int32_t* cu_seqlens, int num_seqs,
                                             int64_t total_tokens, int num_heads, int head_dim, int num_splits,
                                             void* out, void* stream);

/*
 * Split count qfa_fp8_varlen_attn_split uses for num_splits = 0: as many
 * ranges as keep every workgroup of the launch in one round of the 256
 * compute units (256-query tiles x heads x ranges <= 256), each of at least
 * two 128-key tiles of a sequence of the batch's mean length, at most 16; 1
 * when that is fewer than two.  (A second round of workgroups costs about
 * what the split saves.)  Host-only, no device access; 1 for sizes the attention
 * entry points refuse.
 */
int qfa_fp8_varlen_attn_auto_splits(int num_seqs, int64_t total_tokens, int num_heads);

/*
 * Workspace bytes qfa_fp8_varlen_attn_split needs for num_splits (0 = the
 * automatic count): for S > 1 ranges, S * num_heads * (total_tokens / 256 +
 * num_seqs) * 256 query rows of 128 fp16 plus 2 float32, rounded up; 0 when
 * the count resolves to 1 or an argument is out of range.  Host-only.
 */
size_t qfa_fp8_varlen_attn_workspace_bytes(int num_seqs, int64_t total_tokens, int num_heads, int num_splits);

/*
 * Varlen BF16 attention, the baseline FP8 attention is compared against
 * ([P2] Performance and [P4] Expected performance give every FP8 result as
 * a BF16 -> FP8 pair on the same shapes).
 *   out[i,h,:] = sum_j softmax_j(<q_i,k_j>/sqrt(128)) * v_j
 * over the keys j of the sequence that contains token i, non-causal.
 *   q, k, v        device bf16 [total_tokens, num_heads, 128]
 *   cu_seqlens     device int32[num_seqs + 1], same rules as qfa_fp8_varlen_attn
 *   out            device bf16 [total_tokens, num_heads, 128] (out)
 * Size limits as qfa_fp8_varlen_attn.  Products
 * and sums run in fp32 on bf16
 * MFMA operands; the probabilities are rounded to bf16 for the P*V product.
 * Same status codes as qfa_fp8_varlen_attn.
 */
qfa_status qfa_bf16_varlen_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                int num_seqs, int64_t total_tokens, int num_heads, int head_dim, void* out,
                                void* stream);

/*
 * Debug/checkpoint helpers (synchronise `stream`; not for the hot path).
 * qfa_read_scale_state copies the device state to *out.
 * qfa_check_cu_seqlens reads cu_seqlens back and returns QFA_ERR_DATA unless
 * cu[0] = 0, cu is non-decreasing and cu[num_seqs] = total_tokens.
 */
qfa_status qfa_read_scale_state(const qfa_scale_state* st, qfa_scale_snapshot* out, void* stream);
qfa_status qfa_check_cu_seqlens(const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens,
                                void* stream);

/*
 * Calibrate-once export ([P2] Calibrate-Once, Reuse Workflow; [P4] Create
 * static scales): after dynamic forwards on representative inputs, the scale
 * each tensor learned, with the save margin applied for a scale file:
 *   out_amax[t] = fp32(max(ring[t][0..history_len)) * margin),  t = Q, K, V.
 * The result is an amax-domain value; a state initialised from it with
 * margin 1.0 reproduces fp32(ring max * margin) exactly.
 *   margin    finite and > 0 (1.5 is the pages' default save margin)
 *   out_amax  host float[3] (out); written only on QFA_OK
 * Synchronises `stream` (reads the device state).  QFA_ERR_STATE if the state
 * is not initialised or has seen no dynamic forward; QFA_ERR_VALUE if margin
 * is invalid, a tensor observed only zeros, or a product overflows float32.
 */
qfa_status qfa_export_static_amax(const qfa_scale_state* st, float margin, float* out_amax, void* stream);

/* Static text for a status; thread-local detail of the last failure on this thread. */
const char* qfa_status_string(qfa_status s);
const char* qfa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QFA_H */
