// C ABI of the library: argument validation (before any HIP call), status
// codes, thread-local error text, and dispatch to the kernel launchers.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "qfa_internal.h"

namespace {

thread_local char g_last_error[512] = "";

qfa_status fail(qfa_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

qfa_status ok() {
    g_last_error[0] = '\0';
    return QFA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Surface an asynchronous error left by earlier work on this thread's device
// before enqueuing more.
qfa_status check_pending(const char* where) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(QFA_ERR_HIP, "%s: pending HIP error: %s", where, hipGetErrorString(e));
    return QFA_OK;
}

qfa_status check_launch(hipError_t e, const char* where) {
    if (e != hipSuccess) return fail(QFA_ERR_HIP, "%s: HIP error: %s", where, hipGetErrorString(e));
    return ok();
}

// Shared checks of a [T, H, D] tensor triple.  Returns elements per tensor.
qfa_status check_shape(int64_t total_tokens, int num_heads, int head_dim, int64_t* elems, const char* where) {
    if (head_dim != QFA_HEAD_DIM) return fail(QFA_ERR_UNSUPPORTED, "%s: head_dim %d (only 128 is supported)", where, head_dim);
    if (num_heads <= 0) return fail(QFA_ERR_SHAPE, "%s: num_heads %d must be positive", where, num_heads);
    if (total_tokens < 0) return fail(QFA_ERR_SHAPE, "%s: total_tokens %lld is negative", where, (long long)total_tokens);
    // elements per tensor must fit comfortably in int64 byte offsets
    if (total_tokens > (INT64_C(1) << 40) / ((int64_t)num_heads * head_dim))
        return fail(QFA_ERR_SHAPE, "%s: tensor too large", where);
    *elems = total_tokens * num_heads * head_dim;
    return QFA_OK;
}

// The attention kernels fetch up to 128 token rows of one head through a
// buffer descriptor whose 32-bit range spans those rows at a stride of
// num_heads * 256 bytes (bf16); 65536 heads keep it below 2^31.
constexpr int kMaxAttnHeads = 65536;

// Sequences per launch: at most 2^30, so that the virtual query tiles of one
// head (total_tokens / 256 + num_seqs, total_tokens < 2^31) fit an int.
constexpr int kMaxSeqs = 1 << 30;

// The attention grids: (total_tokens / 256 + num_seqs) query tiles per head
// times num_heads workgroups, times the key ranges of a split launch, whose
// merge adds 16 workgroups per query tile; each must fit an int.
qfa_status check_attn_grid(int num_seqs, int64_t total_tokens, int num_heads, int splits, const char* where) {
    const int64_t tiles = (total_tokens / 256 + num_seqs) * (int64_t)num_heads;
    const int64_t limit = INT64_C(0x7FFFFFFF);
    if (tiles * std::max(splits, 1) > limit || (splits > 1 && tiles * 16 > limit))
        return fail(QFA_ERR_SHAPE, "%s: %lld query tiles x %d key ranges exceed the grid limit", where,
                    (long long)tiles, splits);
    return QFA_OK;
}

// Head dims the padded paths accept: 8..128 in steps of 8 (16-byte bf16 rows).
bool padded_head_dim_ok(int head_dim) { return head_dim >= 8 && head_dim <= QFA_HEAD_DIM && head_dim % 8 == 0; }

}  // namespace

extern "C" {

static_assert(qfa::kAttnScratchBytes == QFA_NOALLOC_SCRATCH_BYTES, "scratch size and its public constant");

size_t qfa_scale_state_bytes(void) { return sizeof(qfa::DeviceState); }

const char* qfa_status_string(qfa_status s) {
    // A C caller may pass any int; reading it as the C++ enum would be
    // undefined outside the declared codes, so take its bits as an int.
    static_assert(sizeof(qfa_status) == sizeof(int), "qfa_status is an int-sized enum");
    int code;
    memcpy(&code, &s, sizeof code);
    switch (code) {
        case QFA_OK: return "ok";
        case QFA_ERR_NULL: return "null pointer";
        case QFA_ERR_SHAPE: return "invalid shape";
        case QFA_ERR_UNSUPPORTED: return "unsupported head_dim";
        case QFA_ERR_ALIGN: return "device pointer not 16-byte aligned";
        case QFA_ERR_MODE: return "invalid mode";
        case QFA_ERR_NO_STATIC: return "static mode without static amax";
        case QFA_ERR_VALUE: return "invalid value";
        case QFA_ERR_STATE: return "scale state not initialised";
        case QFA_ERR_HIP: return "HIP runtime error";
        case QFA_ERR_DATA: return "invalid cu_seqlens contents";
        case QFA_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

const char* qfa_last_error(void) { return g_last_error; }

qfa_status qfa_init_scale_state(qfa_scale_state* st, void* device_buf, int history_len, const float* static_amax,
                                float margin, void* stream) {
    const char* where = "qfa_init_scale_state";
    if (!st || !device_buf) return fail(QFA_ERR_NULL, "%s: null handle or device buffer", where);
    if (!aligned16(device_buf)) return fail(QFA_ERR_ALIGN, "%s: device buffer not 16-byte aligned", where);
    if (history_len < 1 || history_len > QFA_MAX_HISTORY)
        return fail(QFA_ERR_VALUE, "%s: history_len %d not in 1..16", where, history_len);
    float eff[3] = {0.0f, 0.0f, 0.0f};
    if (static_amax) {
        if (!std::isfinite(margin) || !(margin > 0.0f))
            return fail(QFA_ERR_VALUE, "%s: margin must be finite and positive", where);
        for (int t = 0; t < 3; ++t) {
            if (!std::isfinite(static_amax[t]) || !(static_amax[t] > 0.0f))
                return fail(QFA_ERR_VALUE, "%s: static amax[%d] must be finite and positive", where, t);
            volatile float prod = static_amax[t] * margin;  // one float32 multiply, as on the device
            eff[t] = prod;
            if (!std::isfinite(eff[t]))
                return fail(QFA_ERR_VALUE, "%s: static amax[%d] * margin overflows float32", where, t);
        }
    }
    qfa_status ps = check_pending(where);
    if (ps != QFA_OK) return ps;
    const hipError_t e = qfa::launch_init_state((qfa::DeviceState*)device_buf, history_len, eff, (hipStream_t)stream);
    if (e != hipSuccess) return check_launch(e, where);
    st->magic = QFA_STATE_MAGIC;
    st->history_len = history_len;
    st->has_static = static_amax ? 1 : 0;
    for (int t = 0; t < 3; ++t) st->static_amax[t] = static_amax ? static_amax[t] : 0.0f;
    st->margin = static_amax ? margin : 1.0f;
    st->device = device_buf;
    return ok();
}

qfa_status qfa_quantize_qkv(const qfa_scale_state* st, int mode, const void* q, const void* k, const void* v,
                            int64_t total_tokens, int num_heads, int head_dim, uint8_t* q8, uint8_t* k8,
                            uint8_t* v8, void* stream) {
    const char* where = "qfa_quantize_qkv";
    if (!st) return fail(QFA_ERR_NULL, "%s: null state handle", where);
    if (st->magic != QFA_STATE_MAGIC || !st->device) return fail(QFA_ERR_STATE, "%s: state not initialised", where);
    if (mode != QFA_DYNAMIC && mode != QFA_STATIC) return fail(QFA_ERR_MODE, "%s: mode %d", where, mode);
    if (mode == QFA_STATIC && !st->has_static)
        return fail(QFA_ERR_NO_STATIC, "%s: state was initialised without static amax", where);
    int64_t n = 0;
    qfa_status s = check_shape(total_tokens, num_heads, head_dim, &n, where);
    if (s != QFA_OK) return s;
    if (n > 0 && (!q || !k || !v || !q8 || !k8 || !v8)) return fail(QFA_ERR_NULL, "%s: null tensor pointer", where);
    if (n > 0 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(q8) && aligned16(k8) && aligned16(v8)))
        return fail(QFA_ERR_ALIGN, "%s: tensor pointer not 16-byte aligned", where);
    s = check_pending(where);
    if (s != QFA_OK) return s;
    qfa::DeviceState* ds = (qfa::DeviceState*)st->device;
    const hipError_t e =
        mode == QFA_DYNAMIC
            ? qfa::launch_quantize_dynamic(ds, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, n, q8, k8,
                                           v8, (hipStream_t)stream)
            : qfa::launch_quantize_static(ds, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, n, q8, k8,
                                          v8, (hipStream_t)stream);
    return check_launch(e, where);
}

qfa_status qfa_quantize_qkv_packed(const qfa_scale_state* st, int mode, const void* qkv, int64_t total_tokens,
                                   int num_heads, int head_dim, uint8_t* q8, uint8_t* k8, uint8_t* v8, void* stream) {
    const char* where = "qfa_quantize_qkv_packed";
    if (!st) return fail(QFA_ERR_NULL, "%s: null state handle", where);
    if (st->magic != QFA_STATE_MAGIC || !st->device) return fail(QFA_ERR_STATE, "%s: state not initialised", where);
    if (mode != QFA_DYNAMIC && mode != QFA_STATIC) return fail(QFA_ERR_MODE, "%s: mode %d", where, mode);
    if (mode == QFA_STATIC && !st->has_static)
        return fail(QFA_ERR_NO_STATIC, "%s: state was initialised without static amax", where);
    if (!padded_head_dim_ok(head_dim))
        return fail(QFA_ERR_UNSUPPORTED, "%s: head_dim %d (8..128 in steps of 8)", where, head_dim);
    if (num_heads <= 0) return fail(QFA_ERR_SHAPE, "%s: num_heads %d must be positive", where, num_heads);
    if (total_tokens < 0) return fail(QFA_ERR_SHAPE, "%s: total_tokens %lld is negative", where, (long long)total_tokens);
    // 8-code output chunks are indexed in 32 bits
    if (total_tokens > (INT64_C(1) << 31) / ((int64_t)num_heads * 16) - 1)
        return fail(QFA_ERR_SHAPE, "%s: tensor too large", where);
    const bool any = total_tokens > 0;
    if (any && (!qkv || !q8 || !k8 || !v8)) return fail(QFA_ERR_NULL, "%s: null tensor pointer", where);
    if (any && !(aligned16(qkv) && aligned16(q8) && aligned16(k8) && aligned16(v8)))
        return fail(QFA_ERR_ALIGN, "%s: tensor pointer not 16-byte aligned", where);
    qfa_status s = check_pending(where);
    if (s != QFA_OK) return s;
    const hipError_t e = qfa::launch_quantize_packed((qfa::DeviceState*)st->device, mode == QFA_DYNAMIC,
                                                     (const uint16_t*)qkv, total_tokens, num_heads, head_dim, q8, k8,
                                                     v8, (hipStream_t)stream);
    return check_launch(e, where);
}

const float* qfa_descale_ptr(const qfa_scale_state* st) {
    if (!st || st->magic != QFA_STATE_MAGIC || !st->device) return nullptr;
    return ((const qfa::DeviceState*)st->device)->descale;
}

}  // extern "C"

namespace {

// Checks shared by the FP8 attention entry points; *n = code elements per tensor.
qfa_status check_fp8_attn(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                          const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_heads, int head_dim,
                          const void* out, int64_t* n, const char* where) {
    if (!padded_head_dim_ok(head_dim))
        return fail(QFA_ERR_UNSUPPORTED, "%s: head_dim %d (8..128 in steps of 8)", where, head_dim);
    qfa_status s = check_shape(total_tokens, num_heads, QFA_HEAD_DIM, n, where);  // code rows are 128 wide
    if (s != QFA_OK) return s;
    if (num_seqs < 1 || num_seqs > kMaxSeqs)
        return fail(QFA_ERR_SHAPE, "%s: num_seqs %d not in 1..2^30", where, num_seqs);
    if (total_tokens >= (INT64_C(1) << 31)) return fail(QFA_ERR_SHAPE, "%s: total_tokens must be below 2^31", where);
    if (num_heads > kMaxAttnHeads)
        return fail(QFA_ERR_SHAPE, "%s: num_heads %d above %d", where, num_heads, kMaxAttnHeads);
    if (!scales || !cu_seqlens) return fail(QFA_ERR_NULL, "%s: null scales or cu_seqlens", where);
    if (*n > 0 && (!q8 || !k8 || !v8 || !out)) return fail(QFA_ERR_NULL, "%s: null tensor pointer", where);
    if (*n > 0 && !(aligned16(q8) && aligned16(k8) && aligned16(v8) && aligned16(out)))
        return fail(QFA_ERR_ALIGN, "%s: tensor pointer not 16-byte aligned", where);
    if (((uintptr_t)scales & 3u) || ((uintptr_t)cu_seqlens & 3u))
        return fail(QFA_ERR_ALIGN, "%s: scales / cu_seqlens not 4-byte aligned", where);
    return QFA_OK;
}

// Key-range splits for a launch that fills few CUs.  Measured on one
// MI355X with one workgroup per CU: a workgroup streaming n key tiles takes
// about 2.9 n + 9.6 us when every workgroup of the launch fits in one round
// of the 256 CUs, and a second round costs about as much as the split saves.
// So the keys are split into as many ranges as still fit in one round, each
// of at least two 128-key tiles of a sequence of the batch's mean length (the
// split only matters for small batches, whose images are of similar size),
// at most QFA_MAX_SPLITS; 1 when that is fewer than two ranges.
int auto_splits(int num_seqs, int64_t total_tokens, int num_heads) {
    // sizes the attention entry points refuse get 1 (and no overflow below)
    if (total_tokens <= 0 || total_tokens >= (INT64_C(1) << 31) || num_seqs < 1 || num_seqs > kMaxSeqs ||
        num_heads < 1)
        return 1;
    const int64_t query_tiles = ((total_tokens + 255) / 256 + (num_seqs - 1)) * num_heads;
    const int64_t mean_len = (total_tokens + num_seqs - 1) / num_seqs;
    const int64_t nt = (mean_len + 127) / 128;
    int64_t sp = std::min<int64_t>(256 / query_tiles, nt / 2);
    sp = std::min<int64_t>(sp, QFA_MAX_SPLITS);
    return sp >= 2 ? (int)sp : 1;
}

}  // namespace

extern "C" {

int qfa_fp8_varlen_attn_auto_splits(int num_seqs, int64_t total_tokens, int num_heads) {
    return auto_splits(num_seqs, total_tokens, num_heads);
}

size_t qfa_fp8_varlen_attn_workspace_bytes(int num_seqs, int64_t total_tokens, int num_heads, int num_splits) {
    if (num_seqs < 1 || num_seqs > kMaxSeqs || num_heads < 1 || num_heads > kMaxAttnHeads || total_tokens < 0 ||
        total_tokens >= (INT64_C(1) << 31))
        return 0;
    if (num_splits < 0 || num_splits > QFA_MAX_SPLITS) return 0;
    const int sp = num_splits == 0 ? auto_splits(num_seqs, total_tokens, num_heads) : num_splits;
    return qfa::attention_workspace_bytes(num_seqs, (int)total_tokens, num_heads, sp);
}

qfa_status qfa_fp8_varlen_attn_split(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                                     const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_heads,
                                     int head_dim, int num_splits, void* workspace, size_t workspace_bytes,
                                     void* out, void* stream) {
    const char* where = "qfa_fp8_varlen_attn_split";
    int64_t n = 0;
    qfa_status s = check_fp8_attn(q8, k8, v8, scales, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim, out,
                                  &n, where);
    if (s != QFA_OK) return s;
    if (num_splits < 0 || num_splits > QFA_MAX_SPLITS)
        return fail(QFA_ERR_VALUE, "%s: num_splits %d not in 0..%d", where, num_splits, QFA_MAX_SPLITS);
    const int sp = num_splits == 0 ? auto_splits(num_seqs, total_tokens, num_heads) : num_splits;
    s = check_attn_grid(num_seqs, total_tokens, num_heads, sp, where);
    if (s != QFA_OK) return s;
    const size_t need = qfa::attention_workspace_bytes(num_seqs, (int)total_tokens, num_heads, sp);
    if (n > 0 && sp > 1) {
        if (!workspace) return fail(QFA_ERR_WORKSPACE, "%s: %d key ranges need a workspace", where, sp);
        if (!aligned16(workspace)) return fail(QFA_ERR_ALIGN, "%s: workspace not 16-byte aligned", where);
        if (workspace_bytes < need)
            return fail(QFA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", where, workspace_bytes, need);
    }
    s = check_pending(where);
    if (s != QFA_OK) return s;
    if (n == 0) return ok();
    const hipError_t e = qfa::launch_attention_split(q8, k8, v8, scales, cu_seqlens, num_seqs, (int)total_tokens,
                                                     num_heads, head_dim, sp, workspace, out, (hipStream_t)stream);
    return check_launch(e, where);
}

qfa_status qfa_fp8_varlen_attn_split_noalloc(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                                             const float* scales, const int32_t* cu_seqlens, int num_seqs,
                                             int64_t total_tokens, int num_heads, int head_dim, int num_splits,
                                             void* out, void* stream) {
    const char* where = "qfa_fp8_varlen_attn_split_noalloc";
    int64_t n = 0;
    qfa_status s = check_fp8_attn(q8, k8, v8, scales, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim, out,
                                  &n, where);
    if (s != QFA_OK) return s;
    if (num_splits < 0 || num_splits > QFA_MAX_SPLITS)
        return fail(QFA_ERR_VALUE, "%s: num_splits %d not in 0..%d", where, num_splits, QFA_MAX_SPLITS);
    const int sp = num_splits == 0 ? auto_splits(num_seqs, total_tokens, num_heads) : num_splits;
    s = check_attn_grid(num_seqs, total_tokens, num_heads, sp, where);
    if (s != QFA_OK) return s;
    const size_t need = qfa::attention_workspace_bytes(num_seqs, (int)total_tokens, num_heads, sp);
    if (need > QFA_NOALLOC_SCRATCH_BYTES)
        return fail(QFA_ERR_WORKSPACE, "%s: %d key ranges need %zu bytes of workspace, above the library's %zu",
                    where, sp, need, (size_t)QFA_NOALLOC_SCRATCH_BYTES);
    s = check_pending(where);
    if (s != QFA_OK) return s;
    if (n == 0) return ok();
    void* ws = nullptr;
    if (sp > 1) {
        const hipError_t e = qfa::attention_scratch(&ws);
        if (e != hipSuccess) return check_launch(e, where);
    }
    const hipError_t e = qfa::launch_attention_split(q8, k8, v8, scales, cu_seqlens, num_seqs, (int)total_tokens,
                                                     num_heads, head_dim, sp, ws, out, (hipStream_t)stream);
    return check_launch(e, where);
}

qfa_status qfa_fp8_varlen_attn(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                               const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_heads,
                               int head_dim, void* out, void* stream) {
    const char* where = "qfa_fp8_varlen_attn";
    int64_t n = 0;
    qfa_status s = check_fp8_attn(q8, k8, v8, scales, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim, out,
                                  &n, where);
    if (s != QFA_OK) return s;
    s = check_attn_grid(num_seqs, total_tokens, num_heads, 1, where);
    if (s != QFA_OK) return s;
    s = check_pending(where);
    if (s != QFA_OK) return s;
    if (n == 0) return ok();
    const hipError_t e = qfa::launch_attention(q8, k8, v8, scales, cu_seqlens, num_seqs, (int)total_tokens, num_heads,
                                               head_dim, out, (hipStream_t)stream);
    return check_launch(e, where);
}

qfa_status qfa_fp8_varlen_attn_fp8qk(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* scales,
                                     const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, int num_heads,
                                     int head_dim, void* out, void* stream) {
    const char* where = "qfa_fp8_varlen_attn_fp8qk";
    int64_t n = 0;
    qfa_status s = check_fp8_attn(q8, k8, v8, scales, cu_seqlens, num_seqs, total_tokens, num_heads, head_dim, out,
                                  &n, where);
    if (s != QFA_OK) return s;
    s = check_attn_grid(num_seqs, total_tokens, num_heads, 1, where);
    if (s != QFA_OK) return s;
    s = check_pending(where);
    if (s != QFA_OK) return s;
    if (n == 0) return ok();
    const hipError_t e = qfa::launch_attention_fp8qk(q8, k8, v8, scales, cu_seqlens, num_seqs, (int)total_tokens,
                                                     num_heads, head_dim, out, (hipStream_t)stream);
    return check_launch(e, where);
}

qfa_status qfa_bf16_varlen_attn(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int num_seqs,
                                int64_t total_tokens, int num_heads, int head_dim, void* out, void* stream) {
    const char* where = "qfa_bf16_varlen_attn";
    int64_t n = 0;
    qfa_status s = check_shape(total_tokens, num_heads, head_dim, &n, where);
    if (s != QFA_OK) return s;
    if (num_seqs < 1 || num_seqs > kMaxSeqs)
        return fail(QFA_ERR_SHAPE, "%s: num_seqs %d not in 1..2^30", where, num_seqs);
    if (total_tokens >= (INT64_C(1) << 31)) return fail(QFA_ERR_SHAPE, "%s: total_tokens must be below 2^31", where);
    if (num_heads > kMaxAttnHeads)
        return fail(QFA_ERR_SHAPE, "%s: num_heads %d above %d", where, num_heads, kMaxAttnHeads);
    s = check_attn_grid(num_seqs, total_tokens, num_heads, 1, where);
    if (s != QFA_OK) return s;
    if (!cu_seqlens) return fail(QFA_ERR_NULL, "%s: null cu_seqlens", where);
    if (n > 0 && (!q || !k || !v || !out)) return fail(QFA_ERR_NULL, "%s: null tensor pointer", where);
    if (n > 0 && !(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out)))
        return fail(QFA_ERR_ALIGN, "%s: tensor pointer not 16-byte aligned", where);
    if ((uintptr_t)cu_seqlens & 3u) return fail(QFA_ERR_ALIGN, "%s: cu_seqlens not 4-byte aligned", where);
    s = check_pending(where);
    if (s != QFA_OK) return s;
    if (n == 0) return ok();
    const hipError_t e = qfa::launch_attention_bf16(q, k, v, cu_seqlens, num_seqs, (int)total_tokens, num_heads, out,
                                                    (hipStream_t)stream);
    return check_launch(e, where);
}

qfa_status qfa_read_scale_state(const qfa_scale_state* st, qfa_scale_snapshot* out, void* stream) {
    const char* where = "qfa_read_scale_state";
    if (!st || !out) return fail(QFA_ERR_NULL, "%s: null pointer", where);
    if (st->magic != QFA_STATE_MAGIC || !st->device) return fail(QFA_ERR_STATE, "%s: state not initialised", where);
    qfa::DeviceState h;
    hipError_t e = hipMemcpyAsync(&h, st->device, offsetof(qfa::DeviceState, partial), hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return check_launch(e, where);
    memcpy(out->ring, h.ring, sizeof(out->ring));
    memcpy(out->amax_observed, h.amax_observed, sizeof(out->amax_observed));
    memcpy(out->amax_eff, h.amax_eff, sizeof(out->amax_eff));
    memcpy(out->descale, h.descale, sizeof(out->descale));
    memcpy(out->inv, h.inv, sizeof(out->inv));
    out->cursor = h.cursor;
    out->history_len = h.history_len;
    memcpy(out->requantized, h.requantized, sizeof(out->requantized));
    return ok();
}

qfa_status qfa_export_static_amax(const qfa_scale_state* st, float margin, float* out_amax, void* stream) {
    const char* where = "qfa_export_static_amax";
    if (!st || !out_amax) return fail(QFA_ERR_NULL, "%s: null pointer", where);
    if (st->magic != QFA_STATE_MAGIC || !st->device) return fail(QFA_ERR_STATE, "%s: state not initialised", where);
    if (!std::isfinite(margin) || !(margin > 0.0f)) return fail(QFA_ERR_VALUE, "%s: margin must be finite and positive", where);
    qfa::DeviceState h;
    hipError_t e = hipMemcpyAsync(&h, st->device, offsetof(qfa::DeviceState, partial), hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return check_launch(e, where);
    if (h.cursor <= 0) return fail(QFA_ERR_STATE, "%s: no dynamic forward has been observed", where);
    float res[3];
    for (int t = 0; t < 3; ++t) {
        float m = 0.0f;  // unfilled slots hold 0; amax values are never negative
        for (int j = 0; j < h.history_len; ++j) m = h.ring[t][j] > m ? h.ring[t][j] : m;
        if (!(m > 0.0f)) return fail(QFA_ERR_VALUE, "%s: tensor %d observed only zeros", where, t);
        volatile float prod = m * margin;  // one float32 multiply
        res[t] = prod;
        if (!std::isfinite(res[t])) return fail(QFA_ERR_VALUE, "%s: amax[%d] * margin overflows float32", where, t);
    }
    for (int t = 0; t < 3; ++t) out_amax[t] = res[t];
    return ok();
}

qfa_status qfa_check_cu_seqlens(const int32_t* cu_seqlens, int num_seqs, int64_t total_tokens, void* stream) {
    const char* where = "qfa_check_cu_seqlens";
    if (!cu_seqlens) return fail(QFA_ERR_NULL, "%s: null cu_seqlens", where);
    if (num_seqs < 1 || num_seqs > kMaxSeqs)
        return fail(QFA_ERR_SHAPE, "%s: num_seqs %d not in 1..2^30", where, num_seqs);
    if (total_tokens < 0 || total_tokens >= (INT64_C(1) << 31)) return fail(QFA_ERR_SHAPE, "%s: total_tokens out of range", where);
    int32_t* h = (int32_t*)malloc(sizeof(int32_t) * ((size_t)num_seqs + 1));
    if (!h) return fail(QFA_ERR_SHAPE, "%s: host allocation failed", where);
    hipError_t e = hipMemcpyAsync(h, cu_seqlens, sizeof(int32_t) * ((size_t)num_seqs + 1), hipMemcpyDeviceToHost,
                                  (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) {
        free(h);
        return check_launch(e, where);
    }
    qfa_status s = QFA_OK;
    if (h[0] != 0) s = fail(QFA_ERR_DATA, "%s: cu_seqlens[0] = %d, expected 0", where, h[0]);
    for (int b = 0; s == QFA_OK && b < num_seqs; ++b)
        if (h[b + 1] < h[b]) s = fail(QFA_ERR_DATA, "%s: cu_seqlens decreases at %d", where, b);
    if (s == QFA_OK && h[num_seqs] != total_tokens)
        s = fail(QFA_ERR_DATA, "%s: cu_seqlens[%d] = %d, expected %lld", where, num_seqs, h[num_seqs],
                 (long long)total_tokens);
    free(h);
    return s == QFA_OK ? ok() : s;
}

}  // extern "C"
