/* Argument sweep of the C ABI in include/qfa.h, for a build of the library
 * whose host code runs under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_abi_sanitized.py builds both and runs this program).
 *
 * Every entry point is called with edge values (null, misaligned and aligned
 * placeholder pointers; zero, negative, boundary and overflowing sizes;
 * non-finite floats) and with seeded random combinations of them.  The
 * placeholder addresses are never valid device memory, so the program runs
 * only where the HIP runtime sees no GPU: a call that passes the argument
 * checks then fails at its first HIP call (QFA_ERR_HIP) instead of touching
 * memory.  With a GPU present it prints a line and exits without calling
 * anything.
 *
 * Checked for every call: the status is one of the declared codes, a failure
 * leaves a non-empty, terminated qfa_last_error() text, and nothing succeeds
 * that would have had to enqueue work (nothing can, without a device).  The
 * sanitizers abort the process on any out-of-bounds access, use of freed
 * memory, signed overflow, invalid shift or other undefined behaviour in the
 * checks themselves. */
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "qfa.h"

static int failures = 0;
static long calls = 0;

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
/* splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", 2014) */
static uint64_t next_u64(void) {
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static uint64_t pick(uint64_t n) { return next_u64() % n; }

#define N_OF(a) (sizeof(a) / sizeof((a)[0]))

static void* const kPtrs[] = {NULL, (void*)(uintptr_t)0x100000, (void*)(uintptr_t)0x100004,
                              (void*)(uintptr_t)0x100002, (void*)(uintptr_t)0x100010};
static const int kInts[] = {INT_MIN, -65536, -1, 0, 1, 2, 3, 7, 8, 15, 16, 17, 31, 32, 64, 72, 80, 96, 120, 128,
                            129, 136, 255, 256, 257, 65535, 65536, 65537, 1 << 20, 1 << 30, INT_MAX - 1, INT_MAX};
static const int64_t kI64[] = {INT64_MIN, -1, 0, 1, 17, 255, 256, 257, 2304, 8192, 99504, (INT64_C(1) << 31) - 1,
                               INT64_C(1) << 31, INT64_C(1) << 40, INT64_MAX};
static const float kFloats[] = {0.0f, -0.0f, 1.0f, 1.5f, -1.5f, 448.0f, FLT_MIN, 1e-45f, FLT_MAX, INFINITY,
                                -INFINITY, NAN};

/* length of s, looking at most at cap bytes */
static size_t bounded_len(const char* s, size_t cap) {
    size_t n = 0;
    while (n < cap && s[n] != '\0') ++n;
    return n;
}

static void* any_ptr(void) { return kPtrs[pick(N_OF(kPtrs))]; }
static int any_int(void) {
    switch (pick(3)) {
        case 0: return kInts[pick(N_OF(kInts))];
        case 1: return (int)pick(300) - 20;
        default: return (int)(uint32_t)next_u64();
    }
}
static int64_t any_i64(void) {
    switch (pick(3)) {
        case 0: return kI64[pick(N_OF(kI64))];
        case 1: return (int64_t)pick(100000) - 10;
        default: return (int64_t)next_u64();
    }
}
static float any_float(void) { return kFloats[pick(N_OF(kFloats))]; }
static size_t any_size(void) {
    static const size_t sizes[] = {0, 1, 255, 256, (size_t)1 << 20, (size_t)36 << 20, (size_t)1 << 40, SIZE_MAX};
    return sizes[pick(N_OF(sizes))];
}

static void check(const char* what, qfa_status s) {
    ++calls;
    if ((int)s < (int)QFA_OK || (int)s > (int)QFA_ERR_WORKSPACE) {
        printf("FAIL %s: undeclared status %d\n", what, (int)s);
        ++failures;
        return;
    }
    if (strcmp(qfa_status_string(s), "unknown status") == 0) {
        printf("FAIL %s: status %d has no text\n", what, (int)s);
        ++failures;
    }
    if (s != QFA_OK) {
        const char* e = qfa_last_error();
        const size_t n = bounded_len(e, 4096);
        if (n == 0 || n >= 512) {
            printf("FAIL %s: status %d with last error of length %zu\n", what, (int)s, n);
            ++failures;
        }
    }
}

/* A call that enqueues work cannot succeed without a device. */
static void check_not_ok(const char* what, qfa_status s) {
    check(what, s);
    if (s == QFA_OK) {
        printf("FAIL %s: succeeded without a device\n", what);
        ++failures;
    }
}

static void fake_state(qfa_scale_state* st, int initialised) {
    memset(st, 0, sizeof *st);
    if (pick(2) || initialised) {
        st->magic = QFA_STATE_MAGIC;
        st->history_len = 1 + (int)pick(16);
        st->has_static = (int)pick(2);
        for (int t = 0; t < 3; ++t) st->static_amax[t] = 1.0f + (float)t;
        st->margin = 1.5f;
        st->device = pick(4) ? (void*)(uintptr_t)0x100000 : NULL;
    }
}

static void sweep_once(void) {
    qfa_scale_state st;
    float amax[3], out3[3];
    qfa_scale_snapshot snap;
    for (int t = 0; t < 3; ++t) amax[t] = any_float();
    fake_state(&st, 0);
    const void* q = any_ptr();
    void* o = any_ptr();
    switch (pick(14)) {
        case 0:
            check_not_ok("init", qfa_init_scale_state(pick(4) ? &st : NULL, any_ptr(), any_int(),
                                                     pick(2) ? amax : NULL, any_float(), NULL));
            break;
        case 1:
            check("quantize", qfa_quantize_qkv(pick(8) ? &st : NULL, any_int() & (pick(2) ? 1 : -1), q, any_ptr(),
                                               any_ptr(), any_i64(), any_int(), any_int(), (uint8_t*)o,
                                               (uint8_t*)any_ptr(), (uint8_t*)any_ptr(), NULL));
            break;
        case 2:
            check("quantize packed", qfa_quantize_qkv_packed(pick(8) ? &st : NULL, (int)pick(3) - 1, q, any_i64(),
                                                             any_int(), any_int(), (uint8_t*)o, (uint8_t*)any_ptr(),
                                                             (uint8_t*)any_ptr(), NULL));
            break;
        case 3: {
            /* the exact attention and the fp8 Q K^T one share their arguments */
            const int fp8qk = (int)pick(2);
            const qfa_status r = (fp8qk ? qfa_fp8_varlen_attn_fp8qk : qfa_fp8_varlen_attn)(
                (const uint8_t*)q, (const uint8_t*)any_ptr(), (const uint8_t*)any_ptr(), (const float*)any_ptr(),
                (const int32_t*)any_ptr(), any_int(), any_i64(), any_int(), any_int(), o, NULL);
            check(fp8qk ? "fp8 Q K^T attention" : "attention", r);
            break;
        }
        case 4:
            check("split attention",
                  qfa_fp8_varlen_attn_split((const uint8_t*)q, (const uint8_t*)any_ptr(), (const uint8_t*)any_ptr(),
                                            (const float*)any_ptr(), (const int32_t*)any_ptr(), any_int(), any_i64(),
                                            any_int(), any_int(), (int)pick(20) - 2, any_ptr(), any_size(), o, NULL));
            break;
        case 5:
            check("split attention, no allocation",
                  qfa_fp8_varlen_attn_split_noalloc((const uint8_t*)q, (const uint8_t*)any_ptr(),
                                                    (const uint8_t*)any_ptr(), (const float*)any_ptr(),
                                                    (const int32_t*)any_ptr(), any_int(), any_i64(), any_int(),
                                                    any_int(), (int)pick(20) - 2, o, NULL));
            break;
        case 6:
            check("bf16 attention", qfa_bf16_varlen_attn(q, any_ptr(), any_ptr(), (const int32_t*)any_ptr(),
                                                         any_int(), any_i64(), any_int(), any_int(), o, NULL));
            break;
        case 7: {
            const int sp = qfa_fp8_varlen_attn_auto_splits(any_int(), any_i64(), any_int());
            ++calls;
            if (sp < 1 || sp > QFA_MAX_SPLITS) {
                printf("FAIL auto splits %d\n", sp);
                ++failures;
            }
            break;
        }
        case 8: {
            const int nseq = any_int(), heads = any_int(), splits = (int)pick(20) - 2;
            const int64_t tokens = any_i64();
            const size_t a = qfa_fp8_varlen_attn_workspace_bytes(nseq, tokens, heads, splits);
            const size_t b = qfa_fp8_varlen_attn_workspace_bytes(nseq, tokens, heads, splits);
            ++calls;
            if (a != b || (splits == 1 && a != 0) || ((splits < 0 || splits > QFA_MAX_SPLITS) && a != 0)) {
                printf("FAIL workspace bytes %zu / %zu for %d ranges\n", a, b, splits);
                ++failures;
            }
            break;
        }
        case 9:
            check_not_ok("check cu_seqlens",
                         qfa_check_cu_seqlens((const int32_t*)any_ptr(), any_int(), any_i64(), NULL));
            break;
        case 10:
            check_not_ok("read state", qfa_read_scale_state(pick(8) ? &st : NULL, pick(8) ? &snap : NULL, NULL));
            break;
        case 11:
            check_not_ok("export", qfa_export_static_amax(pick(8) ? &st : NULL, any_float(), pick(8) ? out3 : NULL,
                                                          NULL));
            break;
        case 12: {
            const char* text = qfa_status_string((qfa_status)any_int());
            ++calls;
            if (!text || bounded_len(text, 64) == 0) {
                printf("FAIL status text\n");
                ++failures;
            }
            break;
        }
        default: {
            const float* d = qfa_descale_ptr(pick(8) ? &st : NULL);
            ++calls;
            if (d && (st.magic != QFA_STATE_MAGIC || !st.device)) {
                printf("FAIL descale pointer of an uninitialised state\n");
                ++failures;
            }
            break;
        }
    }
}

/* Deterministic edges that random draws reach rarely. */
static void edges(void) {
    void* dev = (void*)(uintptr_t)0x100000;
    const int32_t* cu = (const int32_t*)dev;
    const float* sc = (const float*)dev;
    const uint8_t* c8 = (const uint8_t*)dev;
    qfa_scale_state st;
    fake_state(&st, 1);
    for (size_t i = 0; i < N_OF(kInts); ++i)
        for (size_t j = 0; j < N_OF(kI64); ++j)
            for (size_t k = 0; k < N_OF(kInts); k += 3) {
                const int nseq = kInts[i], heads = kInts[k];
                const int64_t tokens = kI64[j];
                check("edge attention", qfa_fp8_varlen_attn(c8, c8, c8, sc, cu, nseq, tokens, heads, 128, dev, NULL));
                check("edge fp8 Q K^T attention",
                      qfa_fp8_varlen_attn_fp8qk(c8, c8, c8, sc, cu, nseq, tokens, heads, 96, dev, NULL));
                check("edge split", qfa_fp8_varlen_attn_split(c8, c8, c8, sc, cu, nseq, tokens, heads, 80, 0, dev,
                                                              SIZE_MAX, dev, NULL));
                check("edge split, no allocation",
                      qfa_fp8_varlen_attn_split_noalloc(c8, c8, c8, sc, cu, nseq, tokens, heads, 128, 16, dev, NULL));
                check("edge bf16", qfa_bf16_varlen_attn(dev, dev, dev, cu, nseq, tokens, heads, 128, dev, NULL));
                check("edge quantize", qfa_quantize_qkv(&st, QFA_DYNAMIC, dev, dev, dev, tokens, heads, 128,
                                                        (uint8_t*)dev, (uint8_t*)dev, (uint8_t*)dev, NULL));
                check("edge quantize packed", qfa_quantize_qkv_packed(&st, QFA_DYNAMIC, dev, tokens, heads, 72,
                                                                      (uint8_t*)dev, (uint8_t*)dev, (uint8_t*)dev,
                                                                      NULL));
                for (int sp = 0; sp <= QFA_MAX_SPLITS + 1; sp += 4)
                    (void)qfa_fp8_varlen_attn_workspace_bytes(nseq, tokens, heads, sp);
                (void)qfa_fp8_varlen_attn_auto_splits(nseq, tokens, heads);
                calls += 2;
            }
    /* a long text in the error buffer, then a short one: the buffer stays terminated */
    check("long error", qfa_fp8_varlen_attn(c8, c8, c8, sc, cu, INT_MAX, INT64_MAX, INT_MAX, 130, dev, NULL));
    check("short error", qfa_init_scale_state(NULL, NULL, 0, NULL, 0.0f, NULL));
}

int main(void) {
    int devices = 0;
    if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
        printf("a GPU is present: the sweep passes placeholder addresses, so it runs only without one\n");
        return 0;
    }
    edges();
    for (int i = 0; i < 200000; ++i) sweep_once();
    if (failures) {
        printf("%d failures in %ld calls\n", failures, calls);
        return 1;
    }
    printf("ABI sweep ok: %ld calls\n", calls);
    return 0;
}
