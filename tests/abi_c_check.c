/* A plain C99 caller of the C ABI in include/qfa.h: it must compile with a C
 * compiler, link against libqfa.so and get the documented statuses from the
 * argument checks, which return before any HIP call (no GPU needed). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qfa.h"

static int failures = 0;

static void expect(const char* what, qfa_status got, qfa_status want) {
    if (got != want) {
        printf("FAIL %s: got %d (%s), want %d (%s); last error: %s\n", what, (int)got, qfa_status_string(got),
               (int)want, qfa_status_string(want), qfa_last_error());
        ++failures;
    }
}

int main(void) {
    qfa_scale_state st;
    float amax[3] = {1.0f, 2.0f, 3.0f};
    float bad[3] = {1.0f, -2.0f, 3.0f};
    int32_t cu[2] = {0, 4};
    /* 16-byte aligned fake device addresses: never dereferenced, the calls fail validation first */
    void* dev = (void*)(uintptr_t)0x100000;
    void* misaligned = (void*)(uintptr_t)0x100004;

    memset(&st, 0, sizeof st);
    if (qfa_scale_state_bytes() < 64) { printf("FAIL state bytes %zu\n", qfa_scale_state_bytes()); ++failures; }
    if (strcmp(qfa_status_string(QFA_OK), "ok") != 0) { printf("FAIL status string\n"); ++failures; }

    expect("init: null handle", qfa_init_scale_state(NULL, dev, 16, NULL, 1.5f, NULL), QFA_ERR_NULL);
    expect("init: null buffer", qfa_init_scale_state(&st, NULL, 16, NULL, 1.5f, NULL), QFA_ERR_NULL);
    expect("init: misaligned", qfa_init_scale_state(&st, misaligned, 16, NULL, 1.5f, NULL), QFA_ERR_ALIGN);
    expect("init: history 0", qfa_init_scale_state(&st, dev, 0, NULL, 1.5f, NULL), QFA_ERR_VALUE);
    expect("init: history 17", qfa_init_scale_state(&st, dev, 17, NULL, 1.5f, NULL), QFA_ERR_VALUE);
    expect("init: negative amax", qfa_init_scale_state(&st, dev, 16, bad, 1.5f, NULL), QFA_ERR_VALUE);
    expect("init: zero margin", qfa_init_scale_state(&st, dev, 16, amax, 0.0f, NULL), QFA_ERR_VALUE);
    if (qfa_last_error()[0] == '\0') { printf("FAIL empty last error\n"); ++failures; }

    expect("quantize: uninitialised state",
           qfa_quantize_qkv(&st, QFA_DYNAMIC, dev, dev, dev, 4, 1, 128, dev, dev, dev, NULL), QFA_ERR_STATE);
    expect("attention: head_dim 130",
           qfa_fp8_varlen_attn(dev, dev, dev, (const float*)dev, cu, 1, 4, 1, 130, dev, NULL), QFA_ERR_UNSUPPORTED);
    expect("attention: no sequences",
           qfa_fp8_varlen_attn(dev, dev, dev, (const float*)dev, cu, 0, 4, 1, 128, dev, NULL), QFA_ERR_SHAPE);
    expect("attention: too many heads",
           qfa_fp8_varlen_attn(dev, dev, dev, (const float*)dev, cu, 1, 4, 65537, 128, dev, NULL), QFA_ERR_SHAPE);
    expect("attention: misaligned output",
           qfa_fp8_varlen_attn(dev, dev, dev, (const float*)dev, cu, 1, 4, 1, 128, misaligned, NULL), QFA_ERR_ALIGN);
    expect("fp8 QK^T attention: head_dim 130",
           qfa_fp8_varlen_attn_fp8qk(dev, dev, dev, (const float*)dev, cu, 1, 4, 1, 130, dev, NULL),
           QFA_ERR_UNSUPPORTED);
    expect("bf16 attention: head_dim 64",
           qfa_bf16_varlen_attn(dev, dev, dev, cu, 1, 4, 1, 64, dev, NULL), QFA_ERR_UNSUPPORTED);
    expect("export: null output", qfa_export_static_amax(&st, 1.5f, NULL, NULL), QFA_ERR_NULL);
    if (qfa_descale_ptr(&st) != NULL) { printf("FAIL descale pointer of an uninitialised state\n"); ++failures; }
    expect("split: num_splits 17",
           qfa_fp8_varlen_attn_split(dev, dev, dev, (const float*)dev, cu, 1, 300, 2, 128, 17, dev, (size_t)1 << 30,
                                     dev, NULL), QFA_ERR_VALUE);
    expect("split: no workspace",
           qfa_fp8_varlen_attn_split(dev, dev, dev, (const float*)dev, cu, 1, 300, 2, 128, 4, NULL, 0, dev, NULL),
           QFA_ERR_WORKSPACE);
    if (qfa_fp8_varlen_attn_auto_splits(1, 8192, 16) != 1) { printf("FAIL auto splits of a full launch\n"); ++failures; }
    if (qfa_fp8_varlen_attn_workspace_bytes(1, 2304, 8, 0) == 0) { printf("FAIL workspace bytes\n"); ++failures; }

    if (failures == 0) printf("C ABI checks ok\n");
    return failures == 0 ? 0 : 1;
}
