// Hardware probe for the GPU tests (test infrastructure, not part of libqfa):
// one 64-lane wave runs ONE matrix instruction on operand register images the
// caller supplies, so a test can pin how gfx950 sums the products of each
// instruction kind the attention kernel could use.
//
//   kind 0  v_mfma_f32_16x16x128_f8f6f4, E4M3 x E4M3 (A, B: 32 bytes per lane)
//   kind 1  v_mfma_f32_16x16x32_fp8_fp8             (A, B: 8 bytes per lane)
//   kind 2  v_mfma_f32_16x16x32_f16                 (A, B: 16 bytes per lane)
//   kind 3  v_mfma_f32_16x16x32_bf16                (A, B: 16 bytes per lane)
//
// Buffers (device, caller-owned): a, b = 64 lanes x 32 bytes (lane l's
// register image at byte 32 l; only the first 8 or 16 bytes are read for
// kinds 1-3); c, d = 64 lanes x 4 floats (accumulator in / result out, lane
// l's four accumulator registers at float 4 l).  Every access is inside these
// sizes: one workgroup of exactly 64 threads, thread l touching only its own
// slot.
#include <hip/hip_runtime.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void mfma_probe_kernel(int kind, const unsigned char* a, const unsigned char* b,
                                                        const float* c, float* d) {
    const int l = threadIdx.x;
    const v4f acc = *(const v4f*)(c + 4 * l);
    v4f r = acc;
    if (kind == 0) {
        const v8i x = *(const v8i*)(a + 32 * l), y = *(const v8i*)(b + 32 * l);
        r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, acc, 0, 0, 0, 0, 0, 0);
    } else if (kind == 1) {
        const long x = *(const long*)(a + 32 * l), y = *(const long*)(b + 32 * l);
        r = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(x, y, acc, 0, 0, 0);
    } else if (kind == 2) {
        const f16x8 x = *(const f16x8*)(a + 32 * l), y = *(const f16x8*)(b + 32 * l);
        r = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, acc, 0, 0, 0);
    } else if (kind == 3) {
        const bf16x8 x = *(const bf16x8*)(a + 32 * l), y = *(const bf16x8*)(b + 32 * l);
        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc, 0, 0, 0);
    }
    *(v4f*)(d + 4 * l) = r;
}

extern "C" int mfma_probe(int kind, const void* a, const void* b, const float* c, float* d, void* stream) {
    if (kind < 0 || kind > 3 || !a || !b || !c || !d) return 1;
    mfma_probe_kernel<<<1, 64, 0, (hipStream_t)stream>>>(kind, (const unsigned char*)a, (const unsigned char*)b, c, d);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
