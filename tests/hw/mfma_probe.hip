// Hardware probes (test and measurement infrastructure, not part of libqfa):
// mfma_probe: one 64-lane wave runs ONE matrix instruction on operand
// register images the caller supplies, so a test can pin how gfx950 sums the
// products of each instruction kind the attention kernel could use;
// mfma_burn (at the end): the sustained matrix throughput of the whole chip.
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

// Sustained matrix throughput: 2 workgroups of 4 waves per CU (two waves per
// SIMD), each wave issuing 4 independent chains of one instruction kind for
// `rounds` rounds, with random mantissas (exponents fixed, so every value
// stays finite) re-drawn every round so that the multipliers see changing
// data.  Lane 0 of each workgroup writes its s_memtime ticks (the shader
// clock) to cycles[block]; out[block * 256 + thread] receives a sum of the
// accumulators (keeps the work alive).  kind: 0 = v_mfma_f32_16x16x32_f16,
// 1 = v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3), 2 = v_mfma_f32_16x16x32_bf16.
template <int kKind>
__global__ __launch_bounds__(256) void mfma_burn_kernel(float* out, unsigned long long* cycles, int rounds) {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    typedef unsigned u8 __attribute__((ext_vector_type(8)));
    const unsigned lane = threadIdx.x & 63;
    u4 aw, bw;
    u8 a8, b8;
    for (int i = 0; i < 4; ++i) {
        aw[i] = 0x3C003C00u ^ ((lane * 2654435761u + i * 40503u) & 0x03FF03FFu);
        bw[i] = 0x3C003C00u ^ ((lane * 2246822519u + i * 3266489917u) & 0x03FF03FFu);
    }
    for (int i = 0; i < 8; ++i) {
        a8[i] = 0x38383838u ^ ((lane * 2654435761u + i * 40503u) & 0x07070707u);
        b8[i] = 0x38383838u ^ ((lane * 2246822519u + i * 668265263u) & 0x07070707u);
    }
    v4f acc[4] = {};
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (kKind == 0)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, aw), __builtin_bit_cast(f16x8, bw),
                                                                acc[i], 0, 0, 0);
            else if constexpr (kKind == 1)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    __builtin_bit_cast(v8i, a8), __builtin_bit_cast(v8i, b8), acc[i], 0, 0, 0, 127, 0, 127);
            else
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aw),
                                                                 __builtin_bit_cast(bf16x8, bw), acc[i], 0, 0, 0);
        }
        const unsigned m = (unsigned)r * 2654435761u;
        if constexpr (kKind == 1) {
            a8 ^= m & 0x07070707u;
            b8 ^= (m >> 3) & 0x07070707u;
        } else {
            aw ^= m & 0x03FF03FFu;
            bw ^= (m >> 5) & 0x03FF03FFu;
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    out[blockIdx.x * 256 + threadIdx.x] = acc[0][0] + acc[1][1] + acc[2][2] + acc[3][3];
    if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
}

// out: grid * 256 floats, cycles: grid entries (device, caller-owned).
extern "C" int mfma_burn(int kind, int grid, int rounds, float* out, unsigned long long* cycles, void* stream) {
    if (kind < 0 || kind > 2 || grid <= 0 || rounds <= 0 || !out || !cycles) return 1;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0) mfma_burn_kernel<0><<<grid, 256, 0, s>>>(out, cycles, rounds);
    else if (kind == 1) mfma_burn_kernel<1><<<grid, 256, 0, s>>>(out, cycles, rounds);
    else mfma_burn_kernel<2><<<grid, 256, 0, s>>>(out, cycles, rounds);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
