// dsa_device.h -- device-side helpers shared by the gfx950 kernels of libdsa_amd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Order-preserving map of a float onto an unsigned key: larger float -> larger key.
__device__ __forceinline__ uint32_t float_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16x16x128 FP8 (OCP e4m3fn) matrix-core product, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, 32 bytes each; the four
// lane groups (l / 16) cover disjoint quarters of K.  Output lane l holds rows
// 4 * (l / 16) + i, i = 0..3, of column l % 16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 matrix-core product: lane l supplies 8 K-values of row/column l % 16
// (lane group l / 16 selects the K slice); output layout as above.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

}  // namespace dsa
