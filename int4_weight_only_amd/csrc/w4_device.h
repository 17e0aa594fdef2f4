// w4_device.h -- device helpers shared by the gfx950 kernels of libw4.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Store one output element, as fp32 or as the round-to-nearest-even bf16 image of the fp32 value.
__device__ __forceinline__ void store_out(void *y, int64_t idx, float v, bool out_f32) {
    if (out_f32)
        static_cast<float *>(y)[idx] = v;
    else
        static_cast<uint16_t *>(y)[idx] = static_cast<uint16_t>(f32_to_bf16(v));
}

}  // namespace w4
