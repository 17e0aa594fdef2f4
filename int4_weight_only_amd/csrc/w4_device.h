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

// Wave-wide sums through DPP row shifts and row broadcasts (gfx9 wave64): after the four
// row_shr steps lane 15 of each 16-lane row holds the row's sum; row_bcast:15 and row_bcast:31
// fold the rows together, leaving the total in lane 63, which is read back as a uniform value.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, BOUND);
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += __int_as_float(dpp_i<0x111, 0xF, true>(__float_as_int(v)));
    v += __int_as_float(dpp_i<0x112, 0xF, true>(__float_as_int(v)));
    v += __int_as_float(dpp_i<0x114, 0xF, true>(__float_as_int(v)));
    v += __int_as_float(dpp_i<0x118, 0xF, true>(__float_as_int(v)));
    v += __int_as_float(dpp_i<0x142, 0xA, false>(__float_as_int(v)));
    v += __int_as_float(dpp_i<0x143, 0xC, false>(__float_as_int(v)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_dpp(int v) {
    v += dpp_i<0x111, 0xF, true>(v);
    v += dpp_i<0x112, 0xF, true>(v);
    v += dpp_i<0x114, 0xF, true>(v);
    v += dpp_i<0x118, 0xF, true>(v);
    v += dpp_i<0x142, 0xA, false>(v);
    v += dpp_i<0x143, 0xC, false>(v);
    return __builtin_amdgcn_readlane(v, 63);
}

// (a & m) | o in one VALU instruction; the constants sit in VGPRs (a gfx9 VOP3 instruction reads
// at most one scalar operand, so the compiler would otherwise split it in two).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
    return r;
}

// Pins the order of the phases around it: no instruction is scheduled across it, and no memory
// access is moved across it. The vector-memory counter is in order, so a load sunk towards its
// use would sit behind later loads, and waiting for it would wait for them too.
__device__ __forceinline__ void phase_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Raw (untyped, stride 0) buffer descriptors: dword 3 = 0x00020000 selects the 32-bit data
// format the gfx9 family uses for raw buffers. An offset at or past num_records is out of range:
// the load returns 0 and issues no memory request, the store is dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;  // above every num_records used here (< 2^31)
constexpr int kNonTemporal = 2;                 // cache policy bit of a streamed read

// Every descriptor here is built from wave-uniform values; readfirstlane states that, so the
// descriptor lives in scalar registers (a descriptor the compiler thinks divergent would be
// applied lane by lane in a loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    void *p = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(
        p, 0, static_cast<int>(__builtin_amdgcn_readfirstlane(bytes)), kRawBufferWord3);
}

// Store one output element, as fp32 or as the round-to-nearest-even bf16 image of the fp32 value.
__device__ __forceinline__ void store_out(void *y, int64_t idx, float v, bool out_f32) {
    if (out_f32)
        static_cast<float *>(y)[idx] = v;
    else
        static_cast<uint16_t *>(y)[idx] = static_cast<uint16_t>(f32_to_bf16(v));
}

}  // namespace w4
