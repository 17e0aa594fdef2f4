// w4_quant.h -- the per-token int8 activation quantization rule, shared by every kernel that
// quantizes activations (act_quant_int8 and the W4A8 linear that folds it into its prologue), so
// that their codes agree bit for bit.
#pragma once

#include "w4_device.h"

namespace w4 {

// The token scale: s = max|x| / 127, correctly rounded ([Orin 从 FP 线性层到 INT4 DP4A 的数学推导],
// [Infra 2.2 量化的基本概念]).
__device__ __forceinline__ float token_scale_int8(float absmax) {
#pragma clang fp contract(off)
    return absmax / 127.0f;
}

// The code of one activation: clamp(rint(x / s), -127, 127), with one correctly rounded fp32
// division. (A token whose maximum is 0 takes code 0 everywhere; callers apply that.)
__device__ __forceinline__ int quantize_int8(float x, float s) {
#pragma clang fp contract(off)
    float t = x / s;
    t = __builtin_rintf(t);
    t = fmaxf(t, -127.0f);
    t = fminf(t, 127.0f);
    return static_cast<int>(t);
}

// The same code without a division per element. With r = RN(1/s) (the caller computes it once
// per token) and q0 = RN(x r), for |x| <= max|x| (so |x / s| <= 127 (1 + 2^-24)):
//   |q0 - x/s| <= |x/s| (2^-24 + 2^-24 + 2^-48) < 2^-16, and |RN(x/s) - x/s| <= 2^-18,
// so |q0 - RN(x/s)| < 2^-15. If q0 lies more than 2^-14 from every half-integer, no rounding
// boundary (k + 1/2) lies between q0 and RN(x/s), and rint of either is the same integer; in the
// band around a half-integer, and when r is not a normal number (max|x| below about 2^-119), the
// correctly rounded division decides. The codes are those of quantize_int8 for every input.
__device__ __forceinline__ int quantize_int8_fast(float x, float s, float r) {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float k = __builtin_rintf(q0);
    const float d = fabsf(q0 - k);  // exact: q0 and its nearest integer are within 1/2
    float t = k;
    if (__builtin_expect(0.5f - d <= 0x1.0p-14f || !(fabsf(r) < 0x1.0p126f), 0))
        t = __builtin_rintf(x / s);
    t = fmaxf(t, -127.0f);
    t = fminf(t, 127.0f);
    return static_cast<int>(t);
}

// The fast path of quantize_int8_fast alone, for callers that take the fallback for a whole block
// of values: the clamped code rint(x r), and `slow` set if x r lies in the band around a
// half-integer where that code may differ from quantize_int8's (the caller then recomputes the
// block with quantize_int8).
__device__ __forceinline__ float quantize_int8_band(float x, float r, bool &slow) {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float k = __builtin_rintf(q0);
    slow |= 0.5f - fabsf(q0 - k) <= 0x1.0p-14f;
    return fminf(fmaxf(k, -127.0f), 127.0f);
}

}  // namespace w4
