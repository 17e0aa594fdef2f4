// codec.hip -- weight packing (RTN) and per-token int8 activation quantization for gfx950.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化", [Orin] "Jetson Orin AGX INT4 推理优化实践：super
// 分支从 9 tok/s 到 24 tok/s", [Infra] "【infra之路】12-投机解码、量化与推理引擎对比".
//
// Both kernels produce integers and bit patterns, so every fp32 step is one IEEE operation in a
// fixed order (correctly rounded division, round-to-nearest-even, no contraction).
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

// One wavefront per (output row, group).  [Lab5 INT4 线性量化]:
//   SYM : s = bf16(max|r|/7), z = 8;  ASYM: s = bf16((max-min)/15), z = bf16(rint(-min/s))
//   code = clamp(rint(r/s + z), 0, 15), stored two per byte with the earlier column low.
// The group's statistics include its padded columns (value 0), so pads encode to z.
template <int MODE>
__global__ void __launch_bounds__(256) pack_kernel(const float *__restrict__ w, int64_t d_out,
                                                   int64_t d_in, int64_t ldw, int64_t span,
                                                   int64_t n_groups, int64_t k_pad,
                                                   uint8_t *__restrict__ qweight,
                                                   uint16_t *__restrict__ scales,
                                                   uint16_t *__restrict__ zeros) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (item >= d_out * n_groups) return;  // uniform across the wave
    const int64_t j = item / n_groups;
    const int64_t G = item - j * n_groups;
    const int64_t k0 = G * span;
    const float *wr = w + j * ldw;

    // max|r|, max r, min r over the padded group: exact, so the reduction order is irrelevant.
    float amax = 0.0f, mx = -INFINITY, mn = INFINITY;
    for (int64_t t = lane; t < span; t += kWave) {
        const int64_t k = k0 + t;
        const float r = k < d_in ? wr[k] : 0.0f;
        amax = fmaxf(amax, fabsf(r));
        mx = fmaxf(mx, r);
        mn = fminf(mn, r);
    }
    amax = wave_max(amax);
    mx = wave_max(mx);
    mn = wave_min(mn);

    float s32;
    if (MODE == 0) {
        s32 = amax / 7.0f;
    } else {
        const float range = mx - mn;
        s32 = range / 15.0f;
    }
    s32 = s32 + 0.0f;  // a zero scale is stored as +0
    const uint32_t s_bits = f32_to_bf16(s32);
    const float s = bf16_to_f32(s_bits);
    float zf = 8.0f;
    if (MODE == 1) {
        if (s != 0.0f) {
            const float neg_mn = -mn;
            const float ratio = neg_mn / s;
            zf = __builtin_rintf(ratio);
            zf = zf + 0.0f;  // a zero point of -0 is stored as +0
        } else {
            zf = 0.0f;
        }
        const uint32_t z_bits = f32_to_bf16(zf);
        zf = bf16_to_f32(z_bits);
        if (lane == 0) zeros[j * n_groups + G] = static_cast<uint16_t>(z_bits);
    }
    if (lane == 0) scales[j * n_groups + G] = static_cast<uint16_t>(s_bits);

    uint8_t *out = qweight + j * (k_pad / 2) + k0 / 2;
    for (int64_t p = lane; p < span / 2; p += kWave) {
        uint32_t code[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t k = k0 + 2 * p + e;
            const float r = k < d_in ? wr[k] : 0.0f;
            if (s == 0.0f) {
                code[e] = static_cast<uint32_t>(zf);
            } else {
                float v = r / s;
                v = v + zf;
                v = __builtin_rintf(v);
                v = fmaxf(v, 0.0f);
                v = fminf(v, 15.0f);
                code[e] = static_cast<uint32_t>(v);
            }
        }
        out[p] = static_cast<uint8_t>(code[0] | (code[1] << 4));
    }
}

// One workgroup of 256 threads per token row.  [Orin 从 FP 线性层到 INT4 DP4A 的数学推导],
// [Infra 2.2 量化的基本概念]:  s = max|x|/127,  q = clamp(rint(x/s), -127, 127).
__global__ void __launch_bounds__(256) act_quant_kernel(const uint16_t *__restrict__ x,
                                                        int64_t K, int64_t ldx,
                                                        int8_t *__restrict__ q, int64_t ldq,
                                                        float *__restrict__ s_x,
                                                        int32_t *__restrict__ q_sum) {
#pragma clang fp contract(off)
    __shared__ float red_f[256 / kWave];
    __shared__ int red_i[256 / kWave];
    const int64_t m = blockIdx.x;
    const uint16_t *xr = x + m * ldx;
    const int tid = threadIdx.x, wid = tid / kWave, lane = tid & (kWave - 1);

    float a = 0.0f;
    for (int64_t k = tid; k < K; k += 256) a = fmaxf(a, fabsf(bf16_to_f32(xr[k])));
    a = wave_max(a);
    if (lane == 0) red_f[wid] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));

    const float s = a / 127.0f;
    int sum = 0;
    int8_t *qr = q + m * ldq;
    for (int64_t k = tid; k < K; k += 256) {
        int qi = 0;
        if (a != 0.0f) {
            float v = bf16_to_f32(xr[k]) / s;
            v = __builtin_rintf(v);
            v = fmaxf(v, -127.0f);
            v = fminf(v, 127.0f);
            qi = static_cast<int>(v);
        }
        qr[k] = static_cast<int8_t>(qi);
        sum += qi;
    }
    sum = wave_sum(sum);
    if (lane == 0) red_i[wid] = sum;
    __syncthreads();
    if (tid == 0) {
        s_x[m] = s;
        if (q_sum) q_sum[m] = red_i[0] + red_i[1] + red_i[2] + red_i[3];
    }
}

hipError_t launch_pack(const float *w, int64_t d_out, int64_t d_in, int64_t ldw, int64_t span,
                       int64_t n_groups, int64_t k_pad, int mode, uint8_t *qweight,
                       uint16_t *scales, uint16_t *zeros, hipStream_t stream) {
    const int64_t items = d_out * n_groups;
    const int waves_per_block = 4;
    const dim3 grid(static_cast<unsigned>((items + waves_per_block - 1) / waves_per_block));
    if (mode == 0)
        hipLaunchKernelGGL(pack_kernel<0>, grid, dim3(256), 0, stream, w, d_out, d_in, ldw, span,
                           n_groups, k_pad, qweight, scales, zeros);
    else
        hipLaunchKernelGGL(pack_kernel<1>, grid, dim3(256), 0, stream, w, d_out, d_in, ldw, span,
                           n_groups, k_pad, qweight, scales, zeros);
    return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                            int64_t ldq, float *s_x, int32_t *q_sum, hipStream_t stream) {
    hipLaunchKernelGGL(act_quant_kernel, dim3(static_cast<unsigned>(M)), dim3(256), 0, stream, x,
                       K, ldx, q, ldq, s_x, q_sum);
    return hipGetLastError();
}

}  // namespace w4
