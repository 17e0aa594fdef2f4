// codec.hip -- weight packing (RTN) and per-token int8 activation quantization for gfx950.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化", [Orin] "Jetson Orin AGX INT4 推理优化实践：super
// 分支从 9 tok/s 到 24 tok/s", [Infra] "【infra之路】12-投机解码、量化与推理引擎对比".
//
// Both kernels produce integers and bit patterns, so every fp32 step is one IEEE operation in a
// fixed order (correctly rounded division, round-to-nearest-even, no contraction).
#include "w4_device.h"
#include "w4_quant.h"
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

// One workgroup of T threads per token row.  [Orin 从 FP 线性层到 INT4 DP4A 的数学推导],
// [Infra 2.2 量化的基本概念]:  s = max|x|/127,  q = clamp(rint(x/s), -127, 127).
// A thread owns the 8-column chunks tid, tid + T, ...; the first kAqCache of them stay in
// registers between the max pass and the quantization pass, so a row of up to T * kAqCache * 8
// columns is read from memory once.  Rows of up to 8192 columns run 256 threads caching 4 chunks
// (more workgroups in flight per CU, and most threads hold work), as do rows of up to 20480
// columns caching 10 when there are many rows; other rows run 1024 threads caching 4 (and
// re-reading what does not fit).  Loads are 16 bytes (ldx % 8 == 0 keeps
// every chunk that starts before K inside the row); columns >= K are masked.

__device__ __forceinline__ float chunk_absmax(const uint4 &v, int64_t col, int64_t K) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (u[e >> 1] >> 16) : (u[e >> 1] & 0xFFFFu);
        const float f = col + e < K ? fabsf(bf16_to_f32(bits)) : 0.0f;
        a = fmaxf(a, f);
    }
    return a;
}

// Quantizes the chunk at `col` and stores the codes of its columns < K; returns their sum.
__device__ __forceinline__ int chunk_quantize(const uint4 &v, int64_t col, int64_t K, float a,
                                              float s, float r, int8_t *__restrict__ qr) {
#pragma clang fp contract(off)
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    int qi[8];
    int sum = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (u[e >> 1] >> 16) : (u[e >> 1] & 0xFFFFu);
        const int t = quantize_int8_fast(bf16_to_f32(bits), s, r);
        qi[e] = (a != 0.0f && col + e < K) ? t : 0;
        sum += qi[e];
    }
    if (col + 8 <= K) {
        uint2 packed;
        packed.x = (qi[0] & 0xFF) | ((qi[1] & 0xFF) << 8) | ((qi[2] & 0xFF) << 16) |
                   (static_cast<uint32_t>(qi[3] & 0xFF) << 24);
        packed.y = (qi[4] & 0xFF) | ((qi[5] & 0xFF) << 8) | ((qi[6] & 0xFF) << 16) |
                   (static_cast<uint32_t>(qi[7] & 0xFF) << 24);
        *reinterpret_cast<uint2 *>(qr + col) = packed;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < K) qr[col + e] = static_cast<int8_t>(qi[e]);
    }
    return sum;
}

template <int kAqThreads, int kAqCache>
__global__ void __launch_bounds__(kAqThreads) act_quant_kernel(const uint16_t *__restrict__ x,
                                                               int64_t K, int64_t ldx,
                                                               int8_t *__restrict__ q, int64_t ldq,
                                                               float *__restrict__ s_x,
                                                               int32_t *__restrict__ q_sum) {
#pragma clang fp contract(off)
    constexpr int kWaves = kAqThreads / kWave;
    __shared__ float red_f[kWaves];
    __shared__ int red_i[kWaves];
    const int64_t m = blockIdx.x;
    const uint16_t *xr = x + m * ldx;
    int8_t *qr = q + m * ldq;
    const int tid = threadIdx.x, wid = tid / kWave, lane = tid & (kWave - 1);
    const int64_t n_chunks = (K + 7) / 8;

    uint4 cache[kAqCache];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kAqCache; ++i) {
        const int64_t c = tid + static_cast<int64_t>(i) * kAqThreads;
        cache[i] = c < n_chunks ? *reinterpret_cast<const uint4 *>(xr + 8 * c)
                                : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kAqCache; ++i) {
        const int64_t c = tid + static_cast<int64_t>(i) * kAqThreads;
        if (c < n_chunks) a = fmaxf(a, chunk_absmax(cache[i], 8 * c, K));
    }
    for (int64_t c = tid + static_cast<int64_t>(kAqCache) * kAqThreads; c < n_chunks;
         c += kAqThreads)
        a = fmaxf(a, chunk_absmax(*reinterpret_cast<const uint4 *>(xr + 8 * c), 8 * c, K));
    a = wave_max(a);
    if (lane == 0) red_f[wid] = a;
    __syncthreads();
    a = red_f[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) a = fmaxf(a, red_f[w]);

    const float s = token_scale_int8(a);
    const float r = 1.0f / s;  // correctly rounded; quantize_int8_fast needs it
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kAqCache; ++i) {
        const int64_t c = tid + static_cast<int64_t>(i) * kAqThreads;
        if (c < n_chunks) sum += chunk_quantize(cache[i], 8 * c, K, a, s, r, qr);
    }
    for (int64_t c = tid + static_cast<int64_t>(kAqCache) * kAqThreads; c < n_chunks;
         c += kAqThreads)
        sum += chunk_quantize(*reinterpret_cast<const uint4 *>(xr + 8 * c), 8 * c, K, a, s, r, qr);
    sum = wave_sum(sum);
    if (lane == 0) red_i[wid] = sum;
    __syncthreads();
    if (tid == 0) {
        int total = 0;
        for (int w = 0; w < kWaves; ++w) total += red_i[w];
        s_x[m] = s;
        if (q_sum) q_sum[m] = total;
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
    const dim3 grid(static_cast<unsigned>(M));
    if (K <= 256 * 8 * 4)
        hipLaunchKernelGGL((act_quant_kernel<256, 4>), grid, dim3(256), 0, stream, x, K, ldx, q,
                           ldq, s_x, q_sum);
    else if (K <= 256 * 8 * 10 && M >= 256)  // (a few long rows: more threads per row)
        hipLaunchKernelGGL((act_quant_kernel<256, 10>), grid, dim3(256), 0, stream, x, K, ldx, q,
                           ldq, s_x, q_sum);
    else
        hipLaunchKernelGGL((act_quant_kernel<1024, 4>), grid, dim3(1024), 0, stream, x, K, ldx,
                           q, ldq, s_x, q_sum);
    return hipGetLastError();
}

}  // namespace w4
