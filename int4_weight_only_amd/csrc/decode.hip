// decode.hip -- decode-time linear kernels for gfx950: W4A16 GEMV (bf16 activations) and W4A8
// GEMV (int8 activations, int32 accumulation).
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化", [Orin] "Jetson Orin AGX INT4 推理优化实践：super
// 分支从 9 tok/s 到 24 tok/s".
//
// Decode reads every weight once per token and does little arithmetic per byte
// ([Lab5 基础], [Orin 模型尺寸和 decode 的真实瓶颈]), so both kernels are built around the HBM
// stream of packed weights:
//   * a chunk is 16 bytes of a packed row = 32 consecutive columns, always inside one group;
//   * a "stream" is S waves of a workgroup; wave s of the stream owns chunk steps
//     t in [s*T, (s+1)*T) of every row it visits, lane l loading chunk (s*T + t)*64 + l, so each
//     load instruction reads 1 KiB of contiguous packed bytes;
//   * the activations of the wave's fixed chunk columns are loaded once and stay in registers
//     while the stream walks its rows (the rows-share-one-activation-load idea of
//     [Orin o2-all 和 o4-all 为什么能加速], applied to every row a wave visits);
//   * lane partials are summed across the wave with cross-lane shuffles and across the S waves
//     of a stream through LDS; the sums run in a fixed order, so results are deterministic.
#include <stdlib.h>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kChunkCols = 32;  // columns per 16-byte chunk
constexpr int kBlockThreads = 256;  // launch size of every decode kernel (= its launch bound)
constexpr int kMaxS = kBlockThreads / kWave;  // waves sharing one row

// ---------------------------------------------------------------------------------------------
// W4A16.  Dequantization happens inside the dot product ([Lab5 融合INT4反量化与矩阵乘]):
//   for one u32 of packed codes (columns k0..k7, k_i in bits 4i..4i+3):
//     (w & 0x000F000F) | 0x6400_6400  = fp16 pair (1024 + c0, 1024 + c4)
//     (w & 0x00F000F0) | 0x6400_6400  = fp16 pair (1024 + 16 c1, 1024 + 16 c5)
//   and the same on w >> 8 for (c2, c6), (c3, c7).  One packed fp16 add / fma then gives the
//   exact integers (c - z) (|c - z| <= 2048), and v_dot2_f32_f16 multiplies them by the
//   activations paired the same way, accumulating in fp32.  Each chunk's sum is scaled by its
//   group's s in fp32.  Activations are carried in fp16 after an exact power-of-two rescale per
//   lane (bf16 has 8 significant bits, fp16 11), so the products are exact.
// Zero points that are not integers of magnitude <= 1024 (never produced by w4_pack, but legal
// bf16 inputs) are split into such an integer and a residual applied through the chunk's
// activation sum.
// ---------------------------------------------------------------------------------------------
template <int MT, int T, int U, bool ZP>
__global__ void __launch_bounds__(kBlockThreads) gemv_w4a16_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int M, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int64_t d_out, int64_t d_in, int64_t k_pad,
    int chunk_group_shift, int64_t n_groups, void *__restrict__ y, int64_t ldy, int out_f32,
    int S, int R) {
    extern __shared__ float partial[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int n_streams_blk = (blockDim.x / kWave) / S;
    const int stream_blk = wid / S;
    const int s_idx = wid - stream_blk * S;
    const int64_t total_streams = (int64_t)gridDim.x * n_streams_blk;
    const int64_t stream_id = (int64_t)blockIdx.x * n_streams_blk + stream_blk;
    const int64_t cpr = k_pad / kChunkCols;
    const int64_t row_bytes = k_pad / 2;

    // Rows are visited in batches of U; the loads of the next batch (codes, scales and zero
    // points) are issued before the current batch is computed, and the first batch is requested
    // before the activation set-up.  Vector-memory loads retire in order, so every load the
    // compute needs is part of a batch: nothing issued later can make it wait for the prefetch.
    struct Batch {
        u32x4_t w[U][T];
        uint32_t sz[U][T];  // scale bits | zero-point bits << 16
    };
    auto load_batch = [&](int it0, Batch &dst) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = stream_id + (int64_t)(it0 + u) * total_streams;
            const bool row_ok = (it0 + u) < R && row < d_out;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                // Loads are unconditional (an out-of-range lane reads row 0, chunk 0, and its
                // data is never used) so the compiler can count outstanding loads exactly.
                const int64_t c = (int64_t)(s_idx * T + t) * kWave + lane;
                const bool ok = row_ok && c < cpr;
                const int64_t rr = ok ? row : 0;
                const int64_t cc = ok ? c : 0;
                dst.w[u][t] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t *>(qweight + rr * row_bytes) + cc);
                const int64_t gi = rr * n_groups + (cc >> chunk_group_shift);
                uint32_t v = scales[gi];
                if (ZP) v |= static_cast<uint32_t>(zeros[gi]) << 16;
                dst.sz[u][t] = v;
            }
        }
    };
    Batch wa, wb;
    load_batch(0, wa);

    // ---- activations of this lane's chunk columns, in registers for the whole kernel ----
    // Two passes over the (cached) activations keep the set-up's register use low: the first
    // finds the lane's max |x| per token, the second converts and pairs the values.
    half2_t xf[MT][T][16];
    float xsum[MT][T];
    int xexp[MT];
    auto load_piece = [&](int m, int64_t c, int p, float *dst) {
        const int64_t col = c * kChunkCols + 8 * p;
        const bool ok = m < M && c < cpr && col < d_in;
        const uint4 v = *reinterpret_cast<const uint4 *>(x + (ok ? (int64_t)m * ldx + col : 0));
        const uint32_t u[4] = {ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t bits = (e & 1) ? (u[e >> 1] >> 16) : (u[e >> 1] & 0xFFFFu);
            dst[e] = (col + e < d_in) ? bf16_to_f32(bits) : 0.0f;
        }
    };
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        float amax = 0.0f;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t c = (int64_t)(s_idx * T + t) * kWave + lane;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float v[8];
                load_piece(m, c, p, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
            }
        }
        // x' = x * 2^-E with max|x'| in [2^14, 2^15): every bf16 value converts to fp16 exactly
        // unless it is below max|x| * 2^-24, where the rounding error is negligible.
        const int e = amax > 0.0f ? ilogbf(amax) - 14 : 0;
        xexp[m] = e;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t c = (int64_t)(s_idx * T + t) * kWave + lane;
            float sum = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float v[8];
                load_piece(m, c, j, v);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    half2_t h;
                    h.x = static_cast<half_t>(ldexpf(v[i], -e));
                    h.y = static_cast<half_t>(ldexpf(v[i + 4], -e));
                    xf[m][t][4 * j + i] = h;
                    sum += static_cast<float>(h.x) + static_cast<float>(h.y);
                }
            }
            xsum[m][t] = sum;
        }
    }

    const half2_t one16 = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
    auto compute_batch = [&](int it0, const Batch &bt) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = it0 + u;
            if (it >= R) break;  // uniform across the block
            const int64_t row = stream_id + (int64_t)it * total_streams;
            float acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
            if (row < d_out) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int64_t c = (int64_t)(s_idx * T + t) * kWave + lane;
                    if (c >= cpr) continue;
                    const float s = bf16_to_f32(bt.sz[u][t] & 0xFFFFu);
                    float z = 8.0f;
                    if (ZP) z = bf16_to_f32(bt.sz[u][t] >> 16);
                    const bool zint = (z == __builtin_rintf(z)) && fabsf(z) <= 1024.0f;
                    const float zi = zint ? z : 0.0f;
                    const float zres = z - zi;
                    const half_t n0 = static_cast<half_t>(-(1024.0f + zi));
                    const half_t n1 = static_cast<half_t>(-(64.0f + zi));
                    const half2_t nz0 = {n0, n0};
                    const half2_t nz1 = {n1, n1};
                    const uint32_t wv[4] = {bt.w[u][t][0], bt.w[u][t][1], bt.w[u][t][2],
                                            bt.w[u][t][3]};
                    float d0[MT], d1[MT];
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        d0[m] = 0.0f;
                        d1[m] = 0.0f;
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w0 = wv[j];
                        const uint32_t w8 = w0 >> 8;
                        const half2_t a0 = as_half2((w0 & 0x000F000Fu) | 0x64006400u) + nz0;
                        const half2_t a1 = __builtin_elementwise_fma(
                            as_half2((w0 & 0x00F000F0u) | 0x64006400u), one16, nz1);
                        const half2_t a2 = as_half2((w8 & 0x000F000Fu) | 0x64006400u) + nz0;
                        const half2_t a3 = __builtin_elementwise_fma(
                            as_half2((w8 & 0x00F000F0u) | 0x64006400u), one16, nz1);
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            d0[m] = __builtin_amdgcn_fdot2(a0, xf[m][t][4 * j + 0], d0[m], false);
                            d1[m] = __builtin_amdgcn_fdot2(a1, xf[m][t][4 * j + 1], d1[m], false);
                            d0[m] = __builtin_amdgcn_fdot2(a2, xf[m][t][4 * j + 2], d0[m], false);
                            d1[m] = __builtin_amdgcn_fdot2(a3, xf[m][t][4 * j + 3], d1[m], false);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const float chunk = (d0[m] + d1[m]) - zres * xsum[m][t];
                        acc[m] = fmaf(s, chunk, acc[m]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float v = wave_sum_dpp(ldexpf(acc[m], xexp[m]));
                if (lane == 0) partial[((stream_blk * R + it) * S + s_idx) * MT + m] = v;
            }
        }
    };

    for (int it0 = 0; it0 < R; it0 += 2 * U) {
        if (it0 + U < R) load_batch(it0 + U, wb);
        compute_batch(it0, wa);
        if (it0 + U >= R) break;
        if (it0 + 2 * U < R) load_batch(it0 + 2 * U, wa);
        compute_batch(it0 + U, wb);
    }
    __syncthreads();
    const int n_out = n_streams_blk * R * MT;
    for (int idx = threadIdx.x; idx < n_out; idx += blockDim.x) {
        const int sb = idx / (R * MT);
        const int rem = idx - sb * R * MT;
        const int it = rem / MT;
        const int m = rem - it * MT;
        const int64_t r = ((int64_t)blockIdx.x * n_streams_blk + sb) + (int64_t)it * total_streams;
        if (r >= d_out || m >= M) continue;
        float v = 0.0f;
        for (int s2 = 0; s2 < S; ++s2) v += partial[((sb * R + it) * S + s2) * MT + m];
        if (bias) v += bf16_to_f32(bias[r]);
        store_out(y, (int64_t)m * ldy + r, v, out_f32 != 0);
    }
}

// ---------------------------------------------------------------------------------------------
// W4A8 ([Orin 从 FP 线性层到 INT4 DP4A 的数学推导], [Orin DP4A 做了什么]).
// For one u32 of codes: (w & 0x0F0F0F0F) holds the codes of columns 0,2,4,6 as bytes and
// ((w >> 4) & 0x0F0F0F0F) those of columns 1,3,5,7; the int8 activations are permuted the same
// way once, and v_dot4_i32_i8 accumulates code * q exactly.  The offset of 8 is removed with the
// lane's own activation sum: sum (c - 8) q = sum c q - 8 sum q, all in int32.
// ---------------------------------------------------------------------------------------------
template <int MT, int T, int U>
__global__ void __launch_bounds__(kBlockThreads) gemv_w4a8_kernel(
    const int8_t *__restrict__ q, int64_t ldq, int M, const float *__restrict__ s_x,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ s_w,
    const uint16_t *__restrict__ bias, int64_t d_out, int64_t d_in, int64_t k_pad,
    void *__restrict__ y, int64_t ldy, int out_f32, int32_t *__restrict__ acc_out, int S,
    int R) {
    extern __shared__ int ipartial[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int n_streams_blk = (blockDim.x / kWave) / S;
    const int stream_blk = wid / S;
    const int s_idx = wid - stream_blk * S;
    const int64_t total_streams = (int64_t)gridDim.x * n_streams_blk;
    const int64_t stream_id = (int64_t)blockIdx.x * n_streams_blk + stream_blk;
    const int64_t cpr = k_pad / kChunkCols;
    const int64_t row_bytes = k_pad / 2;

    auto load_batch = [&](int it0, u32x4_t (&dst)[U][T]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = stream_id + (int64_t)(it0 + u) * total_streams;
            const bool row_ok = (it0 + u) < R && row < d_out;
#pragma unroll
            for (int t = 0; t < T; ++t) {
                // unconditional loads (see the W4A16 kernel); unused lanes read row 0, chunk 0
                const int64_t c = (int64_t)(s_idx * T + t) * kWave + lane;
                const bool ok = row_ok && c < cpr;
                dst[u][t] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t *>(qweight + (ok ? row : 0) * row_bytes) +
                    (ok ? c : 0));
            }
        }
    };
    u32x4_t wa[U][T], wb[U][T];
    load_batch(0, wa);

    uint32_t xe[MT][T][4], xo[MT][T][4];
    int qsum[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        int sum = 0;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t c = (int64_t)(s_idx * T + t) * kWave + lane;
            uint32_t u[8];
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int64_t col = c * kChunkCols + 16 * p;
                const bool ok = m < M && c < cpr && col < d_in;
                const uint4 v =
                    *reinterpret_cast<const uint4 *>(q + (ok ? (int64_t)m * ldq + col : 0));
                u[4 * p + 0] = ok ? v.x : 0u;
                u[4 * p + 1] = ok ? v.y : 0u;
                u[4 * p + 2] = ok ? v.z : 0u;
                u[4 * p + 3] = ok ? v.w : 0u;
            }
            // zero the columns at or beyond d_in, and add up the rest
#pragma unroll
            for (int b = 0; b < 32; ++b) {
                const int64_t col = c * kChunkCols + b;
                const uint32_t shift = 8 * (b & 3);
                if (col >= d_in) u[b >> 2] &= ~(0xFFu << shift);
                sum += static_cast<int8_t>((u[b >> 2] >> shift) & 0xFFu);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                xe[m][t][j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x06040200u);
                xo[m][t][j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x07050301u);
            }
        }
        qsum[m] = sum;
    }

    auto compute_batch = [&](int it0, const u32x4_t (&w)[U][T]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = it0 + u;
            if (it >= R) break;  // uniform across the block
            const int64_t row = stream_id + (int64_t)it * total_streams;
            int acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = 0;
            if (row < d_out) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const uint32_t wv[4] = {w[u][t][0], w[u][t][1], w[u][t][2], w[u][t][3]};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int lo = static_cast<int>(wv[j] & 0x0F0F0F0Fu);
                        const int hi = static_cast<int>((wv[j] >> 4) & 0x0F0F0F0Fu);
#pragma unroll
                        for (int m = 0; m < MT; ++m) {
                            acc[m] = __builtin_amdgcn_sdot4(lo, static_cast<int>(xe[m][t][j]),
                                                            acc[m], false);
                            acc[m] = __builtin_amdgcn_sdot4(hi, static_cast<int>(xo[m][t][j]),
                                                            acc[m], false);
                        }
                    }
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[m] -= 8 * qsum[m];
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int v = wave_sum_dpp(acc[m]);
                if (lane == 0) ipartial[((stream_blk * R + it) * S + s_idx) * MT + m] = v;
            }
        }
    };

    for (int it0 = 0; it0 < R; it0 += 2 * U) {
        if (it0 + U < R) load_batch(it0 + U, wb);
        compute_batch(it0, wa);
        if (it0 + U >= R) break;
        if (it0 + 2 * U < R) load_batch(it0 + 2 * U, wa);
        compute_batch(it0 + U, wb);
    }
    __syncthreads();
    const int n_out = n_streams_blk * R * MT;
    for (int idx = threadIdx.x; idx < n_out; idx += blockDim.x) {
        const int sb = idx / (R * MT);
        const int rem = idx - sb * R * MT;
        const int it = rem / MT;
        const int m = rem - it * MT;
        const int64_t r = ((int64_t)blockIdx.x * n_streams_blk + sb) + (int64_t)it * total_streams;
        if (r >= d_out || m >= M) continue;
        int a = 0;
        for (int s2 = 0; s2 < S; ++s2) a += ipartial[((sb * R + it) * S + s2) * MT + m];
        if (acc_out) acc_out[(int64_t)m * d_out + r] = a;
        const float scale = bf16_to_f32(s_w[r]) * s_x[m];
        float v = scale * static_cast<float>(a);
        if (bias) v += bf16_to_f32(bias[r]);
        store_out(y, (int64_t)m * ldy + r, v, out_f32 != 0);
    }
}

// Rows per batch: the double-buffered weights of 2 * U * T chunks stay within 64 registers.
constexpr int batch_rows(int T) { return T >= 5 ? 1 : (8 / T > 4 ? 4 : 8 / T); }

struct DecodePlan {
    int T, S, waves, grid, R;
};

// Workgroups per compute unit of the persistent decode grid.
constexpr int kDecodeBlocksPerCu = 2;
int decode_blocks_per_cu() { return kDecodeBlocksPerCu; }

// Waves (at most kMaxS, all in one 256-thread workgroup) x T steps needed to cover a row of
// `cpr` chunks; returns T, or a value above t_max if even kMaxS waves are not enough.
int steps_needed(int64_t cpr, int S) {
    return static_cast<int>((cpr + (int64_t)kWave * S - 1) / ((int64_t)kWave * S));
}

// Split a row's chunks over S waves x T steps (T <= t_max, S <= kMaxS), then spread rows over
// the grid.  The caller has checked that steps_needed(cpr, kMaxS) <= t_max.
DecodePlan plan_decode(int64_t d_out, int64_t cpr, int t_max) {
    DecodePlan p{};
    int S = 1;
    while (steps_needed(cpr, S) > t_max && S < kMaxS) S *= 2;
    p.S = S;
    p.T = steps_needed(cpr, S);
    p.waves = kBlockThreads / kWave;
    const int n_streams_blk = p.waves / S;
    // A persistent grid of a few blocks per CU; every stream walks R rows.
    const int64_t want_blocks = (d_out + n_streams_blk - 1) / n_streams_blk;
    int64_t blocks = (int64_t)device_cu_count() * decode_blocks_per_cu();
    // at most 64 rows per stream (bounds the per-row LDS partials)
    const int64_t min_blocks =
        (d_out + (int64_t)n_streams_blk * 64 - 1) / ((int64_t)n_streams_blk * 64);
    if (blocks < min_blocks) blocks = min_blocks;
    if (blocks > want_blocks) blocks = want_blocks;
    const int64_t streams = blocks * n_streams_blk;
    p.R = static_cast<int>((d_out + streams - 1) / streams);
    // with R fixed, use no more blocks than the rows need
    p.grid = static_cast<int>((d_out + (int64_t)p.R * n_streams_blk - 1) /
                              ((int64_t)p.R * n_streams_blk));
    return p;
}

template <int MT, int T>
hipError_t launch_w4a16_t(const DecodePlan &p, bool zp, const uint16_t *x, int64_t ldx, int M,
                          const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                          const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                          int shift, int64_t n_groups, void *y, int64_t ldy, bool out_f32,
                          hipStream_t stream) {
    const size_t lds = sizeof(float) * (size_t)(p.waves / p.S) * p.R * p.S * MT;
    constexpr int U = batch_rows(T);
    if (zp)
        hipLaunchKernelGGL((gemv_w4a16_kernel<MT, T, U, true>), dim3(p.grid),
                           dim3(p.waves * kWave), lds, stream, x, ldx, M, qweight, scales, zeros,
                           bias, d_out, d_in, k_pad, shift, n_groups, y, ldy, out_f32 ? 1 : 0,
                           p.S, p.R);
    else
        hipLaunchKernelGGL((gemv_w4a16_kernel<MT, T, U, false>), dim3(p.grid),
                           dim3(p.waves * kWave), lds, stream, x, ldx, M, qweight, scales, zeros,
                           bias, d_out, d_in, k_pad, shift, n_groups, y, ldy, out_f32 ? 1 : 0,
                           p.S, p.R);
    return hipGetLastError();
}

// Largest T instantiated per token count (register budget of the activation fragments).
constexpr int kW4A16TMax[5] = {0, 8, 4, 3, 2};
constexpr int kW4A8TMax[5] = {0, 8, 6, 4, 3};

template <int MT, int T>
hipError_t launch_w4a16_upto(const DecodePlan &p, bool zp, const uint16_t *x, int64_t ldx, int M,
                             const uint8_t *qweight, const uint16_t *scales,
                             const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                             int64_t d_in, int64_t k_pad, int shift, int64_t n_groups, void *y,
                             int64_t ldy, bool out_f32, hipStream_t stream) {
    if (p.T == T)
        return launch_w4a16_t<MT, T>(p, zp, x, ldx, M, qweight, scales, zeros, bias, d_out, d_in,
                                     k_pad, shift, n_groups, y, ldy, out_f32, stream);
    if constexpr (T > 1)
        return launch_w4a16_upto<MT, T - 1>(p, zp, x, ldx, M, qweight, scales, zeros, bias, d_out,
                                            d_in, k_pad, shift, n_groups, y, ldy, out_f32, stream);
    return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_w4a16_mt(const DecodePlan &p, bool zp, const uint16_t *x, int64_t ldx, int M,
                           const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                           const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                           int shift, int64_t n_groups, void *y, int64_t ldy, bool out_f32,
                           hipStream_t stream) {
    return launch_w4a16_upto<MT, kW4A16TMax[MT]>(p, zp, x, ldx, M, qweight, scales, zeros, bias,
                                                 d_out, d_in, k_pad, shift, n_groups, y, ldy,
                                                 out_f32, stream);
}

template <int MT, int T>
hipError_t launch_w4a8_t(const DecodePlan &p, const int8_t *q, int64_t ldq, int M,
                         const float *s_x, const uint8_t *qweight, const uint16_t *s_w,
                         const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                         void *y, int64_t ldy, bool out_f32, int32_t *acc, hipStream_t stream) {
    const size_t lds = sizeof(int) * (size_t)(p.waves / p.S) * p.R * p.S * MT;
    constexpr int U = batch_rows(T);
    hipLaunchKernelGGL((gemv_w4a8_kernel<MT, T, U>), dim3(p.grid), dim3(p.waves * kWave), lds, stream,
                       q, ldq, M, s_x, qweight, s_w, bias, d_out, d_in, k_pad, y, ldy,
                       out_f32 ? 1 : 0, acc, p.S, p.R);
    return hipGetLastError();
}

template <int MT, int T>
hipError_t launch_w4a8_upto(const DecodePlan &p, const int8_t *q, int64_t ldq, int M,
                            const float *s_x, const uint8_t *qweight, const uint16_t *s_w,
                            const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                            void *y, int64_t ldy, bool out_f32, int32_t *acc,
                            hipStream_t stream) {
    if (p.T == T)
        return launch_w4a8_t<MT, T>(p, q, ldq, M, s_x, qweight, s_w, bias, d_out, d_in, k_pad, y,
                                    ldy, out_f32, acc, stream);
    if constexpr (T > 1)
        return launch_w4a8_upto<MT, T - 1>(p, q, ldq, M, s_x, qweight, s_w, bias, d_out, d_in,
                                           k_pad, y, ldy, out_f32, acc, stream);
    return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_w4a8_mt(const DecodePlan &p, const int8_t *q, int64_t ldq, int M,
                          const float *s_x, const uint8_t *qweight, const uint16_t *s_w,
                          const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                          void *y, int64_t ldy, bool out_f32, int32_t *acc, hipStream_t stream) {
    return launch_w4a8_upto<MT, kW4A8TMax[MT]>(p, q, ldq, M, s_x, qweight, s_w, bias, d_out, d_in,
                                               k_pad, y, ldy, out_f32, acc, stream);
}

int log2_exact(int64_t v) {
    int s = 0;
    while (((int64_t)1 << s) < v) ++s;
    return s;
}

}  // namespace

hipError_t launch_gemv(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    // Group-aligned shapes: the int8 matrix cores, with the codes as an operand as they are.
    if (gemv_i8_preferred(M, d_out, k_pad) &&
        gemv_i8_supported(M, d_out, d_in, k_pad, span, n_groups, ldx))
        return launch_gemv_i8(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, k_pad, span,
                              n_groups, y, ldy, out_f32, false, stream);
    // Two or more tokens: the matrix-core path reads the weights once for all of them.
    if (gemv_mfma_supported(M, d_out, d_in, k_pad, span, n_groups, ldx, zeros != nullptr))
        return launch_gemv_mfma(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, k_pad, span,
                                n_groups, y, ldy, out_f32, stream);
    const int64_t cpr = k_pad / kChunkCols;
    // chunks per group is a power of two (group sizes 32..256); one group per row -> shift 62
    const int shift = n_groups == 1 ? 62 : log2_exact(span / kChunkCols);
    // the streaming kernel serves rows up to its LDS budget; longer rows (and tokens in tiles of
    // up to 4) fall back to the per-row kernels below
    if (gemv_stream_supported(M, k_pad))
        return launch_gemv_stream(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, k_pad,
                                  shift, n_groups, y, ldy, out_f32, stream);
    const bool zp = zeros != nullptr;
    const size_t out_elem = out_f32 ? sizeof(float) : sizeof(uint16_t);
    int mt_max = 4;
    while (mt_max > 1 && steps_needed(cpr, kMaxS) > kW4A16TMax[mt_max]) --mt_max;
    if (steps_needed(cpr, kMaxS) > kW4A16TMax[mt_max]) return hipErrorInvalidValue;
    for (int64_t m0 = 0; m0 < M; m0 += mt_max) {
        const int mt = static_cast<int>(M - m0 < mt_max ? M - m0 : mt_max);
        const DecodePlan p = plan_decode(d_out, cpr, kW4A16TMax[mt]);
        if (p.T > kW4A16TMax[mt] || p.waves * kWave != kBlockThreads) return hipErrorInvalidValue;
        const uint16_t *xm = x + m0 * ldx;
        void *ym = static_cast<char *>(y) + m0 * ldy * out_elem;
        hipError_t err;
        switch (mt) {
            case 1:
                err = launch_w4a16_mt<1>(p, zp, xm, ldx, mt, qweight, scales, zeros, bias, d_out,
                                         d_in, k_pad, shift, n_groups, ym, ldy, out_f32, stream);
                break;
            case 2:
                err = launch_w4a16_mt<2>(p, zp, xm, ldx, mt, qweight, scales, zeros, bias, d_out,
                                         d_in, k_pad, shift, n_groups, ym, ldy, out_f32, stream);
                break;
            case 3:
                err = launch_w4a16_mt<3>(p, zp, xm, ldx, mt, qweight, scales, zeros, bias, d_out,
                                         d_in, k_pad, shift, n_groups, ym, ldy, out_f32, stream);
                break;
            default:
                err = launch_w4a16_mt<4>(p, zp, xm, ldx, mt, qweight, scales, zeros, bias, d_out,
                                         d_in, k_pad, shift, n_groups, ym, ldy, out_f32, stream);
                break;
        }
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

hipError_t launch_w4a8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                       const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                       bool out_f32, int32_t *acc, hipStream_t stream) {
    // two or more tokens: the matrix-core kernel reads the weights once per 16 of them
    if (w4a8_tok_supported(M, d_out, d_in, k_pad, ldq))
        return launch_w4a8_tok(q, s_x, M, ldq, qweight, s_w, bias, d_out, d_in, k_pad, y, ldy,
                               out_f32, acc, stream);
    if (w4a8_stream_supported(M, k_pad, false))  // see launch_gemv
        return launch_w4a8_stream(q, false, const_cast<float *>(s_x), M, ldq, qweight, s_w, bias,
                                  d_out, d_in, k_pad, y, ldy, out_f32, acc, stream);
    const int64_t cpr = k_pad / kChunkCols;
    const size_t out_elem = out_f32 ? sizeof(float) : sizeof(uint16_t);
    int mt_max = 4;
    while (mt_max > 1 && steps_needed(cpr, kMaxS) > kW4A8TMax[mt_max]) --mt_max;
    if (steps_needed(cpr, kMaxS) > kW4A8TMax[mt_max]) return hipErrorInvalidValue;
    for (int64_t m0 = 0; m0 < M; m0 += mt_max) {
        const int mt = static_cast<int>(M - m0 < mt_max ? M - m0 : mt_max);
        const DecodePlan p = plan_decode(d_out, cpr, kW4A8TMax[mt]);
        if (p.T > kW4A8TMax[mt] || p.waves * kWave != kBlockThreads) return hipErrorInvalidValue;
        const int8_t *qm = q + m0 * ldq;
        void *ym = static_cast<char *>(y) + m0 * ldy * out_elem;
        int32_t *am = acc ? acc + m0 * d_out : nullptr;
        hipError_t err;
        switch (mt) {
            case 1:
                err = launch_w4a8_mt<1>(p, qm, ldq, mt, s_x + m0, qweight, s_w, bias, d_out, d_in,
                                        k_pad, ym, ldy, out_f32, am, stream);
                break;
            case 2:
                err = launch_w4a8_mt<2>(p, qm, ldq, mt, s_x + m0, qweight, s_w, bias, d_out, d_in,
                                        k_pad, ym, ldy, out_f32, am, stream);
                break;
            case 3:
                err = launch_w4a8_mt<3>(p, qm, ldq, mt, s_x + m0, qweight, s_w, bias, d_out, d_in,
                                        k_pad, ym, ldy, out_f32, am, stream);
                break;
            default:
                err = launch_w4a8_mt<4>(p, qm, ldq, mt, s_x + m0, qweight, s_w, bias, d_out, d_in,
                                        k_pad, ym, ldy, out_f32, am, stream);
                break;
        }
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// The fused path is the streaming kernel only: the per-row fallback kernels take int8 codes.
bool w4a8_linear_supported(int64_t M, int64_t k_pad) {
    return w4a8_stream_supported(M, k_pad, true);
}

hipError_t launch_w4a8_linear(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                              const uint16_t *s_w, const uint16_t *bias, int64_t d_out,
                              int64_t d_in, int64_t k_pad, void *y, int64_t ldy, bool out_f32,
                              float *s_x, int32_t *acc, hipStream_t stream) {
    if (!w4a8_linear_supported(M, k_pad)) return hipErrorInvalidValue;
    return launch_w4a8_stream(x, true, s_x, M, ldx, qweight, s_w, bias, d_out, d_in, k_pad, y,
                              ldy, out_f32, acc, stream);
}

}  // namespace w4
