// gemm_w4a8.hip -- W4A8 prefill GEMM on the int8 matrix cores (gfx950), any number of tokens.
//
// Pages: [Orin] "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s" (sections "从 FP
// 线性层到 INT4 DP4A 的数学推导": y = s_W s_x sum (code - 8) q + b with int8 activations and an
// integer accumulator; "INT32 accumulator 是否安全": the int32 bound; "DP4A 做了什么": integer dot
// products of 4-bit codes against 8-bit operands), [Infra] "【infra之路】12-投机解码、量化与推理
// 引擎对比" (section 2.3: W8A8-style integer GEMMs with int32 accumulation at large batch).
//
// acc[m][n] = sum_{k < d_in} (code[n][k] - 8) q[m][k] is computed exactly as
// sum_k code q - 8 sum_k q on v_mfma_i32_16x16x64_i8: the 4-bit codes (0..15) are int8 operands as
// they are, and each token's sum of q is taken from the same activation registers. The epilogue
// is y = (s_W[n] s_x[m]) acc + b[n] in fp32, as in the W4A8 GEMV.
//
// Tiling: 256 threads (4 waves, 2 x 2), a block tile of 128 tokens x 128 output rows, K in steps
// of 128 columns. Each wave owns 64 x 64 outputs (4 x 4 MFMA tiles) and loads its operands from
// memory into registers one step ahead, without LDS:
//   * weights: lane (n, kq) of an N tile reads the 16 bytes (32 codes, columns 32 kq .. + 31 of
//     the step) of row n; the low nibbles (w & 0x0F0F0F0F, the even columns) and the high ones
//     ((w >> 4) & 0x0F0F0F0F, the odd columns) are the B operands of two MFMAs;
//   * activations: lane (m, kq) of an M tile reads the same 32 columns of token m and permutes the
//     bytes into the even and the odd columns, so both MFMAs pair each code with its activation
//     (any order of K works as long as both operands follow it).
// Loads are raw buffer loads: a token past M, a row past d_out or a column past d_in reads zeros.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kG8Threads = 256;
constexpr int kG8Tile = 128;  // tokens and output rows per block
constexpr int kG8Step = 128;  // columns per K step
constexpr int kG8T = 4;       // 16 x 16 MFMA tiles per wave in each dimension
constexpr int kG8Xcds = 8;

template <bool RAGGED>
__global__ void __launch_bounds__(kG8Threads) gemm_w4a8_kernel(
    const int8_t *__restrict__ q, int M, int64_t ldq, const float *__restrict__ s_x,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ s_w,
    const uint16_t *__restrict__ bias, int d_out, int d_in, int row_bytes, int n_steps,
    int tiles_m, int tiles_n, void *__restrict__ y, int64_t ldy, int out_f32,
    int32_t *__restrict__ acc_out) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wid >> 1, wn = wid & 1;
    const int r16 = lane & 15, kq = lane >> 4;

    // XCD-aware order: hardware block b runs on XCD b % 8; the blocks of one XCD take consecutive
    // tiles, tokens fastest, so that they share a weight tile in their L2.
    const int nblocks = tiles_m * tiles_n;
    const int b = static_cast<int>(blockIdx.x);
    int t = b;
    if (nblocks % kG8Xcds == 0) t = (b % kG8Xcds) * (nblocks / kG8Xcds) + b / kG8Xcds;
    const int m0 = (t % tiles_m) * kG8Tile + wm * 64;
    const int n0 = (t / tiles_m) * kG8Tile + wn * 64;

    const rsrc_t rq = make_rsrc(q, static_cast<uint32_t>(M) * static_cast<uint32_t>(ldq));
    const rsrc_t rw = make_rsrc(qweight, static_cast<uint32_t>(d_out) * static_cast<uint32_t>(row_bytes));
    // per-lane parts of the offsets (the host keeps every offset below 2^31)
    uint32_t a_lane[kG8T], b_lane[kG8T];
#pragma unroll
    for (int i = 0; i < kG8T; ++i) {
        const int m = m0 + 16 * i + r16;
        a_lane[i] = m < M ? static_cast<uint32_t>(m) * static_cast<uint32_t>(ldq) + 32u * kq
                          : kOutOfRange;
        const int n = n0 + 16 * i + r16;
        b_lane[i] = n < d_out ? static_cast<uint32_t>(n) * static_cast<uint32_t>(row_bytes) + 16u * kq
                              : kOutOfRange;
    }

    struct Raw {
        u32x4_t a[kG8T][2];  // 32 activation bytes per M tile
        u32x4_t w[kG8T];     // 32 codes per N tile
    };
    auto load = [&](int step, Raw &R) {
        const int col = step * kG8Step + 32 * kq;  // this lane's first column
#pragma unroll
        for (int i = 0; i < kG8T; ++i) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bool ok = col + 16 * h < d_in && a_lane[i] != kOutOfRange;
                const uint32_t off = ok ? a_lane[i] + static_cast<uint32_t>(step * kG8Step + 16 * h)
                                        : kOutOfRange;
                R.a[i][h] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
            }
            const bool okw = col < d_in && b_lane[i] != kOutOfRange;
            const uint32_t offw =
                okw ? b_lane[i] + static_cast<uint32_t>(step * (kG8Step / 2)) : kOutOfRange;
            R.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, offw, 0, 0);
        }
    };

    i32x4_t acc[kG8T][kG8T];
#pragma unroll
    for (int i = 0; i < kG8T; ++i)
#pragma unroll
        for (int j = 0; j < kG8T; ++j) acc[i][j] = i32x4_t{0, 0, 0, 0};
    int qs[kG8T] = {0, 0, 0, 0};  // this lane's share of each M tile token's sum of q

    // the step that holds column d_in - 1 when d_in % 32 != 0 masks its activation bytes
    const int rag_step = RAGGED ? (d_in - 1) / kG8Step : -1;
    auto compute = [&](int step, const Raw &R) {
        i32x4_t ae[kG8T], ao[kG8T];
#pragma unroll
        for (int i = 0; i < kG8T; ++i) {
            uint32_t u[8] = {R.a[i][0].x, R.a[i][0].y, R.a[i][0].z, R.a[i][0].w,
                             R.a[i][1].x, R.a[i][1].y, R.a[i][1].z, R.a[i][1].w};
            if (RAGGED && step == rag_step) {  // columns at or past d_in may hold anything
                const int col0 = step * kG8Step + 32 * kq;
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const int left = d_in - (col0 + 4 * d);  // bytes of u[d] before d_in
                    u[d] &= left >= 4 ? 0xFFFFFFFFu : (left <= 0 ? 0u : (1u << (8 * left)) - 1u);
                }
            }
#pragma unroll
            for (int d = 0; d < 8; ++d)
                qs[i] = __builtin_amdgcn_sdot4(static_cast<int>(u[d]), 0x01010101, qs[i], false);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                ae[i][jj] = static_cast<int>(__builtin_amdgcn_perm(u[2 * jj + 1], u[2 * jj], 0x06040200u));
                ao[i][jj] = static_cast<int>(__builtin_amdgcn_perm(u[2 * jj + 1], u[2 * jj], 0x07050301u));
            }
        }
#pragma unroll
        for (int j = 0; j < kG8T; ++j) {
            const i32x4_t be = {static_cast<int>(R.w[j].x & 0x0F0F0F0Fu),
                                static_cast<int>(R.w[j].y & 0x0F0F0F0Fu),
                                static_cast<int>(R.w[j].z & 0x0F0F0F0Fu),
                                static_cast<int>(R.w[j].w & 0x0F0F0F0Fu)};
            const i32x4_t bo = {static_cast<int>((R.w[j].x >> 4) & 0x0F0F0F0Fu),
                                static_cast<int>((R.w[j].y >> 4) & 0x0F0F0F0Fu),
                                static_cast<int>((R.w[j].z >> 4) & 0x0F0F0F0Fu),
                                static_cast<int>((R.w[j].w >> 4) & 0x0F0F0F0Fu)};
#pragma unroll
            for (int i = 0; i < kG8T; ++i) {
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ae[i], be, acc[i][j], 0, 0, 0);
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ao[i], bo, acc[i][j], 0, 0, 0);
            }
        }
    };

    // operands one step ahead
    Raw R0, R1;
    load(0, R0);
    int s = 0;
    for (; s + 2 <= n_steps; s += 2) {
        phase_fence();
        load(s + 1, R1);  // (s + 1 < n_steps here)
        phase_fence();
        compute(s, R0);
        phase_fence();
        load(s + 2 < n_steps ? s + 2 : s + 1, R0);
        phase_fence();
        compute(s + 1, R1);
    }
    if (s < n_steps) compute(s, R0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the last reload has landed

    // token sums: the lanes (r16, kq) of an M tile hold the 4 column quarters of token r16; the
    // D lanes (n, kq) hold tokens 4 kq .. 4 kq + 3
    int tsum[kG8T][4];
#pragma unroll
    for (int i = 0; i < kG8T; ++i) {
        int v = qs[i];
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
#pragma unroll
        for (int r = 0; r < 4; ++r) tsum[i][r] = __shfl(v, 4 * kq + r, kWave);
    }

    // epilogue: D[i][j] lane (n, kq) holds tokens m0 + 16 i + 4 kq + r of row n0 + 16 j + n
#pragma unroll
    for (int j = 0; j < kG8T; ++j) {
        const int n = n0 + 16 * j + r16;
        if (n >= d_out) continue;
        const float sw = bf16_to_f32(s_w[n]);
        const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < kG8T; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + 16 * i + 4 * kq + r;
                if (m >= M) continue;
                const int a = acc[i][j][r] - 8 * tsum[i][r];
                const float scale = sw * s_x[m];
                float v = scale * static_cast<float>(a);
                if (bias) v += bv;
                if (acc_out) acc_out[static_cast<int64_t>(m) * d_out + n] = a;
                store_out(y, static_cast<int64_t>(m) * ldy + n, v, out_f32 != 0);
            }
        }
    }
}

}  // namespace

bool gemm_w4a8_supported(int64_t M, int64_t d_out, int64_t ldq, int64_t k_pad) {
    if (M < 1 || d_out < 1) return false;
    // 31-bit buffer offsets: the activations and the packed weights (plus one step past the row)
    if (M * ldq + kG8Step >= (int64_t)kOutOfRange) return false;
    return d_out * (k_pad / 2) + kG8Step < (int64_t)kOutOfRange;
}

hipError_t launch_gemm_w4a8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                            const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                            int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                            bool out_f32, int32_t *acc, hipStream_t stream) {
    if (!gemm_w4a8_supported(M, d_out, ldq, k_pad)) return hipErrorInvalidValue;
    const int tiles_m = static_cast<int>((M + kG8Tile - 1) / kG8Tile);
    const int tiles_n = static_cast<int>((d_out + kG8Tile - 1) / kG8Tile);
    const int n_steps = static_cast<int>((d_in + kG8Step - 1) / kG8Step);
    const bool ragged = (d_in & 31) != 0;
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    if (ragged)
        hipLaunchKernelGGL(gemm_w4a8_kernel<true>, grid, dim3(kG8Threads), 0, stream, q,
                           static_cast<int>(M), ldq, s_x, qweight, s_w, bias,
                           static_cast<int>(d_out), static_cast<int>(d_in),
                           static_cast<int>(k_pad / 2), n_steps, tiles_m, tiles_n, y, ldy,
                           out_f32 ? 1 : 0, acc);
    else
        hipLaunchKernelGGL(gemm_w4a8_kernel<false>, grid, dim3(kG8Threads), 0, stream, q,
                           static_cast<int>(M), ldq, s_x, qweight, s_w, bias,
                           static_cast<int>(d_out), static_cast<int>(d_in),
                           static_cast<int>(k_pad / 2), n_steps, tiles_m, tiles_n, y, ldy,
                           out_f32 ? 1 : 0, acc);
    return hipGetLastError();
}

}  // namespace w4
