// gemm.hip -- W4A16 prefill GEMM for gfx950 on the bf16 matrix cores.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "Prefill和Decode分流": large M runs a
// dense matrix product after dequantization, amortized over many tokens; "融合INT4反量化与矩阵乘":
// no dense weight is written back to memory).  The TPU page ("Yeniden paketlenmiş QAT Gemma 4
// 26B-A4B ...", section "vLLM'in TPU backend'inde değişen ne oldu") dequantizes each weight chunk
// in fast on-chip memory before the multiply; here the on-chip memory is LDS.
//
// Exactness: a weight tile is written to LDS as the exact integers (code - z) in bf16 (|c - z| is
// at most 8 bits for every zero point w4_pack produces), so the bf16 MFMA products x * (c - z) are
// exact and accumulate in fp32.  Each group's fp32 partial product is multiplied by its scale
// s[n][G] once, in fp32 -- the dequantized weight s (c - z) is never rounded to bf16.
//
// Tiling: 256 threads (4 waves, 2 x 2); block tile 128 tokens x 128 output channels; K step 32
// (one v_mfma_f32_16x16x32_bf16 deep); each wave owns 64 x 64 = 4 x 4 MFMA tiles.  Global loads of
// step k+1 are in flight while step k runs from the other LDS buffer.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_STRIDE = BK + 8;  // elements per LDS row (padded against bank conflicts)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

template <bool ZP>
__global__ void __launch_bounds__(256) gemm_w4a16_kernel(
    const uint16_t *__restrict__ x, int64_t M, int64_t ldx, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int64_t d_out, int64_t d_in, int64_t k_pad,
    int steps_per_group, int64_t n_groups, void *__restrict__ y, int64_t ldy, int out_f32) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN * LDS_STRIDE];
    __shared__ float ss[2][BN];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int wm = wid >> 1, wn = wid & 1;
    const int64_t tiles_m = (M + BM - 1) / BM;
    const int64_t tile_n = (int64_t)blockIdx.x / tiles_m;
    const int64_t m0 = ((int64_t)blockIdx.x - tile_n * tiles_m) * BM;
    const int64_t n0 = tile_n * BN;
    const int64_t row_bytes = k_pad / 2;
    const int n_steps = static_cast<int>(k_pad / BK);

    // loader roles: thread -> (tile row, half of the 32-column step)
    const int ld_row = tid >> 1;
    const int ld_half = tid & 1;
    const int64_t xm = m0 + ld_row;
    const int64_t wrow = n0 + ld_row;

    uint4 xr[2];
    uint2 wr;
    float zr_f = 8.0f;
    float sr_f = 0.0f;

    auto load_step = [&](int step) {
        const int64_t k0 = (int64_t)step * BK + 16 * ld_half;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t col = k0 + 8 * p;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (xm < M && col < d_in) {
                v = *reinterpret_cast<const uint4 *>(x + xm * ldx + col);
                if (col + 8 > d_in) {  // zero the columns at or beyond d_in
                    uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e >= d_in) u[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                    v = make_uint4(u[0], u[1], u[2], u[3]);
                }
            }
            xr[p] = v;
        }
        const int64_t G = (int64_t)step / steps_per_group;
        if (wrow < d_out) {
            wr = *reinterpret_cast<const uint2 *>(qweight + wrow * row_bytes + k0 / 2);
            if (ZP) zr_f = bf16_to_f32(zeros[wrow * n_groups + G]);
            sr_f = bf16_to_f32(scales[wrow * n_groups + G]);
        } else {
            wr = make_uint2(0, 0);
            sr_f = 0.0f;
        }
    };

    auto store_step = [&](int buf) {
        uint16_t *xd = &xs[buf][ld_row * LDS_STRIDE + 16 * ld_half];
        *reinterpret_cast<uint4 *>(xd) = xr[0];
        *reinterpret_cast<uint4 *>(xd + 8) = xr[1];
        // dequantize 16 codes to the exact bf16 integers (c - z)
        const uint32_t wv[2] = {wr.x, wr.y};
        uint32_t out[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t byte = (wv[b >> 2] >> (8 * (b & 3))) & 0xFFu;
            const float lo = static_cast<float>(byte & 0xFu) - zr_f;
            const float hi = static_cast<float>(byte >> 4) - zr_f;
            out[b] = pack_bf16x2(lo, hi);
        }
        uint16_t *wd = &ws[buf][ld_row * LDS_STRIDE + 16 * ld_half];
        *reinterpret_cast<uint4 *>(wd) = make_uint4(out[0], out[1], out[2], out[3]);
        *reinterpret_cast<uint4 *>(wd + 8) = make_uint4(out[4], out[5], out[6], out[7]);
        if (ld_half == 0) ss[buf][ld_row] = sr_f;
    };

    floatx4_t acc[4][4], dacc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
            dacc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }

    load_step(0);
    store_step(0);
    __syncthreads();

    const int frag_row = lane & 15;
    const int frag_k = 8 * (lane >> 4);
    for (int step = 0; step < n_steps; ++step) {
        const int buf = step & 1;
        if (step + 1 < n_steps) load_step(step + 1);

        bf16x8_t a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t *>(
                &xs[buf][(wm * 64 + i * 16 + frag_row) * LDS_STRIDE + frag_k]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *reinterpret_cast<const bf16x8_t *>(
                &ws[buf][(wn * 64 + j * 16 + frag_row) * LDS_STRIDE + frag_k]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dacc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], dacc[i][j], 0, 0, 0);

        if ((step + 1) % steps_per_group == 0) {
            // end of a group: scale the group's partial products by s[n][G] in fp32
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float s = ss[buf][wn * 64 + j * 16 + frag_row];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(s, dacc[i][j][r], acc[i][j][r]);
                    dacc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
            }
        }
        if (step + 1 < n_steps) store_step(buf ^ 1);
        __syncthreads();
    }

    // epilogue: D[i][j] of a 16x16 tile sits in lane j + 16 * (i / 4), element i % 4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + frag_row;
        if (n >= d_out) continue;
        const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
                if (m < M) store_out(y, m * ldy + n, acc[i][j][r] + bv, out_f32 != 0);
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    const int steps_per_group = static_cast<int>(span / BK);
    const int64_t tiles = ((d_out + BN - 1) / BN) * ((M + BM - 1) / BM);
    const dim3 grid(static_cast<unsigned>(tiles));
    if (zeros)
        hipLaunchKernelGGL(gemm_w4a16_kernel<true>, grid, dim3(256), 0, stream, x, M, ldx, qweight,
                           scales, zeros, bias, d_out, d_in, k_pad, steps_per_group, n_groups, y,
                           ldy, out_f32 ? 1 : 0);
    else
        hipLaunchKernelGGL(gemm_w4a16_kernel<false>, grid, dim3(256), 0, stream, x, M, ldx,
                           qweight, scales, zeros, bias, d_out, d_in, k_pad, steps_per_group,
                           n_groups, y, ldy, out_f32 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace w4
