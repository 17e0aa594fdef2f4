// gptq.hip -- the GPTQ quantizer on the GPU, in fp32, producing the packed format of w4_pack.
//
// Page: [Lab5] "Lab 5: Gemma4 端到端推理优化", section "从 RTN 到 GPTQ": the layer objective
// ||X W^T - X Q^T||_F^2 over calibration activations X [N][d_in]; its Hessian H = (2/N) X^T X;
// dead columns (diag H = 0: their weights are set to zero and H_ii to 1); damping
// H += alpha mean(diag H) I; H^-1 = U^T U with U upper triangular; columns quantized in order,
// e_i = (w_i - q_i) / U_ii and W[:, i:] -= e_i U[i, i:]; the predicted loss
// L_pred = 1/2 sum_i ||w_i - q_i||^2 / U_ii^2. The page builds H, factors it and propagates the
// error in fp32; so does this file.
//
// Steps (each a plain kernel; the host sequences them):
//   * hessian: H = (2/N) X^T X, 64 x 64 output tiles, the tokens staged through LDS in fp32;
//   * factor: dead columns and damping; the reverse Cholesky H = V V^T (V upper triangular),
//     then U = V^-1 by back substitution, so that U^T U = V^-T V^-1 = H^-1. Both run by panels of
//     64 columns from the last panel back: the panel's diagonal block in LDS (one wave), a
//     triangular solve for the rows above it (one thread per row) and a GEMM update of the
//     leading block (the Cholesky), or the substitution inside the panel (one thread per column)
//     and a GEMM for the rows above it (the inverse);
//   * quantize: blocks of 32 columns. Four lanes per output row run the block's columns in
//     order (the group's scale and zero by w4_pack's rule from the current weights at the group's
//     first column, the code, e_i, the updates inside the block, the row's loss), then a GEMM
//     applies the block's errors to the columns after it: W[:, b+32:] -= E U[b:b+32, b+32:].
#include "w4_device.h"
#include "w4_launch.h"

#include <algorithm>
#include <mutex>
#include <vector>

namespace w4 {

// The column loop's block errors for callers that cannot allocate (w4_gptq_quantize_noalloc):
// a file-scope device array, kGqScratchRows rows of 32 floats (8 MiB). Each GPU the library
// runs on holds its own copy until the process ends; every call on one GPU shares it, so calls
// that overlap on one GPU race. Nothing in it needs clearing: the block kernel writes every entry
// of the rows in use before the trailing update reads it. Host code never passes the array's
// name to a kernel (that is a host-side stand-in): it passes the device address from
// hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) float scratch[kGqScratchRows * 32];

hipError_t gptq_scratch(float **ptr) {
    static std::mutex mu;
    static std::vector<float *> by_device;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= static_cast<int>(by_device.size())) by_device.resize(dev + 1, nullptr);
    if (by_device[dev] == nullptr) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        by_device[dev] = static_cast<float *>(p);
    }
    *ptr = by_device[dev];
    return hipSuccess;
}

namespace {

constexpr int kGqTile = 64;
constexpr int kGqBlock = 32;  // columns per quantization block

// H[a][b] = (2/N) sum_n x[n][a] x[n][b]; 256 threads, 4 x 4 outputs each.
__global__ void __launch_bounds__(256) gptq_hessian_kernel(const uint16_t *__restrict__ x,
                                                           int N, int d_in, int64_t ldx,
                                                           float scale, float *__restrict__ h) {
    __shared__ float xa[16][kGqTile + 1], xb[16][kGqTile + 1];
    const int a0 = blockIdx.y * kGqTile, b0 = blockIdx.x * kGqTile;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[4][4] = {};
    for (int n0 = 0; n0 < N; n0 += 16) {
        for (int e = threadIdx.x; e < 16 * kGqTile; e += 256) {
            const int r = e / kGqTile, c = e % kGqTile, n = n0 + r;
            const int ca = a0 + c, cb = b0 + c;
            xa[r][c] = n < N && ca < d_in ? bf16_to_f32(x[n * ldx + ca]) : 0.0f;
            xb[r][c] = n < N && cb < d_in ? bf16_to_f32(x[n * ldx + cb]) : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int r = 0; r < 16; ++r) {
            float va[4], vb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                va[i] = xa[r][ty + 16 * i];
                vb[i] = xb[r][tx + 16 * i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(va[i], vb[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int a = a0 + ty + 16 * i, b = b0 + tx + 16 * j;
            if (a < d_in && b < d_in) h[(int64_t)a * d_in + b] = scale * acc[i][j];
        }
}

// Dead columns and damping, one block: dead[i] = (H_ii == 0); H_ii = 1 there; then
// H_ii += alpha mean(diag H).
__global__ void __launch_bounds__(1024) gptq_prepare_kernel(float *__restrict__ h, int n,
                                                            float alpha,
                                                            uint8_t *__restrict__ dead) {
    __shared__ float part[1024];
    float s = 0.0f;
    for (int i = threadIdx.x; i < n; i += 1024) {
        float d = h[(int64_t)i * n + i];
        const bool z = d == 0.0f;
        if (z) d = 1.0f;
        dead[i] = z ? 1 : 0;
        h[(int64_t)i * n + i] = d;
        s += d;
    }
    part[threadIdx.x] = s;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
        __syncthreads();
    }
    const float lam = alpha * (part[0] / static_cast<float>(n));
    for (int i = threadIdx.x; i < n; i += 1024) h[(int64_t)i * n + i] += lam;
}

// ---- blocked factorization: panels of kGqPanel columns, from the last panel back ----
constexpr int kGqPanel = 64;

// Reverse Cholesky of the panel's diagonal block (its lower triangle, already updated by every
// later panel): V[P][P] (upper), one wave; lane i holds row i of the block in registers, and at
// step k lane k publishes its row through LDS.
__global__ void __launch_bounds__(kGqPanel) gptq_chol_diag_kernel(const float *__restrict__ h,
                                                                  int n, int p0, int nb,
                                                                  float *__restrict__ v) {
    __shared__ float rowk[kGqPanel];
    const int i = threadIdx.x;
    float r[kGqPanel];
#pragma unroll
    for (int j = 0; j < kGqPanel; ++j)
        r[j] = i < nb && j <= i ? h[(int64_t)(p0 + i) * n + p0 + j] : 0.0f;
    for (int k = nb - 1; k >= 0; --k) {
        if (i == k) {
#pragma unroll
            for (int j = 0; j < kGqPanel; ++j) rowk[j] = r[j];
        }
        __syncthreads();
        const float d = rowk[k];
        // column k of V: V[i][k] = a[k][i] / sqrt(d) for i <= k
        if (i <= k) v[(int64_t)(p0 + i) * n + p0 + k] = rowk[i] / sqrtf(d);
        // row i of the leading k x k block: a[i][j] -= a[k][i] a[k][j] / d, j <= i < k
        if (i < k) {
            const float f = rowk[i] / d;
#pragma unroll
            for (int j = 0; j < kGqPanel; ++j)
                if (j <= i) r[j] -= f * rowk[j];
        }
        __syncthreads();  // every lane has read row k before the next one is published
    }
}

// V[i][P] for the rows above the panel: h'[j] = H[p0 + j][i] (updated by the later panels)
// = sum_{m >= j} V[i][p0 + m] V[p0 + j][p0 + m], solved from the last j back; one thread a row.
__global__ void __launch_bounds__(256) gptq_chol_trsm_kernel(const float *__restrict__ h, int n,
                                                             int p0, int nb,
                                                             float *__restrict__ v) {
    __shared__ float vp[kGqPanel][kGqPanel + 1];
    for (int e = threadIdx.x; e < kGqPanel * kGqPanel; e += 256) {
        const int j = e / kGqPanel, m = e % kGqPanel;
        vp[j][m] = j < nb && m < nb && m >= j ? v[(int64_t)(p0 + j) * n + p0 + m] : 0.0f;
    }
    __syncthreads();
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= p0) return;
    float x[kGqPanel];
#pragma unroll
    for (int j = 0; j < kGqPanel; ++j) x[j] = j < nb ? h[(int64_t)(p0 + j) * n + i] : 0.0f;
#pragma unroll
    for (int j = kGqPanel - 1; j >= 0; --j) {
        if (j < nb) {
            float t = x[j];
#pragma unroll
            for (int m = j + 1; m < kGqPanel; ++m) t -= x[m] * vp[j][m];
            x[j] = t / vp[j][j];
        }
    }
#pragma unroll
    for (int j = 0; j < kGqPanel; ++j)
        if (j < nb) v[(int64_t)i * n + p0 + j] = x[j];
}

// H[i][j] -= sum_m V[i][p0 + m] V[j][p0 + m] on the lower-triangle 64 x 64 tiles of [0, p0)^2.
__global__ void __launch_bounds__(256) gptq_chol_syrk_kernel(float *__restrict__ h, int n, int p0,
                                                             int nb,
                                                             const float *__restrict__ v) {
    __shared__ float vi[kGqPanel][kGqPanel + 1], vj[kGqPanel][kGqPanel + 1];
    const int e = blockIdx.x;
    int ti = static_cast<int>((sqrtf(8.0f * static_cast<float>(e) + 1.0f) - 1.0f) * 0.5f);
    while (ti * (ti + 1) / 2 > e) --ti;
    while ((ti + 1) * (ti + 2) / 2 <= e) ++ti;
    const int tj = e - ti * (ti + 1) / 2;
    const int r0 = ti * kGqTile, c0 = tj * kGqTile;
    for (int q = threadIdx.x; q < kGqTile * kGqPanel; q += 256) {
        const int r = q / kGqPanel, m = q % kGqPanel;
        vi[r][m] = m < nb ? v[(int64_t)(r0 + r) * n + p0 + m] : 0.0f;
        vj[r][m] = m < nb ? v[(int64_t)(c0 + r) * n + p0 + m] : 0.0f;
    }
    __syncthreads();
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[4][4] = {};
#pragma unroll 8
    for (int m = 0; m < kGqPanel; ++m) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(vi[ty + 16 * a][m], vj[tx + 16 * b][m], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) h[(int64_t)(r0 + ty + 16 * a) * n + c0 + tx + 16 * b] -= acc[a][b];
}

// Back substitution inside the panel, one thread per column j >= p0: for k from the panel's last
// row back, R[i][j] -= V[i][k] / V[k][k] R[k][j] for the panel's rows i < k.
__global__ void __launch_bounds__(256) gptq_inv_panel_kernel(const float *__restrict__ v, int n,
                                                             int p0, int nb,
                                                             float *__restrict__ r) {
    __shared__ float f[kGqPanel][kGqPanel + 1];  // f[i][k] = V[p0 + i][p0 + k] / V[p0 + k][p0 + k]
    for (int e = threadIdx.x; e < kGqPanel * kGqPanel; e += 256) {
        const int i = e / kGqPanel, k = e % kGqPanel;
        f[i][k] = i < nb && k < nb && i < k
                      ? v[(int64_t)(p0 + i) * n + p0 + k] / v[(int64_t)(p0 + k) * n + p0 + k]
                      : 0.0f;
    }
    __syncthreads();
    const int j = p0 + blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    float x[kGqPanel];
#pragma unroll
    for (int i = 0; i < kGqPanel; ++i) x[i] = i < nb ? r[(int64_t)(p0 + i) * n + j] : 0.0f;
#pragma unroll
    for (int k = kGqPanel - 1; k >= 1; --k)
#pragma unroll
        for (int i = 0; i < k; ++i) x[i] -= f[i][k] * x[k];
#pragma unroll
    for (int i = 0; i < kGqPanel; ++i)
        if (i < nb) r[(int64_t)(p0 + i) * n + j] = x[i];
}

// Rows above the panel: R[i][j] -= sum_k V[i][p0 + k] / V[p0 + k][p0 + k] R[p0 + k][j],
// i < p0, j >= p0, 64 x 64 tiles.
__global__ void __launch_bounds__(256) gptq_inv_gemm_kernel(const float *__restrict__ v, int n,
                                                            int p0, int nb,
                                                            float *__restrict__ r) {
    __shared__ float fa[kGqTile][kGqPanel + 1], rb[kGqPanel][kGqTile + 1];
    const int r0 = blockIdx.y * kGqTile, c0 = p0 + blockIdx.x * kGqTile;
    for (int q = threadIdx.x; q < kGqTile * kGqPanel; q += 256) {
        const int i = q / kGqPanel, k = q % kGqPanel;
        fa[i][k] = r0 + i < p0 && k < nb
                       ? v[(int64_t)(r0 + i) * n + p0 + k] / v[(int64_t)(p0 + k) * n + p0 + k]
                       : 0.0f;
        const int kk = q / kGqTile, c = q % kGqTile;
        rb[kk][c] = kk < nb && c0 + c < n ? r[(int64_t)(p0 + kk) * n + c0 + c] : 0.0f;
    }
    __syncthreads();
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[4][4] = {};
#pragma unroll 8
    for (int k = 0; k < kGqPanel; ++k) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(fa[ty + 16 * a][k], rb[k][tx + 16 * b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = r0 + ty + 16 * a, j = c0 + tx + 16 * b;
            if (i < p0 && j < n) r[(int64_t)i * n + j] -= acc[a][b];
        }
}

// R = I (upper part used), and the final U = diag(V)^-1 R (rows scaled), zeros below the diagonal.
__global__ void __launch_bounds__(256) gptq_identity_kernel(float *__restrict__ r, int n) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<int64_t>(n) * n) return;
    r[e] = (e / n == e % n) ? 1.0f : 0.0f;
}

__global__ void __launch_bounds__(256) gptq_scale_rows_kernel(const float *__restrict__ v, int n,
                                                              float *__restrict__ u) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<int64_t>(n) * n) return;
    const int i = static_cast<int>(e / n), j = static_cast<int>(e % n);
    u[e] = j < i ? 0.0f : u[e] / v[(int64_t)i * n + i];
}

// w4_pack's statistics of one group of the current weights (pads are zeros of the group), and
// the code of one value; the same fp32 operations as the packing kernel's rule.
struct GroupQ {
    float s, z;
};

__device__ GroupQ group_stats(const float *__restrict__ row, int k0, int g, int d_in, int mode) {
    float amax = 0.0f, mx = 0.0f, mn = 0.0f;
    for (int t = 0; t < g; ++t) {
        const int k = k0 + t;
        const float r = k < d_in ? row[k] : 0.0f;
        const float a = fabsf(r);
        if (t == 0) {
            amax = a;
            mx = r;
            mn = r;
        } else {
            amax = a > amax ? a : amax;
            mx = r > mx ? r : mx;
            mn = r < mn ? r : mn;
        }
    }
    GroupQ q;
    if (mode == 0) {
        q.s = bf16_to_f32(f32_to_bf16(amax / 7.0f + 0.0f));
        q.z = 8.0f;
    } else {
        q.s = bf16_to_f32(f32_to_bf16((mx - mn) / 15.0f + 0.0f));
        float zf = 0.0f;
        if (q.s != 0.0f) zf = rintf(-mn / q.s) + 0.0f;
        q.z = bf16_to_f32(f32_to_bf16(zf));
    }
    return q;
}

__device__ __forceinline__ float code_of(float r, GroupQ q) {
    if (q.s == 0.0f) return q.z;
    return fminf(fmaxf(rintf(r / q.s + q.z), 0.0f), 15.0f);
}

// One block of 32 columns, four lanes per output row (lane part p holds columns 8p .. 8p + 7 in
// registers): group statistics at group starts (group starts fall on block starts, since groups
// are multiples of 32 columns), then the columns in order -- the owning lane takes the code, the
// error and e = err / U_cc, the row's four lanes share e and update their later columns.
// E[j][c] receives e for the trailing update; the codes go to qweight (pads of the last group
// too).
__global__ void __launch_bounds__(256) gptq_block_kernel(
    float *__restrict__ w, int d_out, int d_in, int64_t ldw, const float *__restrict__ u, int n,
    int b0, int g, int mode, uint8_t *__restrict__ qweight, int64_t row_bytes,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, int n_groups,
    float *__restrict__ ebuf, float *__restrict__ row_loss) {
    __shared__ float ub[kGqBlock][kGqBlock + 1];
    const int cols = max(0, min(kGqBlock, d_in - b0));  // 0: a block of the last group's pads
    for (int e = threadIdx.x; e < kGqBlock * kGqBlock; e += 256) {
        const int i = e / kGqBlock, c = e % kGqBlock;
        ub[i][c] = i < cols && c < cols ? u[(int64_t)(b0 + i) * n + b0 + c] : 0.0f;
    }
    __syncthreads();
    const int j = blockIdx.x * 64 + static_cast<int>(threadIdx.x >> 2);
    const int p = threadIdx.x & 3;
    if (j >= d_out) return;  // (a row's four lanes leave together)
    const int lane = threadIdx.x & (kWave - 1), base = lane & ~3;
    float *row = w + (int64_t)j * ldw;
    float wv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) wv[t] = 8 * p + t < cols ? row[b0 + 8 * p + t] : 0.0f;
    GroupQ q{0.0f, 8.0f};
    const int G0 = b0 / g;
    if (b0 % g != 0) {  // the block continues a group: its statistics are stored
        q.s = bf16_to_f32(scales[(int64_t)j * n_groups + G0]);
        q.z = mode == 0 ? 8.0f : bf16_to_f32(zeros[(int64_t)j * n_groups + G0]);
    } else {  // a group starts here: statistics of the current weights
        if (g == kGqBlock) {  // the group is this block, in the registers of the four lanes
            float amax = fabsf(wv[0]), mx = wv[0], mn = wv[0];
#pragma unroll
            for (int t = 1; t < 8; ++t) {
                amax = fmaxf(amax, fabsf(wv[t]));
                mx = fmaxf(mx, wv[t]);
                mn = fminf(mn, wv[t]);
            }
#pragma unroll
            for (int o = 1; o < 4; o <<= 1) {
                amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
                mn = fminf(mn, __shfl_xor(mn, o, kWave));
            }
            if (mode == 0) {
                q.s = bf16_to_f32(f32_to_bf16(amax / 7.0f + 0.0f));
                q.z = 8.0f;
            } else {
                q.s = bf16_to_f32(f32_to_bf16((mx - mn) / 15.0f + 0.0f));
                float zf = 0.0f;
                if (q.s != 0.0f) zf = rintf(-mn / q.s) + 0.0f;
                q.z = bf16_to_f32(f32_to_bf16(zf));
            }
        } else {  // the group reaches past the block: its columns in memory are current
            q = group_stats(row, b0, g, d_in, mode);
        }
        if (p == 0) {
            scales[(int64_t)j * n_groups + G0] = static_cast<uint16_t>(f32_to_bf16(q.s));
            if (mode != 0) zeros[(int64_t)j * n_groups + G0] = static_cast<uint16_t>(f32_to_bf16(q.z));
        }
    }
    float loss = 0.0f;
    uint32_t packed = 0u;
#pragma unroll
    for (int c = 0; c < kGqBlock; ++c) {
        const int owner = c >> 3, t = c & 7;
        float e = 0.0f;
        if (p == owner) {
            if (c < cols) {
                const float code = code_of(wv[t], q);
                const float qv = q.s * (code - q.z);
                const float err = wv[t] - qv;
                const float d = ub[c][c];
                loss += 0.5f * (err * err) / (d * d);
                e = err / d;
                ebuf[(int64_t)j * kGqBlock + c] = e;
                packed |= static_cast<uint32_t>(code) << (4 * t);
            } else {
                ebuf[(int64_t)j * kGqBlock + c] = 0.0f;
                packed |= static_cast<uint32_t>(code_of(0.0f, q)) << (4 * t);
            }
        }
        e = __shfl(e, base + owner, kWave);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
            if (8 * p + tt > c) wv[tt] -= e * ub[c][8 * p + tt];
    }
    *reinterpret_cast<uint32_t *>(qweight + (int64_t)j * row_bytes + b0 / 2 + 4 * p) = packed;
#pragma unroll
    for (int o = 1; o < 4; o <<= 1) loss += __shfl_xor(loss, o, kWave);
    if (row_loss && p == 0) row_loss[j] = (b0 == 0 ? 0.0f : row_loss[j]) + loss;
}

// Trailing update: W[:, c0:] -= E U[b0:b0+32, c0:], 64 x 64 tiles of W (rows x columns).
__global__ void __launch_bounds__(256) gptq_trail_kernel(float *__restrict__ w, int d_out,
                                                         int d_in, int64_t ldw,
                                                         const float *__restrict__ u, int n,
                                                         int b0, const float *__restrict__ ebuf) {
    __shared__ float es[kGqTile][kGqBlock + 1], us[kGqBlock][kGqTile + 1];
    const int c0 = b0 + kGqBlock + blockIdx.x * kGqTile, r0 = blockIdx.y * kGqTile;
    for (int e = threadIdx.x; e < kGqTile * kGqBlock; e += 256) {
        const int r = e / kGqBlock, c = e % kGqBlock;
        es[r][c] = r0 + r < d_out ? ebuf[(int64_t)(r0 + r) * kGqBlock + c] : 0.0f;
        const int i = e / kGqTile, cc = e % kGqTile;
        us[i][cc] = c0 + cc < d_in && b0 + i < d_in ? u[(int64_t)(b0 + i) * n + c0 + cc] : 0.0f;
    }
    __syncthreads();
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    float acc[4][4] = {};
#pragma unroll 8
    for (int i = 0; i < kGqBlock; ++i) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(es[ty + 16 * a][i], us[i][tx + 16 * b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = r0 + ty + 16 * a, c = c0 + tx + 16 * b;
            if (r < d_out && c < d_in) w[(int64_t)r * ldw + c] -= acc[a][b];
        }
}

__global__ void __launch_bounds__(256) gptq_dead_kernel(float *__restrict__ w, int d_out, int d_in,
                                                        int64_t ldw,
                                                        const uint8_t *__restrict__ dead) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<int64_t>(d_out) * d_in) return;
    const int c = static_cast<int>(e % d_in);
    if (dead[c]) w[(e / d_in) * ldw + c] = 0.0f;
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

}  // namespace

hipError_t launch_gptq_hessian(const uint16_t *x, int64_t N, int64_t d_in, int64_t ldx, float *h,
                               hipStream_t stream) {
    const unsigned t = static_cast<unsigned>((d_in + kGqTile - 1) / kGqTile);
    hipLaunchKernelGGL(gptq_hessian_kernel, dim3(t, t), dim3(256), 0, stream, x,
                       static_cast<int>(N), static_cast<int>(d_in), ldx,
                       2.0f / static_cast<float>(N), h);
    return hipGetLastError();
}

hipError_t launch_gptq_factor(float *h, int64_t d_in, float alpha, float *u, float *v,
                              uint8_t *dead, hipStream_t stream) {
    const int n = static_cast<int>(d_in);
    hipLaunchKernelGGL(gptq_prepare_kernel, dim3(1), dim3(1024), 0, stream, h, n, alpha, dead);
    const int last = (n - 1) / kGqPanel * kGqPanel;
    // reverse Cholesky H = V V^T, panel by panel from the last
    for (int p0 = last; p0 >= 0; p0 -= kGqPanel) {
        const int nb = std::min(kGqPanel, n - p0);
        hipLaunchKernelGGL(gptq_chol_diag_kernel, dim3(1), dim3(kGqPanel), 0, stream, h, n, p0,
                           nb, v);
        if (p0 > 0) {
            hipLaunchKernelGGL(gptq_chol_trsm_kernel, dim3(blocks_for(p0)), dim3(256), 0, stream,
                               h, n, p0, nb, v);
            const int t = p0 / kGqTile;
            hipLaunchKernelGGL(gptq_chol_syrk_kernel, dim3(static_cast<unsigned>(t * (t + 1) / 2)),
                               dim3(256), 0, stream, h, n, p0, nb, v);
        }
    }
    // U = V^-1: R = diag(V) U by block back substitution from the last panel, then the rows
    // scaled
    hipLaunchKernelGGL(gptq_identity_kernel, dim3(blocks_for((int64_t)n * n)), dim3(256), 0,
                       stream, u, n);
    for (int p0 = last; p0 >= 0; p0 -= kGqPanel) {
        const int nb = std::min(kGqPanel, n - p0);
        hipLaunchKernelGGL(gptq_inv_panel_kernel, dim3(blocks_for(n - p0)), dim3(256), 0, stream,
                           v, n, p0, nb, u);
        if (p0 > 0)
            hipLaunchKernelGGL(gptq_inv_gemm_kernel,
                               dim3(static_cast<unsigned>((n - p0 + kGqTile - 1) / kGqTile),
                                    static_cast<unsigned>((p0 + kGqTile - 1) / kGqTile)),
                               dim3(256), 0, stream, v, n, p0, nb, u);
    }
    hipLaunchKernelGGL(gptq_scale_rows_kernel, dim3(blocks_for((int64_t)n * n)), dim3(256), 0,
                       stream, v, n, u);
    return hipGetLastError();
}

hipError_t launch_gptq_quantize(float *w, int64_t d_out, int64_t d_in, int64_t ldw,
                                const float *u, const uint8_t *dead, int64_t span, int mode,
                                uint8_t *qweight, uint16_t *scales, uint16_t *zeros,
                                int64_t n_groups, int64_t k_pad, float *ebuf, float *row_loss,
                                hipStream_t stream) {
    const int n = static_cast<int>(d_in);
    if (dead)
        hipLaunchKernelGGL(gptq_dead_kernel, dim3(blocks_for(d_out * d_in)), dim3(256), 0, stream,
                           w, static_cast<int>(d_out), n, ldw, dead);
    for (int b0 = 0; b0 < k_pad; b0 += kGqBlock) {  // (blocks past d_in write pad codes)
        hipLaunchKernelGGL(gptq_block_kernel, dim3(static_cast<unsigned>((d_out + 63) / 64)),
                           dim3(256), 0, stream, w,
                           static_cast<int>(d_out), n, ldw, u, n, b0, static_cast<int>(span), mode,
                           qweight, k_pad / 2, scales, zeros, static_cast<int>(n_groups), ebuf,
                           row_loss);
        const int rest = n - b0 - kGqBlock;
        if (rest > 0)
            hipLaunchKernelGGL(gptq_trail_kernel,
                               dim3(static_cast<unsigned>((rest + kGqTile - 1) / kGqTile),
                                    static_cast<unsigned>((d_out + kGqTile - 1) / kGqTile)),
                               dim3(256), 0, stream, w, static_cast<int>(d_out), n, ldw, u, n, b0,
                               ebuf);
    }
    return hipGetLastError();
}

}  // namespace w4
