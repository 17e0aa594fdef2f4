// decode_w4a8_mfma.hip -- W4A8 decode for several tokens (2 <= M <= 64) on the int8 matrix cores.
//
// Pages: [Orin] "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s" (sections
// "从 FP 线性层到 INT4 DP4A 的数学推导": y = s_W s_x sum (c - 8) q + b with int32 sums; "DP4A 做了什么";
// "INT32 accumulator 是否安全"), [Lab5] "Lab 5: Gemma4 端到端推理优化" (section "Prefill和Decode分流":
// the small-M decode path reads every weight once per step for all tokens).
//
// The streaming W4A8 kernel takes the tokens in tiles of at most four and reads the weights once
// per tile. This kernel reads them once for 16 tokens, on v_mfma_i32_16x16x64_i8:
//   * a persistent grid gives each block a contiguous slice of about d_out / (number of compute
//     units) rows, as T tiles of 16 rows; the block's waves split the row's 128-column chunks in
//     pairs (a pair is one 128-byte line of each row) and each wave streams its (pair, tile)
//     units, as the few-token W4A16 kernel does;
//   * weights: a unit is two 16-byte loads per lane (row 16 i + n of the tile, the lane's quarter
//     of both chunks of the pair); `w & 0x0F0F0F0F` and `(w >> 4) & 0x0F0F0F0F` are the even-
//     and odd-column codes as unsigned int8 operands, used as they are;
//   * activations: per pair, lane (m, q) loads the int8 q of token m at columns 32 q .. 32 q + 31
//     of each chunk and splits them into the even and odd columns (v_perm_b32), in the byte order
//     of the code operands;
//   * per unit four MFMAs add sum c q into the tile's int32 accumulators, which stay in registers
//     across the wave's pairs; per pair, four more with a ones operand give the tokens' sum q;
//   * the waves' int32 sums meet in LDS (exact, any order), and the epilogue computes
//     acc = sum c q - 8 sum q and y = (s_W s_x) acc (+ b), the arithmetic of the streaming kernel,
//     so the two give the same y bit for bit.
// Loads are raw buffer loads: a row past the block, a unit past a wave's share, a token past M or
// a column past the row end read zeros without touching memory; activation bytes at and past d_in
// are masked to zero (they also cancel whatever codes meet them).
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kQtThreads = 512;  // at most 8 waves per block
constexpr int kQtMaxWaves = kQtThreads / kWave;
constexpr int kQtTile = 16;      // tokens per MFMA tile
constexpr int kQtMaxT = 12;      // 16-row tiles per block at most
constexpr uint32_t kQtNoToken = 0x40000000u;  // activation offset of a lane without a token
// From this many tokens on the matrix-core kernel replaces the streaming kernel's tiles of four
// (C5 shapes, graph replays: 2 tokens 9.2 / 10.8 us against 9.6 / 12.4 us, 4 tokens 9.3 / 12.0
// against 12.5 / 23.5 us, 16 tokens 10.2 / 16.7 against 49 / 87 us)
constexpr int kW4A8TokMinM = 2;

// Units in flight per wave (a unit is 2 KiB of a wave's loads: 2 x 16 B per lane), each in a
// constant slot of a loop body of two pairs.
template <int T>
struct QtShape {
    static constexpr int P = (2 * T) % 4 == 0 ? 4 : 2;
    static_assert((2 * T) % P == 0, "ring slots must repeat within two pairs");
};

// The activations of one pair for one lane: 2 chunks x 32 int8 (two 16-byte pieces each).
struct QRaw {
    u32x4_t v[2][2];
};

// The pair as MFMA operands: even and odd columns of each chunk.
struct QOp {
    i32x4_t lo[2], hi[2];
};

template <int T>
__global__ void __launch_bounds__(kQtThreads) gemv_w4a8_tok_kernel(
    const int8_t *__restrict__ q, int64_t ldq, int M, int d_in, const float *__restrict__ s_x,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ s_w,
    const uint16_t *__restrict__ bias, int d_out, int row_bytes, int C, int rows_per_block,
    void *__restrict__ y, int64_t ldy, int out_f32, int32_t *__restrict__ acc_out) {
    constexpr int P = QtShape<T>::P;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int W = blockDim.x / kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r0 = blockIdx.x * rows_per_block;
    const int R = d_out - r0 < rows_per_block ? d_out - r0 : rows_per_block;  // >= 1
    const int n = lane & 15, qq = lane >> 4;
    const int npairs = (C + 1) >> 1;
    const int p0 = npairs * w / W;
    const int np = npairs * (w + 1) / W - p0;  // this wave's pairs (>= 1: W <= npairs)

    const uint32_t rb = static_cast<uint32_t>(row_bytes);
    const rsrc_t rw = make_rsrc(qweight + (int64_t)r0 * row_bytes, static_cast<uint32_t>(R) * rb);
    // (the host keeps M ldq below 2^30)
    const rsrc_t rq = make_rsrc(q, static_cast<uint32_t>(M) * static_cast<uint32_t>(ldq));

    // wave-uniform part of an offset, through an opaque scalar (see the W4A16 kernel)
    auto uni = [](uint32_t v) {
        asm volatile("" : "+s"(v));
        return v;
    };

    // ---- weight unit (j, i): pair p0 + j, tile i; lane (n, qq) reads row 16 i + n, bytes
    // 128 pr + 16 qq and 128 pr + 64 + 16 qq. Past the wave's share: bit 31, zeros. ----
    const uint32_t w_lane = static_cast<uint32_t>(n) * rb + 16u * qq;
    auto wload = [&](int j, int i, u32x4_t &lo, u32x4_t &hi) {
        const uint32_t past = static_cast<uint32_t>((np - 1 - j) >> 31) << 31;
        const uint32_t u = uni((16u * static_cast<uint32_t>(i) * rb +
                                128u * static_cast<uint32_t>(p0 + j)) | past);
        lo = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + u, 0, 0);
        hi = __builtin_amdgcn_raw_buffer_load_b128(rw, w_lane + u + 64u, 0, 0);
    };

    // ---- activations of pair j for token tile tt: lane (m, qq), token 16 tt + m, columns
    // 256 pr + 128 h + 32 qq .. + 31 ----
    auto qload = [&](int tt, int j, QRaw &X) {
        const uint32_t past = static_cast<uint32_t>((np - 1 - j) >> 31) << 31;
        const int token = tt * kQtTile + n;
        const uint32_t q_lane = token < M ? static_cast<uint32_t>(token) *
                                                    static_cast<uint32_t>(ldq) + 32u * qq
                                          : kQtNoToken;
        const uint32_t u = uni((256u * static_cast<uint32_t>(p0 + j)) | past);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                X.v[h][t] = __builtin_amdgcn_raw_buffer_load_b128(
                    rq, q_lane + u + static_cast<uint32_t>(128 * h + 16 * t), 0, 0);
    };

    // even / odd columns: operand byte 4 d + b is column 8 d + 2 b (+ 1 for odd) of the lane's 32,
    // the byte order of (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) over the lane's code dwords
    auto convert = [&](int j, const QRaw &X, QOp &O) {
        const int colq = 256 * (p0 + j) + 32 * qq;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t u[8];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                u[4 * t + 0] = X.v[h][t].x;
                u[4 * t + 1] = X.v[h][t].y;
                u[4 * t + 2] = X.v[h][t].z;
                u[4 * t + 3] = X.v[h][t].w;
            }
            if (__builtin_expect(256 * (p0 + j + 1) > d_in, 0)) {  // bytes at and past d_in
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int left = d_in - (colq + 128 * h + 4 * e);
                    u[e] &= left >= 4 ? 0xFFFFFFFFu : (left <= 0 ? 0u : (1u << (8 * left)) - 1u);
                }
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                O.lo[h][d] = static_cast<int>(__builtin_amdgcn_perm(u[2 * d + 1], u[2 * d], 0x06040200u));
                O.hi[h][d] = static_cast<int>(__builtin_amdgcn_perm(u[2 * d + 1], u[2 * d], 0x07050301u));
            }
        }
    };

    QRaw xr;
    u32x4_t rlo[P], rhi[P];
    i32x4_t acc[T];
    const i32x4_t zero4 = {0, 0, 0, 0};
    const i32x4_t ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

    auto compute = [&](int i, const u32x4_t &wlo, const u32x4_t &whi, const QOp &O) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4_t wd = h ? whi : wlo;
            i32x4_t blo, bhi;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                blo[d] = static_cast<int>(wd[d] & 0x0F0F0F0Fu);
                bhi[d] = static_cast<int>((wd[d] >> 4) & 0x0F0F0F0Fu);
            }
            acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(O.lo[h], blo, acc[i], 0, 0, 0);
            acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(O.hi[h], bhi, acc[i], 0, 0, 0);
        }
    };

    // LDS: the waves' sums [W][T][64] int32 x 4, then their token sums [W][64] int32 x 4
    i32x4_t *red = reinterpret_cast<i32x4_t *>(lds);
    i32x4_t *sred = red + W * T * kWave;

    const int TT = (M + kQtTile - 1) / kQtTile;
    for (int tt = 0; tt < TT; ++tt) {
        // prime: the first pair's activations, then the ring
        phase_fence();
        qload(tt, 0, xr);
        phase_fence();
#pragma unroll
        for (int s = 0; s < P; ++s) {
            phase_fence();
            wload(s / T, s % T, rlo[s], rhi[s]);
        }
        phase_fence();
#pragma unroll
        for (int i = 0; i < T; ++i) acc[i] = zero4;
        i32x4_t sq = zero4;  // this wave's sum q of the tokens whose D rows the lane holds

        int j = 0;
        for (; j + 2 <= np; j += 2) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                QOp O;
                convert(j + jj, xr, O);
                phase_fence();
                qload(tt, j + jj + 1, xr);
                phase_fence();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    sq = __builtin_amdgcn_mfma_i32_16x16x64_i8(O.lo[h], ones, sq, 0, 0, 0);
                    sq = __builtin_amdgcn_mfma_i32_16x16x64_i8(O.hi[h], ones, sq, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < T; ++i) {
                    const int ul = jj * T + i;
                    const int s = ul % P;
                    compute(i, rlo[s], rhi[s], O);
                    const int un = ul + P;
                    phase_fence();
                    wload(j + un / T, un % T, rlo[s], rhi[s]);
                    phase_fence();
                }
            }
        }
        if (j < np) {  // an odd last pair: its units sit in slots 0 .. T - 1 (j T is a multiple of P)
            QOp O;
            convert(j, xr, O);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                sq = __builtin_amdgcn_mfma_i32_16x16x64_i8(O.lo[h], ones, sq, 0, 0, 0);
                sq = __builtin_amdgcn_mfma_i32_16x16x64_i8(O.hi[h], ones, sq, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < T; ++i) compute(i, rlo[i % P], rhi[i % P], O);
        }

        // ---- the waves' sums, then the epilogue ----
#pragma unroll
        for (int i = 0; i < T; ++i) red[(w * T + i) * kWave + lane] = acc[i];
        sred[w * kWave + lane] = sq;
        __syncthreads();
        for (int e = tid; e < T * kWave; e += W * kWave) {
            const int l = e % kWave, i = e / kWave;
            i32x4_t a = red[e], s = sred[l];
            for (int ww = 1; ww < W; ++ww) {
                a += red[ww * T * kWave + e];
                s += sred[ww * kWave + l];
            }
            const int row = 16 * i + (l & 15);
            if (row < R) {
                const int gr = r0 + row;
                const float sw = bf16_to_f32(s_w[gr]);
                const float bv = bias ? bf16_to_f32(bias[gr]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int token = tt * kQtTile + 4 * (l >> 4) + r;
                    if (token < M) {
                        const int av = a[r] - 8 * s[r];
                        float v = (sw * s_x[token]) * static_cast<float>(av);
                        if (bias) v += bv;
                        store_out(y, static_cast<int64_t>(token) * ldy + gr, v, out_f32 != 0);
                        if (acc_out) acc_out[static_cast<int64_t>(token) * d_out + gr] = av;
                    }
                }
            }
        }
        __syncthreads();
    }
    // the ring's last loads (zeros, out of range) have no memory traffic; nothing else is pending
}

struct QtPlan {
    int blocks, rows_per_block, T, W;
    bool ok;
};

constexpr int kQtTiles[] = {1, 2, 3, 4, 5, 6, 8, 10, 12};

uint32_t qt_lds(int T, int W) { return static_cast<uint32_t>(W) * (T + 1) * kWave * 16u; }

// Rows: one slice per compute unit (more slices when one would exceed the tile cap); waves: the
// row's pairs split evenly (the most waves within 5% of an even split, else the best).
QtPlan plan_qt(int64_t d_out, int64_t k_pad) {
    QtPlan p{};
    const int64_t cus = device_cu_count();
    const int64_t C = (k_pad + 127) / 128;
    const int64_t npairs = (C + 1) / 2;
    int W = 1;
    if (npairs <= kQtMaxWaves) {
        W = static_cast<int>(npairs);
    } else {
        double best = 1e30;
        for (int cand = kQtMaxWaves; cand >= 4; --cand) {
            const double waste = static_cast<double>((npairs + cand - 1) / cand) * cand / npairs;
            if (waste <= 1.05) {
                W = cand;
                break;
            }
            if (waste < best) {
                best = waste;
                W = cand;
            }
        }
    }
    for (int64_t split = 1; split <= 64; split *= 2) {
        int64_t rpb = (d_out + cus * split - 1) / (cus * split);
        if (rpb < 1) rpb = 1;
        int T = 0;
        for (int v : kQtTiles)
            if ((rpb + 15) / 16 <= v) {
                T = v;
                break;
            }
        if (T == 0 || T > kQtMaxT) continue;
        p.rows_per_block = static_cast<int>(rpb);
        p.blocks = static_cast<int>((d_out + rpb - 1) / rpb);
        p.T = T;
        p.W = W;
        p.ok = true;
        return p;
    }
    return p;
}

template <int T>
hipError_t launch_qt_t(const QtPlan &p, const int8_t *q, int64_t ldq, int64_t M, int64_t d_in,
                       const float *s_x, const uint8_t *qweight, const uint16_t *s_w,
                       const uint16_t *bias, int64_t d_out, int64_t k_pad, void *y, int64_t ldy,
                       bool out_f32, int32_t *acc, hipStream_t stream) {
    const int C = static_cast<int>((k_pad + 127) / 128);
    hipLaunchKernelGGL((gemv_w4a8_tok_kernel<T>), dim3(p.blocks), dim3(p.W * kWave),
                       qt_lds(T, p.W), stream, q, ldq, static_cast<int>(M),
                       static_cast<int>(d_in), s_x, qweight, s_w, bias, static_cast<int>(d_out),
                       static_cast<int>(k_pad / 2), C, p.rows_per_block, y, ldy, out_f32 ? 1 : 0,
                       acc);
    return hipGetLastError();
}

}  // namespace

bool w4a8_tok_supported(int64_t M, int64_t d_out, int64_t d_in, int64_t k_pad, int64_t ldq) {
    if (M < kW4A8TokMinM || M > 64 || d_out < 1 || d_in < 1 || d_in > k_pad) return false;
    const QtPlan p = plan_qt(d_out, k_pad);
    if (!p.ok) return false;
    // 31-bit offsets: a block's weight rows (plus a pair past the row), and every token's q
    const int64_t C = (k_pad + 127) / 128;
    if (int64_t(16) * p.T * (k_pad / 2) + 128 * (C + 2) >= (int64_t)kOutOfRange) return false;
    return M * ldq + 512 < (int64_t)kQtNoToken;
}

hipError_t launch_w4a8_tok(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                           const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                           int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                           bool out_f32, int32_t *acc, hipStream_t stream) {
    const QtPlan p = plan_qt(d_out, k_pad);
    if (!p.ok) return hipErrorInvalidValue;
#define W4_QT_CASE(TV)                                                                          \
    case TV:                                                                                    \
        return launch_qt_t<TV>(p, q, ldq, M, d_in, s_x, qweight, s_w, bias, d_out, k_pad, y,   \
                               ldy, out_f32, acc, stream);
    switch (p.T) {
        W4_QT_CASE(1)
        W4_QT_CASE(2)
        W4_QT_CASE(3)
        W4_QT_CASE(4)
        W4_QT_CASE(5)
        W4_QT_CASE(6)
        W4_QT_CASE(8)
        W4_QT_CASE(10)
        W4_QT_CASE(12)
        default:
            return hipErrorInvalidValue;
    }
#undef W4_QT_CASE
}

}  // namespace w4
