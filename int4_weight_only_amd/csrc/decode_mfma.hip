// decode_mfma.hip -- W4A16 decode for a few tokens (2 <= M <= 64) on the fp16 matrix cores.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "Linear形状采样" and "Prefill和Decode分流":
// the small-M decode path reads every weight once per step for all tokens; "融合INT4反量化与矩阵乘":
// the weight is dequantized in registers inside the product), [Orin] "Jetson Orin AGX INT4 推理优化
// 实践：super 分支从 9 tok/s 到 24 tok/s" (section "模型尺寸和 decode 的真实瓶颈": y = W x + b, and
// decode time is the weight stream).
//
// Two kernels:
//   * xprep: the activations, once per call, into fp16 MFMA fragments in a workspace.  For each
//     token and 128-column chunk, a power-of-two exponent e is chosen so that the chunk's largest
//     |x| * 2^-e lies in [2^14, 2^15); bf16 carries 8 significant bits and fp16 11, so every
//     value down to 2^-17 of that range is exact (smaller ones are fp16 subnormals: absolute
//     error at most 2^-25 * 2^e).  The chunk's sum of x * 2^-e is kept for zero points that are
//     not small integers.
//   * the decode kernel: a persistent grid, one block per slice of d_out / (number of compute
//     units) output rows (two blocks per unit for slices above 96 rows), in tiles of 16 rows; the
//     waves of a block split the K chunks, and their
//     partial sums meet in LDS in a fixed order (deterministic).  Per chunk and tile a lane loads
//     16 bytes of one row (32 codes), dequantizes them to the exact integers (c - z) in fp16 with
//     the magic-number form ((w & 0x000F000F) | 0x64006400 = (1024 + c0, 1024 + c4), one packed
//     fp16 add or fma removes 1024 + z), and four v_mfma_f32_16x16x32_f16 multiply them with the
//     activation fragments: A = 16 tokens x 32 columns, B = 32 columns x 16 rows.  The fp32 result
//     of the chunk is scaled by s[row][group] * 2^e[token] and accumulated in fp32.
//
// Weight loads are raw buffer loads through a descriptor covering exactly the block's rows, so a
// row past the block or a chunk past the row reads zeros without touching memory; every load is
// unconditional and sits in a ring of P chunks in flight per wave. They use the default cache
// policy: a load covers one 64-byte half of 16 rows' lines and the same wave reads the other
// half next, which the streaming (non-temporal) hint made about 10% slower.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 128;        // columns per chunk (four 32-deep MFMAs)
constexpr int kTokTile = 16;       // tokens per MFMA tile
constexpr int kMaxWaves = 8;       // waves per decode block
constexpr int kPrepThreads = 256;  // 16 tokens x 16 column octets

// ---------------------------------------------------------------------------------------------
// Workspace layout (all offsets in bytes from its start; tt = token tile, c = chunk):
//   frag[tt][c][t][lane]  16 bytes: the 8 fp16 activations of MFMA t (0..3) for lane
//                         lane = 16 q + m: token 16 tt + m, columns 128 c + 32 q + 8 t + {0..7}
//                         in the order 0 4 1 5 2 6 3 7 (the order of the dequantized pairs)
//   expo[tt][c][16]       int32 exponent e of each token of the tile
//   xsum[tt][c][16]       fp32 sum of x * 2^-e over the chunk
// ---------------------------------------------------------------------------------------------
struct WsLayout {
    int64_t frag, expo, xsum, total;
};

WsLayout ws_layout(int64_t M, int64_t k_pad) {
    const int64_t tt = (M + kTokTile - 1) / kTokTile;
    const int64_t C = (k_pad + kChunk - 1) / kChunk;
    WsLayout L{};
    L.frag = 0;
    L.expo = tt * C * 4 * 64 * 16;
    L.xsum = L.expo + tt * C * kTokTile * 4;
    L.total = L.xsum + tt * C * kTokTile * 4;
    return L;
}

__global__ void __launch_bounds__(kPrepThreads) xprep_kernel(
    const uint16_t *__restrict__ x, int M, int64_t ldx, int d_in, int C, uint4 *__restrict__ frag,
    int *__restrict__ expo, float *__restrict__ xsum) {
    const int c = blockIdx.x, tt = blockIdx.y;
    const int tid = threadIdx.x;
    const int m = tid >> 4;   // token within the tile
    const int j = tid & 15;   // column octet within the chunk: j = 4 q + t
    const int token = tt * kTokTile + m;
    const int col = c * kChunk + 8 * j;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (token < M && col < d_in) raw = *reinterpret_cast<const uint4 *>(x + token * ldx + col);
    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t bits = (e & 1) ? (u[e >> 1] >> 16) : (u[e >> 1] & 0xFFFFu);
        v[e] = col + e < d_in ? bf16_to_f32(bits) : 0.0f;
        amax = fmaxf(amax, fabsf(v[e]));
    }
    // the 16 threads of a token are 16 consecutive lanes
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    const int ex = amax > 0.0f ? ilogbf(amax) - 14 : 0;
    _Float16 h[8];
    float sum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float s = ldexpf(v[e], -ex);
        h[e] = static_cast<_Float16>(s);
        sum += s;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sum += __shfl_xor(sum, o, kWave);
    const int q = j >> 2, t = j & 3;
    half8_t out = {h[0], h[4], h[1], h[5], h[2], h[6], h[3], h[7]};
    frag[((static_cast<int64_t>(tt) * C + c) * 4 + t) * 64 + q * 16 + m] =
        *reinterpret_cast<const uint4 *>(&out);
    if (j == 0) {
        expo[(static_cast<int64_t>(tt) * C + c) * kTokTile + m] = ex;
        xsum[(static_cast<int64_t>(tt) * C + c) * kTokTile + m] = sum;
    }
}

// One ring slot: the activation fragments, exponents (and sums) of a chunk, and T tiles of
// weights with their scales (and zero points).
template <int T, bool ZP>
struct Slot {
    uint32_t xa[4][4];
    uint32_t xe[4];
    uint32_t xs[4];
    uint32_t w[T][4];
    uint32_t s[T];
    uint32_t z[T];
};

// Exact fp16 (c - zi) pairs of the 8 codes of one packed dword, in the order
// (c0, c4), (c1, c5), (c2, c6), (c3, c7).  zlo = (1024 + zi) and zhi = (64 + zi) as fp16 pairs.
__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t zlo_neg, uint32_t zhi_neg) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const uint32_t w8 = w >> 8;
    const uint32_t p0 = and_or(w, 0x000F000Fu, 0x64006400u);
    const uint32_t p1 = and_or(w, 0x00F000F0u, 0x64006400u);
    const uint32_t p2 = and_or(w8, 0x000F000Fu, 0x64006400u);
    const uint32_t p3 = and_or(w8, 0x00F000F0u, 0x64006400u);
    const half2_t zl = __builtin_bit_cast(half2_t, zlo_neg);
    const half2_t zh = __builtin_bit_cast(half2_t, zhi_neg);
    const half2_t sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const half2_t v0 = __builtin_bit_cast(half2_t, p0) + zl;
    const half2_t v1 = __builtin_bit_cast(half2_t, p1) * sixteenth + zh;
    const half2_t v2 = __builtin_bit_cast(half2_t, p2) + zl;
    const half2_t v3 = __builtin_bit_cast(half2_t, p3) * sixteenth + zh;
    half8_t r = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    return r;
}

template <int T, int P, bool ZP>
__global__ void __launch_bounds__(kMaxWaves * kWave) gemv_mfma_kernel(
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias,
    const uint4 *__restrict__ frag, const int *__restrict__ expo, const float *__restrict__ xsum,
    int d_out, int row_bytes, int n_groups, int group_shift, int C, int M, int TT,
    int rows_per_block, void *__restrict__ y, int64_t ldy, int out_f32) {
    extern __shared__ floatx4_t red[];  // [W][T][64]
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int W = blockDim.x / kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r0 = blockIdx.x * rows_per_block;
    const int r1 = d_out < r0 + rows_per_block ? d_out : r0 + rows_per_block;
    const int nrows = r1 - r0;
    const int c0 = (C * w) / W, c1 = (C * (w + 1)) / W;  // this wave's chunks
    const int L = c1 - c0;
    const int n = lane & 15, q = lane >> 4;

    const rsrc_t rq = make_rsrc(qweight + static_cast<int64_t>(r0) * row_bytes,
                                static_cast<uint32_t>(nrows) * static_cast<uint32_t>(row_bytes));
    const uint32_t gbytes = static_cast<uint32_t>(nrows) * static_cast<uint32_t>(n_groups) * 2u;
    const rsrc_t rs = make_rsrc(scales + static_cast<int64_t>(r0) * n_groups, gbytes);
    const rsrc_t rz = make_rsrc(ZP ? zeros + static_cast<int64_t>(r0) * n_groups : scales,
                                ZP ? gbytes : 0u);
    const uint32_t frag_bytes = static_cast<uint32_t>(TT) * C * 4 * 64 * 16;
    const uint32_t tok_bytes = static_cast<uint32_t>(TT) * C * kTokTile * 4;
    const rsrc_t rf = make_rsrc(frag, frag_bytes);
    const rsrc_t re = make_rsrc(expo, tok_bytes);
    const rsrc_t rx = make_rsrc(xsum, tok_bytes);

    for (int tt = 0; tt < TT; ++tt) {
        const bool tok_ok = tt * kTokTile + n < M;  // this lane's activation row holds a token
        auto load = [&](int b, Slot<T, ZP> &S) {
            const int c = c0 + b;
            const bool ok = b < L;
            const uint32_t fbase = ((static_cast<uint32_t>(tt) * C + c) * 4) * 1024u + lane * 16u;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 v = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               rf, ok && tok_ok ? fbase + t * 1024u : kOutOfRange, 0, 0));
                S.xa[t][0] = v.x; S.xa[t][1] = v.y; S.xa[t][2] = v.z; S.xa[t][3] = v.w;
            }
            const uint32_t tbase = ((static_cast<uint32_t>(tt) * C + c) * kTokTile + 4 * q) * 4u;
            {
                const uint4 v = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(re, ok ? tbase : kOutOfRange, 0, 0));
                S.xe[0] = v.x; S.xe[1] = v.y; S.xe[2] = v.z; S.xe[3] = v.w;
            }
            if (ZP) {
                const uint4 v = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? tbase : kOutOfRange, 0, 0));
                S.xs[0] = v.x; S.xs[1] = v.y; S.xs[2] = v.z; S.xs[3] = v.w;
            }
            const uint32_t kb = static_cast<uint32_t>(c) * 64u + 16u * q;  // byte within the row
            const bool kok = ok && kb + 16u <= static_cast<uint32_t>(row_bytes);
            const uint32_t G = static_cast<uint32_t>(c) >> group_shift;
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const uint32_t row = 16u * i + n;
                const uint4 v = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               rq, kok ? row * row_bytes + kb : kOutOfRange, 0, 0));
                S.w[i][0] = v.x; S.w[i][1] = v.y; S.w[i][2] = v.z; S.w[i][3] = v.w;
                const uint32_t go = ok ? (row * n_groups + G) * 2u : kOutOfRange;
                S.s[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, go, 0, 0);
                if (ZP) S.z[i] = __builtin_amdgcn_raw_buffer_load_b16(rz, go, 0, 0);
            }
        };

        floatx4_t acc[T];
#pragma unroll
        for (int i = 0; i < T; ++i) acc[i] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

        auto compute = [&](const Slot<T, ZP> &S) {
            half8_t a[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                a[t] = __builtin_bit_cast(half8_t, make_uint4(S.xa[t][0], S.xa[t][1], S.xa[t][2],
                                                              S.xa[t][3]));
#pragma unroll
            for (int i = 0; i < T; ++i) {
                // zero point = integer zi (|zi| <= 1024, exact in the fp16 form) + residual zr
                uint32_t zlo = 0xE408E408u;  // -(1024 + 8) as an fp16 pair
                uint32_t zhi = 0xD480D480u;  // -(64 + 8)
                float zr = 0.0f;
                if (ZP) {
                    const float z = bf16_to_f32(S.z[i]);
                    float zi = __builtin_rintf(z);
                    zi = fminf(fmaxf(zi, -1024.0f), 1024.0f);
                    zr = z - zi;
                    const uint32_t hl = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-(1024.0f + zi)));
                    const uint32_t hh = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-(64.0f + zi)));
                    zlo = hl | (hl << 16);
                    zhi = hh | (hh << 16);
                }
                floatx4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], dequant8(S.w[i][t], zlo, zhi),
                                                               d, 0, 0, 0);
                const float sv = bf16_to_f32(S.s[i]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = ldexpf(sv, static_cast<int>(S.xe[r]));
                    float v = d[r];
                    if (ZP) v = fmaf(-zr, __uint_as_float(S.xs[r]), v);
                    acc[i][r] = fmaf(f, v, acc[i][r]);
                }
            }
        };

        Slot<T, ZP> ring[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            phase_fence();
            load(p, ring[p]);
        }
        phase_fence();
        // Slots past the wave's last chunk were loaded out of range (zeros): computing them adds
        // exactly 0, and leaving the computation unconditional keeps the loop free of branches
        // (after a skipped slot, the compiler would wait for its loads before reusing registers).
        int b = 0;
        do {
#pragma unroll
            for (int p = 0; p < P; ++p) {
                compute(ring[p]);
                phase_fence();
                load(b + p + P, ring[p]);
                phase_fence();
            }
            b += P;
        } while (b < L);

        // partial sums of the W waves meet in LDS; summed in wave order
#pragma unroll
        for (int i = 0; i < T; ++i) red[(w * T + i) * kWave + lane] = acc[i];
        __syncthreads();
        for (int e = tid; e < T * kWave; e += W * kWave) {
            floatx4_t v = red[e];
            for (int ww = 1; ww < W; ++ww) {
                const floatx4_t o = red[ww * T * kWave + e];
                v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
            }
            const int i = e / kWave, l = e % kWave;
            const int row = r0 + 16 * i + (l & 15);
            if (row < r1) {
                const float bv = bias ? bf16_to_f32(bias[row]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int token = tt * kTokTile + 4 * (l >> 4) + r;
                    if (token < M) store_out(y, static_cast<int64_t>(token) * ldy + row, v[r] + bv,
                                             out_f32 != 0);
                }
            }
        }
        __syncthreads();
    }
    // the ring's last loads (zeros, out of range) have no memory traffic; nothing else is pending
}

template <int T, int P, bool ZP>
hipError_t launch_t(const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                    const uint16_t *bias, const uint4 *frag, const int *expo, const float *xsum,
                    int d_out, int row_bytes, int n_groups, int group_shift, int C, int M, int TT,
                    int rows_per_block, int blocks, int W, void *y, int64_t ldy, bool out_f32,
                    hipStream_t stream) {
    const size_t lds = static_cast<size_t>(W) * T * kWave * sizeof(floatx4_t);
    hipLaunchKernelGGL((gemv_mfma_kernel<T, P, ZP>), dim3(blocks), dim3(W * kWave), lds, stream,
                       qweight, scales, zeros, bias, frag, expo, xsum, d_out, row_bytes, n_groups,
                       group_shift, C, M, TT, rows_per_block, y, ldy, out_f32 ? 1 : 0);
    return hipGetLastError();
}

template <bool ZP>
hipError_t launch_zp(int T, const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                     const uint16_t *bias, const uint4 *frag, const int *expo, const float *xsum,
                     int d_out, int row_bytes, int n_groups, int group_shift, int C, int M,
                     int TT, int rows_per_block, int blocks, int W, void *y, int64_t ldy,
                     bool out_f32, hipStream_t stream) {
#define W4_MFMA_CASE(TV, PV)                                                                     \
    case TV:                                                                                     \
        return launch_t<TV, PV, ZP>(qweight, scales, zeros, bias, frag, expo, xsum, d_out,     \
                                    row_bytes, n_groups, group_shift, C, M, TT, rows_per_block, \
                                    blocks, W, y, ldy, out_f32, stream);
    switch (T) {
        W4_MFMA_CASE(1, 4)
        W4_MFMA_CASE(2, 4)
        W4_MFMA_CASE(3, 2)
        W4_MFMA_CASE(4, 2)
        W4_MFMA_CASE(6, 2)
        default: return hipErrorInvalidValue;
    }
#undef W4_MFMA_CASE
}

// Tiles per block are rounded up to an instantiated count.
constexpr int kMaxTiles = 6;
int round_tiles(int t) {
    static const int kT[] = {1, 2, 3, 4, 6};
    for (int v : kT)
        if (t <= v) return v;
    return 0;
}

}  // namespace

bool gemv_mfma_supported(int64_t M, int64_t d_out, int64_t k_pad, int64_t span, int64_t n_groups) {
    if (M < 2 || M > 64) return false;
    // a group must cover whole 128-column chunks (128 or 256), or be the whole row
    if (n_groups != 1 && span != 128 && span != 256) return false;
    // 32-bit offsets within a block's rows
    (void)d_out;
    return int64_t(kMaxTiles * 16) * (k_pad / 2) < (int64_t(1) << 31);
}

size_t gemv_mfma_workspace_bytes(int64_t M, int64_t k_pad) {
    return static_cast<size_t>(ws_layout(M, k_pad).total);
}

hipError_t launch_gemv_mfma(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                            int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                            int64_t n_groups, void *y, int64_t ldy, bool out_f32, void *workspace,
                            hipStream_t stream) {
    const WsLayout WL = ws_layout(M, k_pad);
    char *ws = static_cast<char *>(workspace);
    uint4 *frag = reinterpret_cast<uint4 *>(ws + WL.frag);
    int *expo = reinterpret_cast<int *>(ws + WL.expo);
    float *xsum = reinterpret_cast<float *>(ws + WL.xsum);
    const int C = static_cast<int>((k_pad + kChunk - 1) / kChunk);
    const int TT = static_cast<int>((M + kTokTile - 1) / kTokTile);
    hipLaunchKernelGGL(xprep_kernel, dim3(C, TT), dim3(kPrepThreads), 0, stream, x,
                       static_cast<int>(M), ldx, static_cast<int>(d_in), C, frag, expo, xsum);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;

    // rows: one slice per compute unit with up to 8 waves; a slice of more than kMaxTiles tiles
    // is cut in two blocks of up to 4 waves each (registers bound the tiles per wave)
    const int cus = device_cu_count();
    int rows_per_block = static_cast<int>((d_out + cus - 1) / cus);
    int max_waves = kMaxWaves;
    if (rows_per_block > kMaxTiles * 16) {
        rows_per_block = static_cast<int>((d_out + 2 * cus - 1) / (2 * cus));
        if (rows_per_block > kMaxTiles * 16) rows_per_block = kMaxTiles * 16;
        max_waves = kMaxWaves / 2;
    }
    const int blocks = static_cast<int>((d_out + rows_per_block - 1) / rows_per_block);
    const int T = round_tiles((rows_per_block + 15) / 16);
    // waves: split the chunks evenly (largest W within 5% of an even split, else the best one)
    int W = 1;
    double best = 1e30;
    for (int cand = max_waves; cand >= 1; --cand) {
        if (cand > C) continue;
        const double waste = static_cast<double>((C + cand - 1) / cand) * cand / C;
        if (waste <= 1.05) { W = cand; break; }
        if (waste < best) { best = waste; W = cand; }
    }
    const int group_shift = n_groups == 1 ? 30 : (span == 256 ? 1 : 0);
    const int row_bytes = static_cast<int>(k_pad / 2);
    if (zeros)
        return launch_zp<true>(T, qweight, scales, zeros, bias, frag, expo, xsum,
                               static_cast<int>(d_out), row_bytes, static_cast<int>(n_groups),
                               group_shift, C, static_cast<int>(M), TT, rows_per_block, blocks, W,
                               y, ldy, out_f32, stream);
    return launch_zp<false>(T, qweight, scales, zeros, bias, frag, expo, xsum,
                            static_cast<int>(d_out), row_bytes, static_cast<int>(n_groups),
                            group_shift, C, static_cast<int>(M), TT, rows_per_block, blocks, W, y,
                            ldy, out_f32, stream);
}

}  // namespace w4
