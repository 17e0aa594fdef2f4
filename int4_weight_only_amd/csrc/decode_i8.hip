// decode_i8.hip -- W4A16 decode for one to four tokens on the int8 matrix cores (gfx950).
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "INT4 线性量化": w = s (q - z) per group;
// "融合INT4反量化与矩阵乘": the codes are consumed inside the product, no dequantized weight is
// written), [Orin] "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s" (sections
// "DP4A 做了什么": integer dot products of 4-bit codes against 8-bit operands with an int32
// accumulator; "INT32 accumulator 是否安全": the bound on the integer sums; "模型尺寸和 decode 的真实
// 瓶颈": decode time is the weight stream).
//
// The dot products of a group run on v_mfma_i32_16x16x64_i8 with the raw codes as one operand:
//   * activations: per token and 128-column group, X = rint(x 2^S) with max|x| 2^S in
//     [2^29, 2^30). X is exact for every |x| >= 2^-22 max|x| (bf16 carries 8 significant bits) and
//     off by at most 2^-30 max|x| otherwise, so an outlier channel in a group costs the other
//     columns of the group nothing measurable ([Infra] section 2.4: activation outliers sit in a
//     few channels). X is written as four signed base-256 digits: the bytes of
//     (X + 0x80808080) ^ 0x80808080 are d0..d3 in [-128, 127] with X = sum_p d_p 256^p. The
//     digits of token t are rows 4t .. 4t+3 of the MFMA's A operand, so one MFMA serves up to
//     four tokens;
//   * weights: a lane's 16 bytes (32 codes) of one row become two int8 operands, the low nibbles
//     (w & 0x0F0F0F0F) and the high nibbles ((w >> 4) & 0x0F0F0F0F) -- three VALU operations per
//     8 codes instead of a dequantization;
//   * two MFMAs per (16 rows x 128 columns) unit give sum c d_p of every digit plane p; the zero
//     point is removed per plane in int32 with the group's digit sums D_p:
//     T_p = sum (c - z) d_p = sum c d_p - z D_p, exactly, so padding columns (c = z) add exactly
//     nothing whatever x holds there; then sum (c - z) X = (T0 + 256 T1) + 65536 (T2 + 256 T3),
//     one fp32 rounding, scaled by s 2^-S.
// Zero points that are not integers of magnitude <= 256 (w4_pack never makes one) split into
// such an integer and a residual applied through the group's sum of X.
//
// Work split: a block of 8 waves owns a contiguous slice of rows, as 16-row tiles (the MFMA's
// N). The slice's (tile, group) units are dealt to the waves in pairs, units 2i and 2i+1 to wave
// i mod 8: a wave's two loads of a pair read whole 128-byte lines of 16 rows back to back, and
// the block's waves read neighbouring lines of the same rows at the same time. The
// waves' partial sums meet in LDS and are added in wave order (deterministic). The slice's
// scales (and zeros) are read once, coalesced, into LDS. Loads are raw buffer loads through
// descriptors covering exactly the slice: a row past the slice or a unit past a wave's share
// reads zeros without touching memory.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kI8Threads = 512;
constexpr int kI8Waves = kI8Threads / kWave;  // 8
constexpr int kI8Burst = 2;                   // loads a wave issues back to back
constexpr int kI8Ring = 2 * kI8Burst;         // units in flight per wave
constexpr int kI8MaxPasses = 8;               // activation loads per thread
constexpr int kI8TableLoads = 16;             // scale (and zero) loads per thread
constexpr int kI8MaxTiles = 16;               // 16-row tiles per block
constexpr int kI8MaxTokens = 4;
constexpr uint32_t kI8LdsLimit = 160 * 1024;

// LDS layout (bytes). a: the digit operands, [group][lo/hi][k-block q][row 0 .. 4M-1] x 16 B;
// stats: [token][group] x {D0, D1, D2, D3, 2^-S, sum X, -, -}; sct / zct: the slice's scales / zeros,
// [16 T rows][n_groups] x 2 B (rows past the slice are never written: only lanes whose results
// are dropped read them); red: [wave][tile][lane] fp32 partial sums.
struct I8Lds {
    uint32_t a, stats, sct, zct, red, total;
};

__host__ __device__ inline uint32_t align16(uint32_t v) { return (v + 15u) & ~15u; }

__host__ __device__ inline I8Lds i8_lds(int M, int n128, int n_groups, int T, bool zp) {
    I8Lds L;
    L.a = 0;
    L.stats = static_cast<uint32_t>(n128) * 2u * 4u * 4u * M * 16u;
    L.sct = L.stats + static_cast<uint32_t>(M) * n128 * 32u;
    const uint32_t table = align16(16u * T * n_groups * 2u);
    L.zct = L.sct + table;
    L.red = L.zct + (zp ? table : 0u);
    L.total = L.red + static_cast<uint32_t>(kI8Waves) * T * kWave * 4u;
    return L;
}

// 4x4 byte transpose: out[p] = byte p of w0, w1, w2, w3 (in that order, low to high).
__device__ __forceinline__ void transpose4(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                           uint32_t out[4]) {
    // t0 = (w0.0, w1.0, w0.2, w1.2), t1 = (w0.1, w1.1, w0.3, w1.3), likewise t2, t3 of w2, w3
    const uint32_t t0 = __builtin_amdgcn_perm(w1, w0, 0x06020400u);
    const uint32_t t1 = __builtin_amdgcn_perm(w1, w0, 0x07030501u);
    const uint32_t t2 = __builtin_amdgcn_perm(w3, w2, 0x06020400u);
    const uint32_t t3 = __builtin_amdgcn_perm(w3, w2, 0x07030501u);
    out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
    out[1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    out[2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// GLU: the gate of the MLP fused into the epilogue ([Lab5 基础]: FFN(x) = W_down [SiLU(W_gate x)
// (.) (W_up x)]; [Orin 后续还能继续优化什么] names this kernel boundary). The weight holds 2 d_out
// rows, gate rows [0, d_out) then up rows [d_out, 2 d_out) (bias likewise, if given); a block's
// slice is output rows [r0, r0 + R), and tile t holds gate rows r0 + 8t .. + 7 in its rows 0..7
// and the matching up rows in its rows 8..15, so a slice takes as many tiles as a plain slice of
// 2R rows. One descriptor spans the gate rows to the end of the up rows; a lane whose row lies
// past R reads zeros. The store combines lanes n and n + 8 of a tile: SiLU(g) u =
// g u / (1 + exp(-g)) in fp32.
template <int M, bool ZP, int XP, bool GLU>
__global__ void __launch_bounds__(kI8Threads) gemv_i8_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int d_out, int d_in, int row_bytes, int n128,
    int n_groups, int gshift, int rows_per_block, void *__restrict__ y, int64_t ldy,
    int out_f32) {
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r0 = blockIdx.x * rows_per_block;
    const int R = d_out - r0 < rows_per_block ? d_out - r0 : rows_per_block;  // >= 1
    const int T = GLU ? (R + 7) >> 3 : (R + 15) >> 4;
    const I8Lds L = i8_lds(M, n128, n_groups, T, ZP);
    // units are dealt in pairs: wave w takes units 16 m + 2 w and 16 m + 2 w + 1 (m = 0, 1, ...)
    // below U, so its two loads of a pair cover the same 128-byte lines
    const int U = T * n128;
    const int nu = (U - 2 * w > 0 ? (U - 2 * w - 1) / (2 * kI8Waves) + 1 : 0) +
                   (U - 2 * w - 1 > 0 ? (U - 2 * w - 2) / (2 * kI8Waves) + 1 : 0);
    const int n = lane & 15, q = lane >> 4;

    // ---- activation loads first (waiting for them must not wait for the weights): item
    // (t, G, j) is token t, group G, columns 8j .. 8j+7; 16 consecutive threads hold a group ----
    const int items = M * n128 * 16;
    const rsrc_t rx = make_rsrc(x, 0x7FFFFFFFu);  // the host keeps the offsets below 2^31
    uint4 xr[XP];  // XP passes: M * n128 * 16 <= XP * kI8Threads
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        const int it = tid + p * kI8Threads;
        const int gi = it >> 4;
        const int t = (gi >= n128) + (gi >= 2 * n128) + (gi >= 3 * n128);
        const int col = (gi - t * n128) * 128 + 8 * (it & 15);
        const uint32_t off = it < items && col < d_in
                                 ? static_cast<uint32_t>(((int64_t)t * ldx + col) * 2)
                                 : kOutOfRange;
        xr[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
    }
    // ---- the slice's scales (and zeros): R * n_groups contiguous bf16 values ----
    // (GLU: each half's table takes half of the loads)
    constexpr int TL = GLU ? kI8TableLoads / 2 : kI8TableLoads;
    const int nsc = R * n_groups;  // <= TL * kI8Threads (host)
    const int64_t up0 = GLU ? (int64_t)d_out : 0;  // first up row (GLU)
    const rsrc_t rs = make_rsrc(scales + (int64_t)r0 * n_groups, static_cast<uint32_t>(nsc) * 2u);
    const rsrc_t rz = make_rsrc(ZP ? zeros + (int64_t)r0 * n_groups : scales,
                                ZP ? static_cast<uint32_t>(nsc) * 2u : 0u);
    const rsrc_t rs2 = make_rsrc(scales + (up0 + r0) * n_groups,
                                 GLU ? static_cast<uint32_t>(nsc) * 2u : 0u);
    const rsrc_t rz2 = make_rsrc(ZP ? zeros + (up0 + r0) * n_groups : scales,
                                 GLU && ZP ? static_cast<uint32_t>(nsc) * 2u : 0u);
    uint32_t sv[TL], zv[ZP ? TL : 1], sv2[GLU ? TL : 1], zv2[GLU && ZP ? TL : 1];
#pragma unroll
    for (int i = 0; i < TL; ++i) {
        const uint32_t off = static_cast<uint32_t>(tid + i * kI8Threads) * 2u;  // past nsc: 0
        sv[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        if (ZP) zv[ZP ? i : 0] = __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0);
        if (GLU) {
            sv2[GLU ? i : 0] = __builtin_amdgcn_raw_buffer_load_b16(rs2, off, 0, 0);
            if (ZP) zv2[GLU && ZP ? i : 0] = __builtin_amdgcn_raw_buffer_load_b16(rz2, off, 0, 0);
        }
    }

    // ---- the weight ring: the k-th unit of this wave is u = 16 (k / 2) + 2w + k % 2 =
    // (tile t, group G); from k to k + 1, u grows by 1 (k even) or by 15 (k odd) ----
    const uint32_t rb = static_cast<uint32_t>(row_bytes);
    const rsrc_t rq = make_rsrc(qweight + (int64_t)r0 * row_bytes, static_cast<uint32_t>(R) * rb);
    // (GLU: the gate rows of the slice through the end of its up rows; the host keeps this below
    // 2^31 bytes)
    const rsrc_t rqg = make_rsrc(qweight + (int64_t)r0 * row_bytes,
                                 GLU ? static_cast<uint32_t>(up0 + R) * rb : 0u);
    const int jump = 2 * kI8Waves - 1;
    const int dt = jump / n128, dG = jump % n128;
    // offsets = a per-lane part (row n of the tile, k-block q) + a wave-uniform part (tile t,
    // group G); a unit past the wave's share gets bit 31 set: arithmetic, not a select -- a
    // select on a wave-uniform condition becomes a branch, and the waits after it drain the
    // ring. Such units may step past the last tile: t is clamped to T, so that every offset
    // stays below 2^31 before bit 31 is added (the host checks 16 (T + 1) rows) and the sum
    // cannot wrap around into the range.
    const uint32_t w_lane =
        GLU ? static_cast<uint32_t>(n < 8 ? n : up0 + n - 8) * rb + 16u * q
            : static_cast<uint32_t>(n) * rb + 16u * q;
    auto load = [&](int k, int t, int G, u32x4_t &dst) {
        const uint32_t past = static_cast<uint32_t>((nu - 1 - k) >> 31) << 31;
        const uint32_t tc = static_cast<uint32_t>(t < T ? t : T);
        if (GLU) {  // 8 rows per half per tile; a lane past the slice's R rows reads zeros
            const uint32_t wo =
                w_lane + ((8u * tc * rb + 64u * static_cast<uint32_t>(G)) | past);
            const bool in = static_cast<int>(8 * tc) + (n & 7) < R;
            dst = __builtin_amdgcn_raw_buffer_load_b128(rqg, in ? wo : kOutOfRange, 0, 0);
            return;
        }
        const uint32_t wo = w_lane + ((16u * tc * rb + 64u * static_cast<uint32_t>(G)) | past);
        dst = __builtin_amdgcn_raw_buffer_load_b128(rq, wo, 0, 0);
    };
    // (the ring depth is even, so slot p always holds a unit with k % 2 == p % 2)
    auto step = [&](int p, int &t, int &G) {
        if (p & 1) {
            t += dt;
            G += dG;
        } else {
            G += 1;
        }
        t = G >= n128 ? t + 1 : t;
        G = G >= n128 ? G - n128 : G;
    };
    static_assert(kI8Ring % 2 == 0, "the ring alternates the two units of a pair");
    u32x4_t ring[kI8Ring];
    int lk = 0, lt = (2 * w) / n128, lG = 2 * w - ((2 * w) / n128) * n128;
#pragma unroll
    for (int p = 0; p < kI8Ring; ++p) {
        phase_fence();
        load(lk, lt, lG, ring[p]);
        ++lk;
        step(p, lt, lG);
    }
    phase_fence();

    // ---- tables, partial sums ----
    uint16_t *sct = reinterpret_cast<uint16_t *>(lds + L.sct);
    uint16_t *zct = reinterpret_cast<uint16_t *>(lds + L.zct);
#pragma unroll
    for (int i = 0; i < TL; ++i) {
        const int idx = tid + i * kI8Threads;
        if (idx < nsc) {
            if (GLU) {  // slice row r sits in table row 16 (r / 8) + r % 8 (gate), + 8 (up)
                const int r = idx / n_groups;
                const int tg = (16 * (r >> 3) + (r & 7)) * n_groups + (idx - r * n_groups);
                const int tu = tg + 8 * n_groups;
                sct[tg] = static_cast<uint16_t>(sv[i]);
                sct[tu] = static_cast<uint16_t>(sv2[GLU ? i : 0]);
                if (ZP) {
                    zct[tg] = static_cast<uint16_t>(zv[ZP ? i : 0]);
                    zct[tu] = static_cast<uint16_t>(zv2[GLU && ZP ? i : 0]);
                }
            } else {
                sct[idx] = static_cast<uint16_t>(sv[i]);
                if (ZP) zct[idx] = static_cast<uint16_t>(zv[ZP ? i : 0]);
            }
        }
    }
    float *red = reinterpret_cast<float *>(lds + L.red);
    for (int i = tid; i < kI8Waves * T * kWave; i += kI8Threads) red[i] = 0.0f;

    // ---- activations -> digits (a branch that holds no load: waiting for the activation
    // loads leaves the weight ring in flight) ----
    const bool ragged = (d_in & 7) != 0;
#pragma unroll
    for (int p = 0; p < XP; ++p) {
        if (p * kI8Threads >= items) break;  // block-uniform
        const int it = tid + p * kI8Threads;
        if (it < items) {  // whole 16-thread groups (items is a multiple of 16)
            const int j = it & 15, gi = it >> 4;
            const int t = (gi >= n128) + (gi >= 2 * n128) + (gi >= 3 * n128);
            const int G = gi - t * n128;
            uint32_t u[4] = {xr[p].x, xr[p].y, xr[p].z, xr[p].w};
            if (__builtin_expect(ragged, 0)) {  // zero the columns at or past d_in
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int col = G * 128 + 8 * j + 2 * k;
                    u[k] &= col + 1 < d_in ? 0xFFFFFFFFu : (col < d_in ? 0x0000FFFFu : 0u);
                }
            }
            // largest magnitude of the group, on the bf16 bit patterns (monotone in |x|)
            uint32_t am = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t a = u[k] & 0x7FFF7FFFu;
                am = max(am, max(a & 0xFFFFu, a >> 16));
            }
            // over the group's 16 lanes, one DPP row: quad swaps, then the half-row and row
            // mirrors (cross-lane moves inside the VALU; LDS-routed shuffles held the prologue up)
            am = max(am, static_cast<uint32_t>(dpp_i<0xB1, 0xF, false>(static_cast<int>(am))));
            am = max(am, static_cast<uint32_t>(dpp_i<0x4E, 0xF, false>(static_cast<int>(am))));
            am = max(am, static_cast<uint32_t>(dpp_i<0x141, 0xF, false>(static_cast<int>(am))));
            am = max(am, static_cast<uint32_t>(dpp_i<0x140, 0xF, false>(static_cast<int>(am))));
            const float amax = __uint_as_float(am << 16);
            const bool finite = am < 0x7F80u;
            const int S = finite && amax > 0.0f ? 29 - ilogbf(amax) : 0;  // max|x| 2^S < 2^30
            // X_e = rint(x_e 2^S) (|X_e| < 2^30); its digits are the bytes of
            // (X_e + 0x80808080) ^ 0x80808080. (A non-finite group gives junk digits; its scale
            // 2^-S is NaN, so its rows come out NaN.)
            uint32_t D[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t bits = (e & 1) ? (u[e >> 1] & 0xFFFF0000u) : (u[e >> 1] << 16);
                const int X = static_cast<int>(__builtin_rintf(ldexpf(__uint_as_float(bits), S)));
                D[e] = (static_cast<uint32_t>(X) + 0x80808080u) ^ 0x80808080u;
            }
            // the lo operand bytes are the columns 8j + {0,2,4,6}, the hi ones 8j + {1,3,5,7}
            uint32_t dlo[4], dhi[4];
            transpose4(D[0], D[2], D[4], D[6], dlo);
            transpose4(D[1], D[3], D[5], D[7], dhi);
            const int ones = 0x01010101;
            int ds[4];
#pragma unroll
            for (int pl = 0; pl < 4; ++pl)
                ds[pl] = __builtin_amdgcn_sdot4(
                    static_cast<int>(dlo[pl]), ones,
                    __builtin_amdgcn_sdot4(static_cast<int>(dhi[pl]), ones, 0, false), false);
#pragma unroll
            for (int pl = 0; pl < 4; ++pl) {  // (the same DPP row reduction)
                ds[pl] += dpp_i<0xB1, 0xF, false>(ds[pl]);
                ds[pl] += dpp_i<0x4E, 0xF, false>(ds[pl]);
                ds[pl] += dpp_i<0x141, 0xF, false>(ds[pl]);
                ds[pl] += dpp_i<0x140, 0xF, false>(ds[pl]);
            }
            // lane (n, q) of B holds columns 32q .. 32q+31 of the group, bytes 4i .. 4i+3 of an
            // operand being columns 32q + 8i + 2b (+1): here q = j / 4, i = j % 4
            const int kq = j >> 2, ki = j & 3;
            uint32_t *ab = reinterpret_cast<uint32_t *>(lds + L.a);
            const int lo0 = (((G * 2 + 0) * 4 + kq) * 4 * M + 4 * t) * 4 + ki;  // in dwords
            const int hi0 = (((G * 2 + 1) * 4 + kq) * 4 * M + 4 * t) * 4 + ki;
#pragma unroll
            for (int pl = 0; pl < 4; ++pl) {
                ab[lo0 + 4 * pl] = dlo[pl];
                ab[hi0 + 4 * pl] = dhi[pl];
            }
            if (j == 0) {
                const float gsc = finite ? ldexpf(1.0f, -S) : __builtin_nanf("");
                const float sx = static_cast<float>(ds[0]) + 256.0f * static_cast<float>(ds[1]) +
                                 65536.0f * static_cast<float>(ds[2]) +
                                 16777216.0f * static_cast<float>(ds[3]);
                i32x4_t *sp = reinterpret_cast<i32x4_t *>(lds + L.stats + (t * n128 + G) * 32);
                sp[0] = i32x4_t{ds[0], ds[1], ds[2], ds[3]};
                sp[1] = i32x4_t{__float_as_int(gsc), __float_as_int(sx), 0, 0};
            }
        }
    }
    __syncthreads();

    // ---- the units ----
    // Lane (n, q) of the result holds D rows 4q .. 4q+3 of column n: token q's four digit-plane
    // sums of row n. A rows >= 4M feed only D rows that are never read, so their lanes read any
    // row (their own row modulo 4M), and lanes of tokens >= M read token 0's statistics (their
    // results are never stored).
    const uint32_t a_group = 2u * 4u * 4u * M * 16u;
    const uint32_t a_hi = 4u * 4u * M * 16u;
    const uint32_t a_lane = L.a + (static_cast<uint32_t>(q) * 4u * M + n % (4 * M)) * 16u;
    const uint32_t s_lane = L.stats + static_cast<uint32_t>(q < M ? q : 0) * n128 * 32u;
    const uint32_t c_lane = static_cast<uint32_t>(n) * n_groups;  // table index of row n
    const i32x4_t zero4 = {0, 0, 0, 0};
    float acc = 0.0f;
    int at = -1;  // the tile acc belongs to
    auto compute = [&](int t, int G, const u32x4_t &wv) {
        const uint32_t ao = a_lane + static_cast<uint32_t>(G) * a_group;
        const i32x4_t alo = *reinterpret_cast<const i32x4_t *>(lds + ao);
        const i32x4_t ahi = *reinterpret_cast<const i32x4_t *>(lds + ao + a_hi);
        const i32x4_t dsum =
            *reinterpret_cast<const i32x4_t *>(lds + s_lane + static_cast<uint32_t>(G) * 32u);
        const i32x4_t st =
            *reinterpret_cast<const i32x4_t *>(lds + s_lane + static_cast<uint32_t>(G) * 32u + 16u);
        const uint32_t ci = c_lane + static_cast<uint32_t>(16 * t * n_groups) +
                            (static_cast<uint32_t>(G) >> gshift);
        const uint32_t sbits = sct[ci];
        const i32x4_t blo = {static_cast<int>(wv.x & 0x0F0F0F0Fu), static_cast<int>(wv.y & 0x0F0F0F0Fu),
                             static_cast<int>(wv.z & 0x0F0F0F0Fu), static_cast<int>(wv.w & 0x0F0F0F0Fu)};
        const i32x4_t bhi = {static_cast<int>((wv.x >> 4) & 0x0F0F0F0Fu),
                             static_cast<int>((wv.y >> 4) & 0x0F0F0F0Fu),
                             static_cast<int>((wv.z >> 4) & 0x0F0F0F0Fu),
                             static_cast<int>((wv.w >> 4) & 0x0F0F0F0Fu)};
        i32x4_t d = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo, zero4, 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi, d, 0, 0, 0);
        int zi = 8;
        float zr = 0.0f;
        if (ZP) {
            const float z = bf16_to_f32(zct[ci]);
            const float zf = fminf(fmaxf(__builtin_rintf(z), -256.0f), 256.0f);
            zi = static_cast<int>(zf);
            zr = z - zf;
        }
        const int t0 = d[0] - zi * dsum[0], t1 = d[1] - zi * dsum[1];
        const int t2 = d[2] - zi * dsum[2], t3 = d[3] - zi * dsum[3];
        const int lo = t0 + (t1 << 8), hi = t2 + (t3 << 8);  // |T_p| <= 15 * 128 * 128: exact
        float f = fmaf(65536.0f, static_cast<float>(hi), static_cast<float>(lo));
        if (ZP) f = fmaf(-zr, __int_as_float(st[1]), f);
        const float sc = bf16_to_f32(sbits) * __int_as_float(st[0]);
        acc = t != at ? 0.0f : acc;
        at = t;
        acc = fmaf(sc, f, acc);
        red[(w * T + t) * kWave + lane] = acc;
    };
    int ck = 0, ct = (2 * w) / n128, cG = 2 * w - ((2 * w) / n128) * n128;
    // full rounds over the two halves of the ring: the half's kI8Burst units are computed, then
    // refilled with kI8Burst loads issued back to back (bursts of neighbouring lines keep the
    // DRAM pages busy; a refill trickling out one load per unit ran about 15% slower). Every
    // slot computed holds a unit of the share; the loads of a round may pass its end and read
    // zeros.
    while (ck + kI8Ring <= nu) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int p = h * kI8Burst; p < (h + 1) * kI8Burst; ++p) {
                compute(ct, cG, ring[p]);
                ++ck;
                step(p, ct, cG);
            }
            phase_fence();
#pragma unroll
            for (int p = h * kI8Burst; p < (h + 1) * kI8Burst; ++p) {
                load(lk, lt, lG, ring[p]);
                ++lk;
                step(p, lt, lG);
            }
            phase_fence();
        }
    }
    // the last nu - ck < kI8Ring units sit in slots 0 .. nu - ck - 1; nothing is loaded after
    // them, so the waits behind these wave-uniform branches hold up nothing
#pragma unroll
    for (int p = 0; p < kI8Ring - 1; ++p) {
        if (ck + p < nu) compute(ct, cG, ring[p]);
        step(p, ct, cG);
    }
    __syncthreads();

    // ---- partial sums of the 8 waves, in wave order ----
    for (int e = tid; e < T * kWave; e += kI8Threads) {
        const int t = e / kWave, l = e % kWave;
        if (GLU && (l & 15) >= 8) continue;  // up rows: combined by the lane 8 below
        float v = 0.0f;
#pragma unroll
        for (int ww = 0; ww < kI8Waves; ++ww) v += red[(ww * T + t) * kWave + l];
        float u = 0.0f;
        if (GLU) {
#pragma unroll
            for (int ww = 0; ww < kI8Waves; ++ww) u += red[(ww * T + t) * kWave + l + 8];
        }
        const int row = GLU ? 8 * t + (l & 15) : 16 * t + (l & 15), tk = l >> 4;
        if (tk < M && row < R) {
            const int gr = r0 + row;
            if (bias) v += bf16_to_f32(bias[gr]);
            if (GLU) {
                if (bias) u += bf16_to_f32(bias[up0 + gr]);
                v = v * u / (1.0f + expf(-v));  // SiLU(g) u
            }
            store_out(y, static_cast<int64_t>(tk) * ldy + gr, v, out_f32 != 0);
        }
    }
    // the ring's loads past the share are out of range (zeros, no memory traffic)
}

// Workgroups per CU: two for short rows; one for long rows, whose per-block activation
// preparation grows with the row.
int i8_blocks_per_cu(int64_t n128) { return n128 <= 32 ? 2 : 1; }

struct I8Plan {
    int blocks, rows_per_block, T;
};

// Rows per block: an even share of d_out over the blocks (a block may hold less than one full
// tile: its missing rows read zeros and cost no memory traffic), at most kI8MaxTiles tiles and
// at most as many rows as the prologue reads scales for. Every block gets the same number of
// rows, so that no compute unit carries two slices while others carry one.
// (glu: d_out counts output rows, each with a gate and an up row: 8 output rows per tile and
// half of the table loads for each of the two)
I8Plan plan_i8(int64_t d_out, int64_t n128, int64_t n_groups, bool glu = false) {
    I8Plan p{};
    const int halves = glu ? 2 : 1;
    const int64_t blocks = (int64_t)device_cu_count() * i8_blocks_per_cu(n128);
    int64_t rpb = (d_out + blocks - 1) / blocks;
    int64_t cap = (int64_t)kI8TableLoads / halves * kI8Threads / n_groups;
    if (cap > 16 * kI8MaxTiles / halves) cap = 16 * kI8MaxTiles / halves;
    if (rpb > cap) rpb = cap;
    if (rpb < 1) rpb = 1;
    const int rows_per_tile = 16 / halves;
    p.rows_per_block = static_cast<int>(rpb);
    p.blocks = static_cast<int>((d_out + rpb - 1) / rpb);
    p.T = static_cast<int>((rpb + rows_per_tile - 1) / rows_per_tile);
    return p;
}

template <int M, bool ZP, int XP, bool GLU>
hipError_t launch_i8_t(const uint16_t *x, int64_t ldx, const uint8_t *qweight,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, int64_t n_groups, int gshift,
                       void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    const int n128 = static_cast<int>(k_pad / 128);
    const I8Plan p = plan_i8(d_out, n128, n_groups, GLU);
    const size_t lds = i8_lds(M, n128, static_cast<int>(n_groups), p.T, ZP).total;
    hipLaunchKernelGGL((gemv_i8_kernel<M, ZP, XP, GLU>), dim3(p.blocks), dim3(kI8Threads), lds,
                       stream, x,
                       ldx, qweight, scales, zeros, bias, static_cast<int>(d_out),
                       static_cast<int>(d_in), static_cast<int>(k_pad / 2), n128,
                       static_cast<int>(n_groups), gshift, p.rows_per_block, y, ldy,
                       out_f32 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

// Which decode kernel serves a call. The library chooses by shape: the int8 kernel for one
// token on shapes where it measured faster -- at least 32 rows per compute unit and rows of at
// most 32 groups of 128 columns. A build with W4_TEST_HOOKS defined (the test library, never the
// product one) also exports w4_test_force_decode_path, so that the tests can run each kernel on
// shapes the choice gives to another: 1 = the int8 kernel wherever it applies, 2 = never it,
// 3 = the column-split kernel of w4_gemv_ws wherever it applies, 0 = the library's choice.
#ifdef W4_TEST_HOOKS
namespace {
int g_forced_path = 0;
}  // namespace
int gemv_path_override() { return g_forced_path == 1 ? 1 : (g_forced_path == 2 ? -1 : 0); }
bool split_forced() { return g_forced_path == 3; }
#else
int gemv_path_override() { return 0; }
bool split_forced() { return false; }
#endif

bool gemv_i8_preferred(int64_t M, int64_t d_out, int64_t k_pad) {
    const int path = gemv_path_override();
    if (path != 0) return path > 0;
    // one to three tokens on tall matrices of short rows (gate/up 37888 x 3584, graph replays:
    // 2 tokens 17.4 us here against 20.8 on the few-token MFMA kernel, 3 tokens 18.2 against 20.8,
    // 4 tokens even)
    return M <= 3 && d_out >= 32 * (int64_t)device_cu_count() && k_pad / 128 <= 32;
}

bool gemv_i8_supported(int64_t M, int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, int64_t ldx, bool glu) {
    if (M < 1 || M > kI8MaxTokens) return false;
    if (k_pad % 128 != 0 || d_in > k_pad || d_in > 65536) return false;
    // every 128-column group lies inside one quantization group
    if (n_groups != 1 && span != 128 && span != 256) return false;
    const int64_t n128 = k_pad / 128;
    if (M * n128 * 16 > (int64_t)kI8MaxPasses * kI8Threads) return false;
    const int64_t table_loads = glu ? kI8TableLoads / 2 : kI8TableLoads;  // per half
    if (d_out < 1 || d_out * (glu ? 2 : 1) > (int64_t(1) << 24) ||
        n_groups > table_loads * kI8Threads)
        return false;
    const I8Plan p = plan_i8(d_out, n128, n_groups, glu);
    if ((int64_t)p.rows_per_block * n_groups > table_loads * kI8Threads) return false;
    if (i8_lds(static_cast<int>(M), static_cast<int>(n128), static_cast<int>(n_groups), p.T,
               true).total > kI8LdsLimit)
        return false;
    // 31-bit offsets: the activations of the tile and the weight rows of a block (up to one
    // tile past the block's last, where the units past a wave's share are clamped)
    if (((M - 1) * ldx + k_pad) * 2 >= (int64_t)kOutOfRange) return false;
    // (glu: the slice's descriptor spans the gate rows to the end of its up rows)
    const int64_t rows_spanned = glu ? d_out + 8 * (p.T + 1) : 16 * (p.T + 1);
    return rows_spanned * (k_pad / 2) < (int64_t)kOutOfRange;
}

hipError_t launch_gemv_i8(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                          const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                          int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                          int64_t n_groups, void *y, int64_t ldy, bool out_f32, bool glu,
                          hipStream_t stream) {
    const int gshift = n_groups == 1 ? 30 : (span == 256 ? 1 : 0);
    const bool zp = zeros != nullptr;
    const int64_t items = M * (k_pad / 128) * 16;
    const int xp = items <= kI8Threads ? 1 : items <= 2 * kI8Threads ? 2 : items <= 4 * kI8Threads ? 4 : 8;
#define W4_I8_GLU(MV, ZPV, XPV)                                                                  \
    (glu ? launch_i8_t<MV, ZPV, XPV, true>(x, ldx, qweight, scales, zeros, bias, d_out, d_in,    \
                                           k_pad, n_groups, gshift, y, ldy, out_f32, stream)     \
         : launch_i8_t<MV, ZPV, XPV, false>(x, ldx, qweight, scales, zeros, bias, d_out, d_in,   \
                                            k_pad, n_groups, gshift, y, ldy, out_f32, stream))
#define W4_I8_ZP(MV, XPV) return zp ? W4_I8_GLU(MV, true, XPV) : W4_I8_GLU(MV, false, XPV);
#define W4_I8_CASE(MV)                                                                           \
    case MV:                                                                                     \
        if (xp == 1) W4_I8_ZP(MV, 1)                                                             \
        if (xp == 2) W4_I8_ZP(MV, 2)                                                             \
        if (xp == 4) W4_I8_ZP(MV, 4)                                                             \
        W4_I8_ZP(MV, 8)
    switch (M) {
        W4_I8_CASE(1)
        W4_I8_CASE(2)
        W4_I8_CASE(3)
        W4_I8_CASE(4)
        default:
            return hipErrorInvalidValue;
    }
#undef W4_I8_ZP
#undef W4_I8_CASE
#undef W4_I8_GLU
}

}  // namespace w4

#ifdef W4_TEST_HOOKS
extern "C" int w4_test_force_decode_path(int path) {
    if (path < 0 || path > 3) return 5;  // W4_ERR_RANGE
    w4::g_forced_path = path;
    return 0;
}
#endif
