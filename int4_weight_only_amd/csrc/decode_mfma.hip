// decode_mfma.hip -- W4A16 decode for a few tokens (2 <= M <= 64) on the fp16 matrix cores.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "Linear形状采样" and "Prefill和Decode分流":
// the small-M decode path reads every weight once per step for all tokens; "融合INT4反量化与矩阵乘":
// the weight is dequantized in registers inside the product), [Orin] "Jetson Orin AGX INT4 推理优化
// 实践：super 分支从 9 tok/s 到 24 tok/s" (section "模型尺寸和 decode 的真实瓶颈": y = W x + b, and
// decode time is the weight stream).
//
// One kernel, no workspace. A persistent grid gives each block a contiguous slice of d_out /
// (number of compute units) output rows, as T tiles of 16 rows; the waves of the block split the
// row's K range in pairs of 128-column chunks (a pair is one 128-byte line of each row), and each
// wave streams the (pair, tile) units of its range:
//   * activations: per pair, a lane (m, q) loads 64 bf16 values of token m (columns 32 q ..
//     32 q + 31 of each chunk) straight from x, and converts them to the fp16 operand of
//     v_mfma_f32_16x16x32_f16 (A = 16 tokens x 32 columns). Per token and pair a power of two
//     2^-e scales the values so that the pair's largest |x| lies in [2^14, 2^15); bf16 carries 8
//     significant bits and fp16 11, so every value down to 2^-17 of that maximum is exact (smaller
//     ones lose bits as fp16 subnormals: absolute error at most 2^-25 2^e). Each chunk of x is
//     converted once per block, by the wave that owns it, and never written back;
//   * weights: a unit is 16 rows x 256 columns, two 16-byte loads per lane that read both halves
//     of the rows' 128-byte lines back to back; the 32 codes of a load become the exact fp16
//     integers (c - z) with the magic-number form ((w & 0x000F000F) | 0x64006400 = (1024 + c0,
//     1024 + c4), one packed fp16 add or fma removes 1024 + z), and four MFMAs multiply them with
//     the activation operand;
//   * the chunks' fp32 results are scaled by s[row][group], added, scaled by 2^e[token] and
//     accumulated in fp32.
// A block's scales (and zero points, as the two fp16 pair constants the dequantization uses)
// are read once, coalesced, into an LDS table. The waves' partial sums meet in LDS and are added
// in wave order (deterministic).
//
// Loads are raw buffer loads: a row past the block, a unit past a wave's share or a column past
// the row end reads zeros without touching memory. Every load is unconditional; a unit or pair
// past the wave's share gets bit 31 of its offset set arithmetically (a select on a wave-uniform
// condition becomes a branch, and the waits after it would drain the ring).
#include <type_traits>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kTokThreads = 512;  // at most 8 waves per block
constexpr int kTokMaxWaves = kTokThreads / kWave;
constexpr int kTokTile = 16;      // tokens per MFMA tile
constexpr int kTokTableBatch = 12;  // table entries a thread loads before it uses them
constexpr int kTokEarlySlots = 1;   // ring slots loaded before the table is built
constexpr uint32_t kTokLdsLimit = 160 * 1024;
// Activation offset of a lane without a token: past the input (below 2^30, host-checked), and
// still below 2^32 with bit 31 added.
constexpr uint32_t kTokNoToken = 0x40000000u;

// Workgroup barrier for LDS-only dependencies, without a memory fence: the caller's LDS accesses
// are completed first (lgkmcnt(0)), but the weight loads of the ring stay in flight across it
// (a fenced barrier waits for every outstanding load).
__device__ __forceinline__ void tok_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS layout (bytes): table [16 T rows][n_groups | 1] entries -- symmetric: the fp32 scale; with zero
// points: {fp32 scale, fp16 pair -(1024 + zi), fp16 pair -(64 + zi), fp32 residual z - zi}
// (rows past the slice are never written: only lanes whose results are dropped read them); red
// [W][T][64] fp32 x 4 partial sums.
struct TokLds {
    uint32_t table, red, total;
};

__host__ __device__ inline uint32_t tok_align16(uint32_t v) { return (v + 15u) & ~15u; }

// Table rows are n_groups | 1 entries apart: with an odd stride the 16 rows a ds_read of one
// tile touches fall into different LDS banks (with n_groups = 28 they fell into two).
__host__ __device__ inline int tok_table_stride(int n_groups) { return n_groups | 1; }

__host__ __device__ inline TokLds tok_lds(int T, int n_groups, int W, bool zp) {
    TokLds L;
    L.table = 0;
    L.red = tok_align16(16u * T * tok_table_stride(n_groups) * (zp ? 16u : 4u));
    L.total = L.red + static_cast<uint32_t>(W) * T * kWave * 16u;
    return L;
}

// The masks and the fp16 exponent pattern of the unpack, held in VGPRs the compiler cannot see
// into: with them as literals it emits a separate AND and OR per dword (gfx950 has no literal
// operands in three-operand VALU encodings), with them in registers one v_and_or_b32.
struct DqMasks {
    uint32_t lo, hi, magic;
};

__device__ __forceinline__ DqMasks dq_masks() {
    DqMasks k{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm volatile("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));  // (no instruction is emitted)
    return k;
}

// Exact fp16 (c - zi) pairs of the 8 codes of one packed dword, in the order
// (c0, c4), (c1, c5), (c2, c6), (c3, c7).  zlo = -(1024 + zi) and zhi = -(64 + zi) as fp16 pairs.
__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t zlo_neg, uint32_t zhi_neg,
                                            const DqMasks &k) {
    // (plain C, not an inline-asm and_or: the compiler's hazard checks do not look into inline
    // asm, and an asm write scheduled right after an MFMA can land in that MFMA's source
    // registers before it has read them)
    const uint32_t w8 = w >> 8;
    const uint32_t p0 = (w & k.lo) | k.magic;
    const uint32_t p1 = (w & k.hi) | k.magic;
    const uint32_t p2 = (w8 & k.lo) | k.magic;
    const uint32_t p3 = (w8 & k.hi) | k.magic;
    const half2_t zl = as_half2(zlo_neg);
    const half2_t zh = as_half2(zhi_neg);
    const half2_t sixteenth = {static_cast<_Float16>(0.0625f), static_cast<_Float16>(0.0625f)};
    const half2_t v0 = as_half2(p0) + zl;
    const half2_t v1 = as_half2(p1) * sixteenth + zh;
    const half2_t v2 = as_half2(p2) + zl;
    const half2_t v3 = as_half2(p3) * sixteenth + zh;
    half8_t r = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
    return r;
}

// The activations of one pair for one lane: 2 chunks x 4 pieces of 8 bf16 values.
struct XRaw {
    u32x4_t v[2][4];
};

// The converted pair: MFMA operands, the factors 2^e of the tokens whose D rows this lane holds,
// and (for non-integer zero points) the sums of the scaled activations.
template <int GPC>
struct XOp {
    half8_t a[2][4];
    float p[4];
    floatx4_t sx[2];  // (one group per chunk only; with more, the units take the sums themselves)
};

// P: weight units in flight per wave; a unit's ring slot is a constant in a loop body of two
// pairs. Two units (4 KiB a wave) beyond two tiles: the waves are bound by the dequantization
// there, and a deeper ring only delays their first compute (C = 28, T = 10, 16 tokens: 21.0 us
// with 2, 22.6 with 4 or 5, 22.5-23.5 with 10). XR: pairs of activations in flight.
template <int T>
struct TokShape {
    static constexpr int P = T == 2 ? 4 : 2;
    static constexpr int XR = T == 1 ? 2 : 1;
    static_assert((2 * T) % P == 0, "ring slots must repeat within two pairs");
};

// A 4 x 4 transpose of dwords across the four 16-lane rows of a wave: on return, v[t] of row r
// holds what v[r] of row t held (two v_permlane32_swap, then two v_permlane16_swap).
__device__ __forceinline__ void row_transpose4(u32x4_t &v) {
    const auto a = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    v[0] = c[0];
    v[1] = c[1];
    v[2] = d[0];
    v[3] = d[1];
}

// GPC: quantization groups per 128-column chunk (1 for groups of 128, 256 or a whole row; 2 for
// 64; 4 for 32). With GPC > 1 a lane's loads are transposed across the four 16-lane rows so that
// each MFMA's 32 columns lie in one group: lane (n, q) of MFMA t holds columns 32 t + 8 q .. + 7.
template <int T, bool ZP, int GPC>
__global__ void __launch_bounds__(kTokThreads) gemv_tok_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int M, int d_in,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias, int d_out,
    int row_bytes, int n_groups, int gshift, int C, int rows_per_block, void *__restrict__ y,
    int64_t ldy, int out_f32) {
    constexpr int P = TokShape<T>::P;
    constexpr int XR = TokShape<T>::XR;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int W = blockDim.x / kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r0 = blockIdx.x * rows_per_block;
    const int R = d_out - r0 < rows_per_block ? d_out - r0 : rows_per_block;  // >= 1
    const int n = lane & 15, q = lane >> 4;
    const int npairs = (C + 1) >> 1;
    const int p0 = npairs * w / W;
    const int np = npairs * (w + 1) / W - p0;  // this wave's pairs
    const TokLds L = tok_lds(T, n_groups, W, ZP);

    const uint32_t rb = static_cast<uint32_t>(row_bytes);
    const rsrc_t rq = make_rsrc(qweight + (int64_t)r0 * row_bytes, static_cast<uint32_t>(R) * rb);
    // the activations' descriptor covers exactly the M x ldx input (the host keeps it below 2^31)
    const rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(M) * static_cast<uint32_t>(ldx) * 2u);

    // Offsets are a per-lane part, fixed for the whole kernel, plus a wave-uniform part passed
    // through an opaque scalar (otherwise the compiler keeps one lane-part-plus-tile-offset VGPR
    // per tile alive across the loop). A unit or pair past the wave's share has bit 31 set in the
    // uniform part (the host keeps every sum below 2^31 before that bit).
    auto uni = [](uint32_t v) {
        asm volatile("" : "+s"(v));
        return v;
    };

    // ---- weight units: unit (j, i) = pair pr = p0 + j of tile i; lane (n, q) reads row 16 i + n,
    // bytes 128 pr + 16 q (first chunk) and 128 pr + 64 + 16 q (second chunk). In a row's last,
    // partial pair the bytes past the row belong to the next row (or lie past the slice and read
    // zeros): their activations are zero, so they add exactly nothing ----
    const uint32_t w_lane = static_cast<uint32_t>(n) * rb + 16u * q;
    auto wload = [&](int j, int i, u32x4_t &lo, u32x4_t &hi) {
        const uint32_t past = static_cast<uint32_t>((np - 1 - j) >> 31) << 31;
        const uint32_t u = uni((16u * static_cast<uint32_t>(i) * rb +
                                128u * static_cast<uint32_t>(p0 + j)) | past);
        lo = __builtin_amdgcn_raw_buffer_load_b128(rq, w_lane + u, 0, 0);
        hi = __builtin_amdgcn_raw_buffer_load_b128(rq, w_lane + u + 64u, 0, 0);
    };

    // ---- activations of pair j for token tile tt: lane (m, q), token 16 tt + m, columns
    // 256 pr + 128 h + 32 q + 8 t .. + 7 (columns past d_in are zeroed after the load) ----
    auto xload = [&](int tt, int j, XRaw &X) {
        const uint32_t past = static_cast<uint32_t>((np - 1 - j) >> 31) << 31;
        const int token = tt * kTokTile + n;
        // (GPC > 1: piece t of a lane is columns 32 t + 8 q .. + 7 of the chunk, else 32 q + 8 t)
        constexpr uint32_t kLaneStep = GPC > 1 ? 16u : 64u, kPieceStep = GPC > 1 ? 64u : 16u;
        const uint32_t x_lane =
            token < M ? static_cast<uint32_t>(token) * static_cast<uint32_t>(ldx) * 2u + kLaneStep * q
                      : kTokNoToken;
        const uint32_t u = uni((512u * static_cast<uint32_t>(p0 + j)) | past);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                X.v[h][t] = __builtin_amdgcn_raw_buffer_load_b128(
                    rx, x_lane + u + static_cast<uint32_t>(256 * h) + kPieceStep * t, 0, 0);
    };

    XRaw xr[XR];
    u32x4_t rlo[P], rhi[P];
    auto prime_x = [&](int tt) {
#pragma unroll
        for (int s = 0; s < XR; ++s) {
            phase_fence();
            xload(tt, s, xr[s]);
        }
        phase_fence();
    };
    auto prime_w = [&](int a, int b) {  // ring slots [a, b)
#pragma unroll
        for (int s = a; s < b; ++s) {
            phase_fence();
            wload(s / T, s % T, rlo[s], rhi[s]);
        }
        phase_fence();
    };

    // this wave's partial sums, [T][64] fp32 x 4 in LDS (read and written once per unit)
    float4 *red = reinterpret_cast<float4 *>(lds + L.red);
    float4 *mine = red + w * T * kWave + lane;
    auto zero_mine = [&]() {
#pragma unroll
        for (int i = 0; i < T; ++i) mine[i * kWave] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    };

    // ---- scale / zero-point table of the slice, kTokTableBatch entries per thread at a time:
    // every load of a batch is issued before any is used ----
    const int nent = R * n_groups;
    const rsrc_t rs = make_rsrc(scales + (int64_t)r0 * n_groups, static_cast<uint32_t>(nent) * 2u);
    const rsrc_t rz = make_rsrc(ZP ? zeros + (int64_t)r0 * n_groups : scales,
                                ZP ? static_cast<uint32_t>(nent) * 2u : 0u);
    const int tstride = static_cast<int>(blockDim.x);
    uint32_t sv[kTokTableBatch], zv[ZP ? kTokTableBatch : 1];
    // entries e0, e0 + stride, ..., NB of them; past nent: out of range, zeros
    auto tload = [&](auto nb, int e0) {
#pragma unroll
        for (int b = 0; b < decltype(nb)::value; ++b) {
            const uint32_t off = static_cast<uint32_t>(e0 + b * tstride) * 2u;
            sv[b] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
            if (ZP) zv[ZP ? b : 0] = __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0);
        }
    };
    auto tstore = [&](auto nb, int e0) {
        const int ts = tok_table_stride(n_groups);
#pragma unroll
        for (int b = 0; b < decltype(nb)::value; ++b) {
            const int e = e0 + b * tstride;
            if (e >= nent) break;
            const int te = (e / n_groups) * ts + e % n_groups;  // its slot in the table
            const float s = bf16_to_f32(sv[b]);
            if (ZP) {
                const float z = bf16_to_f32(zv[ZP ? b : 0]);
                const float zi = fminf(fmaxf(__builtin_rintf(z), -1024.0f), 1024.0f);
                const float zr = z - zi;
                const uint32_t hl =
                    __builtin_bit_cast(uint16_t, static_cast<_Float16>(-(1024.0f + zi)));
                const uint32_t hh =
                    __builtin_bit_cast(uint16_t, static_cast<_Float16>(-(64.0f + zi)));
                const u32x4_t ent = {__float_as_uint(s), hl | (hl << 16), hh | (hh << 16),
                                     __float_as_uint(zr)};
                *reinterpret_cast<u32x4_t *>(lds + L.table + 16u * te) = ent;
            } else {
                *reinterpret_cast<float *>(lds + L.table + 4u * te) = s;
            }
        }
    };

    auto convert = [&](int j, const XRaw &X, XOp<GPC> &O) {
        const int colq = 256 * (p0 + j) + (GPC > 1 ? 8 : 32) * q;
        uint32_t u[2][16];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                u[h][4 * t + 0] = X.v[h][t].x;
                u[h][4 * t + 1] = X.v[h][t].y;
                u[h][4 * t + 2] = X.v[h][t].z;
                u[h][4 * t + 3] = X.v[h][t].w;
            }
        if (__builtin_expect(256 * (p0 + j + 1) > d_in, 0)) {  // zero the columns past d_in
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int col = colq + 128 * h + (GPC > 1 ? 32 : 8) * (k >> 2) + 2 * (k & 3);
                    u[h][k] &= col + 1 < d_in ? 0xFFFFFFFFu : (col < d_in ? 0x0000FFFFu : 0u);
                }
        }
        // largest magnitude of the pair for token m: bf16 and fp16 are both sign-magnitude with
        // magnitude bits monotone in |x|, so an fp16 maximum of the raw bf16 patterns and their
        // negations finds the largest |x| (one v_pk_maximum3_f16 per dword)
        half2_t m2 = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const half2_t v = as_half2(u[h][k]);
                m2 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m2, v), -v);
            }
        const uint32_t mb = as_u32(m2) & 0x7FFF7FFFu;
        uint32_t am = (mb & 0xFFFFu) > (mb >> 16) ? (mb & 0xFFFFu) : (mb >> 16);
        am = max(am, static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), 16, kWave)));
        am = max(am, static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), 32, kWave)));
        const float amax = __uint_as_float(am << 16);
        const int ex = amax > 0.0f ? ilogbf(amax) - 14 : 0;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                __builtin_amdgcn_sched_barrier(0);  // one piece at a time: bounded registers
                float f[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t d = u[h][4 * t + (e >> 1)];
                    const uint32_t bits = (e & 1) ? (d & 0xFFFF0000u) : (d << 16);
                    f[e] = ldexpf(__uint_as_float(bits), -ex);
                }
                // operand order (0, 4), (1, 5), (2, 6), (3, 7): the order of the dequantized pairs
                half8_t a;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const half2_t hp = __builtin_bit_cast(
                        half2_t, __builtin_amdgcn_cvt_pkrtz(f[k], f[k + 4]));
                    a[2 * k] = hp[0];
                    a[2 * k + 1] = hp[1];
                }
                O.a[h][t] = a;
            }
        // D lane (n, q) holds tokens 4 q .. 4 q + 3; their factors sit in lanes 4 q + r
        const float pm = ldexpf(1.0f, ex);
#pragma unroll
        for (int r = 0; r < 4; ++r) O.p[r] = __shfl(pm, 4 * q + r, kWave);
        if (ZP) {  // sums of the scaled activations, through a ones operand, for the residual
                   // zero points (with none, every residual is 0 and they subtract exactly nothing)
            const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                floatx4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (GPC == 1) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(O.a[h][t], ones, s, 0, 0, 0);
                }
                O.sx[h] = s;
            }
        }
    };

    // Load order: the first activations, the first table batch and the first K0 ring slots;
    // the first pair's activations are converted while the table is in flight, and the rest of
    // the ring is loaded once the table is back. (Behind the whole ring the table took 10 us at
    // C = 28, T = 10 on 256 slices: the streaming weight reads starve the scattered table reads.)
    constexpr int K0 = kTokEarlySlots < P ? kTokEarlySlots : P;
    using Batch = std::integral_constant<int, kTokTableBatch>;
    prime_x(0);
    tload(Batch{}, tid);
    phase_fence();
    prime_w(0, K0);
    zero_mine();
    XOp<GPC> O;  // the converted activations of the pair in work
    convert(0, xr[0], O);  // the first pair's, while the table is in flight
    tstore(Batch{}, tid);
    for (int e0 = tid + kTokTableBatch * tstride; e0 < nent; e0 += kTokTableBatch * tstride) {
        tload(Batch{}, e0);
        tstore(Batch{}, e0);
    }
    prime_w(K0, P);
    tok_lds_barrier();  // (the weight loads of the ring stay in flight)

    const int ts = tok_table_stride(n_groups);
    const uint32_t t_lane = static_cast<uint32_t>(n) * ts;  // table row of lane's row n
    const DqMasks dqk = dq_masks();
    auto compute = [&](int i, int j, const u32x4_t &wlo_in, const u32x4_t &whi_in,
                       const XOp<GPC> &O) {
        // every LDS read first (sums, the table entries), then the two chunks' MFMA chains
        // interleaved: they are independent, so neither waits for the other's results
        const float4 a4 = mine[i * kWave];
        u32x4_t wlo = wlo_in, whi = whi_in;
        if constexpr (GPC > 1) {  // piece t of lane (n, q): columns 32 t + 8 q .. + 7
            row_transpose4(wlo);
            row_transpose4(whi);
        }
        float acc[4] = {a4.x, a4.y, a4.z, a4.w};
        if constexpr (GPC == 1) {
            float sc[2];
            uint32_t zlo[2] = {0xE408E408u, 0xE408E408u};  // -(1024 + 8) as an fp16 pair
            uint32_t zhi[2] = {0xD480D480u, 0xD480D480u};  // -(64 + 8)
            float zr[2] = {0.0f, 0.0f};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                int G = (2 * (p0 + j) + h) >> gshift;
                G = G < n_groups ? G : n_groups - 1;  // past the last chunk: x is zero there
                const uint32_t e = t_lane + uni(static_cast<uint32_t>(16 * i * ts + G));
                if (ZP) {
                    const u32x4_t ent =
                        *reinterpret_cast<const u32x4_t *>(lds + L.table + 16u * e);
                    sc[h] = __uint_as_float(ent.x);
                    zlo[h] = ent.y;
                    zhi[h] = ent.z;
                    zr[h] = __uint_as_float(ent.w);
                } else {
                    sc[h] = *reinterpret_cast<const float *>(lds + L.table + 4u * e);
                }
            }
            floatx4_t d[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t wd = (h ? whi : wlo)[t];
                    d[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        O.a[h][t], dequant8(wd, zlo[h], zhi[h], dqk), d[h], 0, 0, 0);
                }
            // sum = s0 d0 + s1 d1 per token, then acc += 2^e sum
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v0 = d[0][r], v1 = d[1][r];
                if (ZP) {  // (zr = 0 unless the zero point is not an integer)
                    v0 = fmaf(-zr[0], O.sx[0][r], v0);
                    v1 = fmaf(-zr[1], O.sx[1][r], v1);
                }
                acc[r] = fmaf(O.p[r], fmaf(sc[1], v1, sc[0] * v0), acc[r]);
            }
        } else {
            // one chunk at a time: its GPC groups are GPC independent MFMA chains already
            constexpr int kPer = 4 / GPC;  // MFMA pieces per group
            float sum[4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float sc[GPC], zr[GPC];
                uint32_t zlo[GPC], zhi[GPC];
#pragma unroll
                for (int g = 0; g < GPC; ++g) {
                    zlo[g] = 0xE408E408u;
                    zhi[g] = 0xD480D480u;
                    zr[g] = 0.0f;
                    int G = (2 * (p0 + j) + h) * GPC + g;
                    G = G < n_groups ? G : n_groups - 1;  // past the last group: x is zero there
                    const uint32_t e = t_lane + uni(static_cast<uint32_t>(16 * i * ts + G));
                    if (ZP) {
                        const u32x4_t ent =
                            *reinterpret_cast<const u32x4_t *>(lds + L.table + 16u * e);
                        sc[g] = __uint_as_float(ent.x);
                        zlo[g] = ent.y;
                        zhi[g] = ent.z;
                        zr[g] = __uint_as_float(ent.w);
                    } else {
                        sc[g] = *reinterpret_cast<const float *>(lds + L.table + 4u * e);
                    }
                }
                floatx4_t d[GPC], sx[GPC];
                const half8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
                for (int g = 0; g < GPC; ++g) {
                    d[g] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
                    sx[g] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int g = t / kPer;
                    const uint32_t wd = (h ? whi : wlo)[t];
                    d[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        O.a[h][t], dequant8(wd, zlo[g], zhi[g], dqk), d[g], 0, 0, 0);
                    if (ZP)  // the group's sums of the scaled activations, for a residual zr
                        sx[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(O.a[h][t], ones, sx[g], 0,
                                                                       0, 0);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int g = 0; g < GPC; ++g) {
                        float v = d[g][r];
                        if (ZP) v = fmaf(-zr[g], sx[g][r], v);  // (zr = 0 for integer z)
                        sum[r] = (h == 0 && g == 0) ? sc[g] * v : fmaf(sc[g], v, sum[r]);
                    }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] = fmaf(O.p[r], sum[r], acc[r]);
        }
        mine[i * kWave] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    };

    const int TT = (M + kTokTile - 1) / kTokTile;
    for (int tt = 0; tt < TT; ++tt) {
        if (tt > 0) {  // the previous tile's sums have been read (barrier below)
            zero_mine();
            prime_x(tt);
            prime_w(0, P);
            convert(0, xr[0], O);
        }
        // bodies of two pairs: every unit and activation slot index is a constant
        int j = 0;
        for (; j + 2 <= np; j += 2) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                if (jj != 0 || j > 0) convert(j + jj, xr[jj % XR], O);  // (pair 0's is done)
                phase_fence();
                xload(tt, j + jj + XR, xr[jj % XR]);
                phase_fence();
#pragma unroll
                for (int i = 0; i < T; ++i) {
                    const int ul = jj * T + i;
                    const int s = ul % P;
                    compute(i, j + jj, rlo[s], rhi[s], O);
                    const int un = ul + P;
                    phase_fence();
                    wload(j + un / T, un % T, rlo[s], rhi[s]);
                    phase_fence();
                }
            }
        }
        // an odd last pair: its activations sit in slot 0 and its units in slots 0 .. T - 1
        // (j T is a multiple of P); nothing is loaded after them
        if (j < np) {
            if (j > 0) convert(j, xr[0], O);
#pragma unroll
            for (int i = 0; i < T; ++i) compute(i, j, rlo[i % P], rhi[i % P], O);
        }

        // ---- partial sums of the W waves, in wave order ----
        __syncthreads();
        for (int e = tid; e < T * kWave; e += W * kWave) {
            float4 v = red[e];
            for (int ww = 1; ww < W; ++ww) {
                const float4 o = red[ww * T * kWave + e];
                v.x += o.x;
                v.y += o.y;
                v.z += o.z;
                v.w += o.w;
            }
            const int i = e / kWave, l = e % kWave;
            const int row = 16 * i + (l & 15);
            if (row < R) {
                const int gr = r0 + row;
                const float bv = bias ? bf16_to_f32(bias[gr]) : 0.0f;
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int token = tt * kTokTile + 4 * (l >> 4) + r;
                    if (token < M)
                        store_out(y, static_cast<int64_t>(token) * ldy + gr, vv[r] + bv,
                                  out_f32 != 0);
                }
            }
        }
        __syncthreads();
    }
    // the ring's last loads (zeros, out of range) have no memory traffic; nothing else is pending
}

struct TokPlan {
    int blocks, rows_per_block, T, W;
    bool ok;
};

constexpr int kTokTiles[] = {1, 2, 3, 4, 5, 6, 8, 10, 12};
constexpr int kTokMaxT = 12;

int round_tok_tiles(int t) {
    for (int v : kTokTiles)
        if (t <= v) return v;
    return 0;
}

// Rows: one slice per compute unit (more slices when one would exceed the tile cap or the LDS);
// waves: the row's pairs split evenly (the most waves within 5% of an even split, else the best).
TokPlan plan_tok(int64_t d_out, int64_t k_pad, int64_t n_groups, bool zp) {
    TokPlan p{};
    const int64_t cus = device_cu_count();
    const int64_t C = (k_pad + 127) / 128;
    const int64_t npairs = (C + 1) / 2;
    int W = 1;
    if (npairs <= kTokMaxWaves) {
        W = static_cast<int>(npairs);
    } else {
        double best = 1e30;
        for (int cand = kTokMaxWaves; cand >= 4; --cand) {
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
        const int64_t blocks_target = cus * split;
        int64_t rpb = (d_out + blocks_target - 1) / blocks_target;
        if (rpb < 1) rpb = 1;
        const int T = round_tok_tiles(static_cast<int>((rpb + 15) / 16));
        if (T == 0 || T > kTokMaxT) continue;
        if (tok_lds(T, static_cast<int>(n_groups), W, zp).total > kTokLdsLimit) continue;
        p.rows_per_block = static_cast<int>(rpb);
        p.blocks = static_cast<int>((d_out + rpb - 1) / rpb);
        p.T = T;
        p.W = W;
        p.ok = true;
        return p;
    }
    p.ok = false;
    return p;
}

template <int T, bool ZP, int GPC>
hipError_t launch_tok_t(const TokPlan &p, const uint16_t *x, int64_t ldx, int64_t M, int64_t d_in,
                        const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                        const uint16_t *bias, int64_t d_out, int64_t k_pad, int64_t n_groups,
                        int gshift, void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    const size_t lds = tok_lds(T, static_cast<int>(n_groups), p.W, ZP).total;
    const int C = static_cast<int>((k_pad + 127) / 128);
    hipLaunchKernelGGL((gemv_tok_kernel<T, ZP, GPC>), dim3(p.blocks), dim3(p.W * kWave), lds, stream, x,
                       ldx, static_cast<int>(M), static_cast<int>(d_in), qweight, scales, zeros,
                       bias, static_cast<int>(d_out), static_cast<int>(k_pad / 2),
                       static_cast<int>(n_groups), gshift, C, p.rows_per_block, y, ldy,
                       out_f32 ? 1 : 0);
    return hipGetLastError();
}

template <bool ZP, int GPC>
hipError_t launch_tok_zp(const TokPlan &p, const uint16_t *x, int64_t ldx, int64_t M, int64_t d_in,
                         const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                         const uint16_t *bias, int64_t d_out, int64_t k_pad, int64_t n_groups,
                         int gshift, void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
#define W4_TOK_CASE(TV)                                                                          \
    case TV:                                                                                     \
        return launch_tok_t<TV, ZP, GPC>(p, x, ldx, M, d_in, qweight, scales, zeros, bias,      \
                                         d_out,                                                  \
                                         k_pad, n_groups, gshift, y, ldy, out_f32, stream);
    switch (p.T) {
        W4_TOK_CASE(1)
        W4_TOK_CASE(2)
        W4_TOK_CASE(3)
        W4_TOK_CASE(4)
        W4_TOK_CASE(5)
        W4_TOK_CASE(6)
        W4_TOK_CASE(8)
        W4_TOK_CASE(10)
        W4_TOK_CASE(12)
        default:
            return hipErrorInvalidValue;
    }
#undef W4_TOK_CASE
}

}  // namespace

bool gemv_mfma_supported(int64_t M, int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                         int64_t n_groups, int64_t ldx, bool zp) {
    if (M < 2 || M > 64 || d_out < 1 || d_in < 1) return false;
    // a group covers whole 128-column chunks (128 or 256), is the whole row, or divides a chunk
    // (32 or 64: the lanes' pieces are then transposed so that an MFMA stays in one group)
    if (n_groups != 1 && span != 32 && span != 64 && span != 128 && span != 256) return false;
    if (d_in > k_pad || k_pad % 32 != 0) return false;
    const TokPlan p = plan_tok(d_out, k_pad, n_groups, zp);
    if (!p.ok) return false;
    // 31-bit offsets: the weight rows of a block's tiles (plus a pair past the row), and the
    // activations of every token
    const int64_t C = (k_pad + 127) / 128;
    if (int64_t(16) * p.T * (k_pad / 2) + 128 * (C + 2) >= (int64_t)kOutOfRange) return false;
    return (M * ldx + 1024) * 2 < (int64_t)kTokNoToken;
}

hipError_t launch_gemv_mfma(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                            int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                            int64_t n_groups, void *y, int64_t ldy, bool out_f32,
                            hipStream_t stream) {
    const bool zp = zeros != nullptr;
    const TokPlan p = plan_tok(d_out, k_pad, n_groups, zp);
    if (!p.ok) return hipErrorInvalidValue;
    const int gshift = n_groups == 1 ? 30 : (span == 256 ? 1 : 0);
    const int gpc = n_groups == 1 || span >= 128 ? 1 : static_cast<int>(128 / span);
#define W4_TOK_GPC(ZPV, GV)                                                                       \
    return launch_tok_zp<ZPV, GV>(p, x, ldx, M, d_in, qweight, scales, zeros, bias, d_out, k_pad, \
                                  n_groups, gshift, y, ldy, out_f32, stream);
    if (zp) {
        if (gpc == 4) W4_TOK_GPC(true, 4)
        if (gpc == 2) W4_TOK_GPC(true, 2)
        W4_TOK_GPC(true, 1)
    }
    if (gpc == 4) W4_TOK_GPC(false, 4)
    if (gpc == 2) W4_TOK_GPC(false, 2)
    W4_TOK_GPC(false, 1)
#undef W4_TOK_GPC
}

}  // namespace w4
