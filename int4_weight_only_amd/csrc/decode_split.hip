// decode_split.hip -- W4A16 decode for a few tokens (2 <= M <= 64) with the reduction dimension
// split over workgroups, on the fp16 matrix cores (gfx950).
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "Linear形状采样" and "Prefill和Decode分流":
// the small-M decode path reads every weight once per step for all tokens; "融合INT4反量化与矩阵乘":
// the weight is dequantized in registers inside the product), [Orin] "Jetson Orin AGX INT4 推理优化
// 实践：super 分支从 9 tok/s 到 24 tok/s" (section "模型尺寸和 decode 的真实瓶颈": y = W x + b, and
// decode time is the weight stream).
//
// On matrices with few rows per compute unit (a transformer's q/k/v, o and down projections),
// a workgroup that owns whole rows needs the activations of every column for a small amount of
// weights: at 16 tokens the down projection's 14 rows per compute unit are 133 KB of codes
// against 606 KB of activations. Here the grid is (row slices) x (column slices): workgroup
// (r, s) owns 16 TB rows and the 128-column chunks [cb0, cb1) of slice s.
//   * activations: the workgroup converts its chunks of a 16-token tile once into LDS, as the
//     fp16 A operands of v_mfma_f32_16x16x32_f16 in lane order, each (token, chunk) scaled by a
//     power of two 2^-e that puts its largest |x| in [2^14, 2^15): bf16 carries 8 significant
//     bits and fp16 11, so every value down to 2^-17 of that maximum is exact. Every wave reads
//     them from LDS;
//   * weights: the waves split the rows (TW tiles of 16 rows each) and stream (chunk, tile)
//     units, one 16-byte load per lane (row n of the tile, 32 codes); the codes become the exact
//     fp16 integers (c - z) with the magic-number form ((w & 0x000F000F) | 0x64006400 =
//     (1024 + c0, 1024 + c4); one packed fp16 add or fma removes 1024 + z) and four MFMAs
//     multiply them with the chunk's activations. A wave's sums stay in registers;
//   * scaling: each group's fp32 result is scaled by s[row][group] 2^e[token][chunk];
//   * output: with one column slice the workgroup writes y (+ bias); otherwise it writes its
//     fp32 partial sums to a caller-provided workspace, and a second kernel adds the slices in
//     slice order (deterministic) and the bias. (Adding them in the last workgroup of each row
//     slice instead -- an arrival counter, device-scope fences -- measured 2-3x slower: every
//     fence writes back and invalidates the L2 of its XCD.)
// A workgroup's scales (and zero points, as the two fp16 pair constants the dequantization uses)
// are read once into an LDS table. Zero points that are not integers of magnitude <= 1024 split
// into that integer and a residual applied through the activations' sums.
// Weight loads are raw buffer loads through a descriptor covering exactly the workgroup's rows:
// a row past them reads zeros; a unit past a wave's share gets an offset outside the range
// (bit 31 set arithmetically), so every load is unconditional.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kSpThreads = 512;                  // 8 waves
constexpr int kSpWaves = kSpThreads / kWave;
constexpr int kSpRing = 8;                       // weight units (1 KiB each) in flight per wave
constexpr int kSpTableLoads = 8;                 // table entries per thread
constexpr int kSpTile = 16;                      // tokens per MFMA tile
constexpr int kSpReduceBatch = 16;               // partial-sum loads in flight per output
constexpr uint32_t kSpLdsLimit = 160 * 1024;
constexpr uint32_t kSpNoToken = 0x40000000u;     // activation offset of a lane past M

// Workgroup barrier for LDS-only dependencies, without a memory fence: the caller's LDS accesses
// are completed first (lgkmcnt(0)), but the weight loads of the ring stay in flight across it
// (a fenced barrier waits for every outstanding load).
__device__ __forceinline__ void sp_lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// LDS layout (bytes): xs [ncb][4 MFMAs][64 lanes] x 16 B (A operands); ex [ncb][16 tokens] fp32
// (2^e); sx [ncb][16 tokens] fp32 (sums of the scaled activations, for residual zero points);
// table [16 TB rows][ngb | 1] -- symmetric: fp32 scale; with zero points: {fp32 scale, fp16 pair
// -(1024 + zi), fp16 pair -(64 + zi), fp32 residual z - zi}; flags [16] (per wave: a residual
// zero point seen).
struct SpLds {
    uint32_t xs, ex, sx, table, flags, total;
};

__host__ __device__ inline SpLds sp_lds(int ncb, int TB, int ngb, bool zp) {
    SpLds L;
    L.xs = 0;
    L.ex = L.xs + static_cast<uint32_t>(ncb) * 4u * kWave * 16u;
    L.sx = L.ex + static_cast<uint32_t>(ncb) * kSpTile * 4u;
    L.table = L.sx + (zp ? static_cast<uint32_t>(ncb) * kSpTile * 4u : 0u);
    L.flags = L.table + ((16u * TB * static_cast<uint32_t>(ngb | 1) * (zp ? 16u : 4u) + 15u) & ~15u);
    L.total = L.flags + 16u * 4u;
    return L;
}

// The most quantization groups ncb consecutive chunks touch (chunk c lies in group c >> gshift).
__host__ __device__ inline int sp_groups(int ncb, int gshift) {
    return gshift >= 30 ? 1 : ((ncb + (1 << gshift) - 1) >> gshift) + 1;
}

// The unpack's masks and fp16 exponent pattern in VGPRs the compiler cannot see into: as
// literals they cost a separate AND and OR per dword (no literal operands in gfx950's
// three-operand VALU encodings), in registers one v_and_or_b32.
struct SpMasks {
    uint32_t lo, hi, magic;
};

__device__ __forceinline__ SpMasks sp_masks() {
    SpMasks k{0x000F000Fu, 0x00F000F0u, 0x64006400u};
    asm volatile("" : "+v"(k.lo), "+v"(k.hi), "+v"(k.magic));  // (no instruction is emitted)
    return k;
}

// Exact fp16 (c - zi) pairs of the 8 codes of one packed dword, in the order
// (c0, c4), (c1, c5), (c2, c6), (c3, c7).  zlo = -(1024 + zi) and zhi = -(64 + zi) as fp16 pairs.
// (plain C: the compiler's hazard checks do not look into inline asm, and an asm write placed
// right after an MFMA could land in that MFMA's source registers before it has read them)
__device__ __forceinline__ half8_t sp_dequant8(uint32_t w, uint32_t zlo_neg, uint32_t zhi_neg,
                                               const SpMasks &k) {
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

// max over the four lanes of a quad (lanes 4k .. 4k+3), through DPP quad permutes
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
    return v;
}
__device__ __forceinline__ float quad_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    return v;
}

// TW: 16-row tiles per wave (the workgroup holds 16 * 8 * TW rows); XK: activation items per
// thread (an item is 32 columns of one token of one chunk). A chunk lies inside one quantization
// group (groups of 128 or 256 columns, or one per row): the K axis of each of a chunk's MFMAs
// takes 8 columns from each 32-column quarter of the chunk.
template <int TW, bool ZP, int XK>
__global__ void __launch_bounds__(kSpThreads) gemv_split_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int M, int d_in,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, const uint16_t *__restrict__ bias, int d_out,
    int row_bytes, int n_groups, int gshift, int C, float *__restrict__ part,
    void *__restrict__ y, int64_t ldy, int out_f32) {
    constexpr int TB = TW * kSpWaves;  // tiles per workgroup
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int n = lane & 15, q = lane >> 4;
    const int r0 = blockIdx.x * 16 * TB;
    const int R = d_out - r0 < 16 * TB ? d_out - r0 : 16 * TB;  // >= 1
    const int S = gridDim.y, s = blockIdx.y;
    const int cb0 = C * s / S, cb1 = C * (s + 1) / S;
    const int ncb = cb1 - cb0;  // >= 1 (S <= C)
    // quantization groups of the slice: [gb0, gb0 + ngb)
    const int gb0 = cb0 >> gshift;
    const int ngb = ((cb1 - 1) >> gshift) - gb0 + 1;
    const int ts = ngb | 1;  // table row stride (odd: the 16 rows of a tile in different banks)
    const int ncb_max = (C + S - 1) / S;
    const SpLds L = sp_lds(ncb_max, TB, sp_groups(ncb_max, gshift), ZP);

    // ---- activation loads first (waiting for them must not wait for the weights): item it of
    // the tile is chunk ci = it / 64, token m = (it / 4) % 16, quarter q4 = it % 4: columns
    // 128 (cb0 + ci) + 32 q4 .. + 31 as 4 pieces of 8 ----
    const int items = ncb * 64;
    const rsrc_t rx = make_rsrc(x, static_cast<uint32_t>(M) * static_cast<uint32_t>(ldx) * 2u);
    uint4 xr[XK][4];
    auto xload = [&](int tt) {
#pragma unroll
        for (int k = 0; k < XK; ++k) {
            const int it = tid + k * kSpThreads;
            const int ci = it >> 6, m = (it >> 2) & 15, q4 = it & 3;
            const int token = tt * kSpTile + m;
            const int col0 = 128 * (cb0 + ci) + 32 * q4;
            const uint32_t row_off = token < M && it < items
                                         ? static_cast<uint32_t>(token) * static_cast<uint32_t>(ldx) * 2u
                                         : kSpNoToken;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int col = col0 + 8 * p;
                xr[k][p] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(
                               rx, col < d_in ? row_off + 2u * static_cast<uint32_t>(col) : kOutOfRange,
                               0, 0));
            }
        }
    };
    xload(0);

    // ---- the table's loads: entry e = (row e / ngb, group gb0 + e % ngb) ----
    const int nent = R * ngb;  // <= kSpTableLoads * kSpThreads (host)
    const rsrc_t rs = make_rsrc(scales + (int64_t)r0 * n_groups,
                                static_cast<uint32_t>(R) * static_cast<uint32_t>(n_groups) * 2u);
    const rsrc_t rz = make_rsrc(ZP ? zeros + (int64_t)r0 * n_groups : scales,
                                ZP ? static_cast<uint32_t>(R) * static_cast<uint32_t>(n_groups) * 2u : 0u);
    uint32_t sv[kSpTableLoads], zv[ZP ? kSpTableLoads : 1];
#pragma unroll
    for (int i = 0; i < kSpTableLoads; ++i) {
        const int e = tid + i * kSpThreads;
        const int row = e / ngb;
        const int g = gb0 + (e - row * ngb);
        const uint32_t off = e < nent ? static_cast<uint32_t>(row * n_groups + g) * 2u : kOutOfRange;
        sv[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
        if (ZP) zv[ZP ? i : 0] = __builtin_amdgcn_raw_buffer_load_b16(rz, off, 0, 0);
    }

    // ---- the weight ring: unit k of the wave is (chunk cb0 + k / TW, tile w TW + k % TW); lane
    // (n, q) reads row 16 tile + n, bytes 64 chunk + 16 q (columns 128 chunk + 32 q .. + 31).
    // In a partial last chunk the bytes past the row belong to the next row (or lie past the
    // workgroup's rows and read zeros): their activations are zero, so they add nothing ----
    const int NU = ncb * TW;
    const uint32_t rb = static_cast<uint32_t>(row_bytes);
    const rsrc_t rq = make_rsrc(qweight + (int64_t)r0 * row_bytes, static_cast<uint32_t>(R) * rb);
    const uint32_t w_lane = (16u * static_cast<uint32_t>(w * TW) + static_cast<uint32_t>(n)) * rb +
                            64u * static_cast<uint32_t>(cb0) + 16u * static_cast<uint32_t>(q);
    auto wload = [&](int k, u32x4_t &dst) {
        const int ci = k / TW, i = k - (k / TW) * TW;
        const uint32_t past = static_cast<uint32_t>((NU - 1 - k) >> 31) << 31;
        const uint32_t u = (16u * static_cast<uint32_t>(i) * rb + 64u * static_cast<uint32_t>(ci)) | past;
        dst = __builtin_amdgcn_raw_buffer_load_b128(rq, w_lane + u, 0, 0);
    };
    u32x4_t ring[kSpRing];
    auto prime = [&]() {
#pragma unroll
        for (int u = 0; u < kSpRing; ++u) {
            phase_fence();
            wload(u, ring[u]);
        }
        phase_fence();
    };
    // (the ring is primed after the activations are converted: issued together, the weight loads
    // delayed the activations by about as much as they saved; measured on the 3584 x 18944 down
    // projection at 16 tokens, 15.2 against 16.0 us)

    // ---- activations -> LDS ----
    auto convert = [&]() {
#pragma unroll
        for (int k = 0; k < XK; ++k) {
            if (k * kSpThreads >= items) break;  // workgroup-uniform
            const int it = tid + k * kSpThreads;
            const int ci = it >> 6, m = (it >> 2) & 15, q4 = it & 3;
            const int col0 = 128 * (cb0 + ci) + 32 * q4;
            uint32_t u[4][4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                u[p][0] = xr[k][p].x;
                u[p][1] = xr[k][p].y;
                u[p][2] = xr[k][p].z;
                u[p][3] = xr[k][p].w;
            }
            if (__builtin_expect(128 * (cb0 + ci + 1) > d_in, 0)) {  // zero the columns past d_in
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < 4; ++p)
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int col = col0 + 8 * p + 2 * d;
                        u[p][d] &= col + 1 < d_in ? 0xFFFFFFFFu : (col < d_in ? 0x0000FFFFu : 0u);
                    }
            }
            // largest magnitude of the token's chunk: bf16 magnitude bits are monotone in |x|
            u16x2_t m2 = {0, 0};
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, u[p][d] & 0x7FFF7FFFu));
            const uint32_t am = quad_max(m2[0] > m2[1] ? m2[0] : m2[1]);
            const float amax = __uint_as_float(am << 16);
            const int ex = amax > 0.0f ? ilogbf(amax) - 14 : 0;
            float psum = 0.0f;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // operand order (0, 4), (1, 5), (2, 6), (3, 7): the order of the dequantized pairs
                half8_t a;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const uint32_t d0 = u[p][kk >> 1], d1 = u[p][2 + (kk >> 1)];
                    const float f0 = ldexpf(__uint_as_float((kk & 1) ? (d0 & 0xFFFF0000u) : (d0 << 16)), -ex);
                    const float f1 = ldexpf(__uint_as_float((kk & 1) ? (d1 & 0xFFFF0000u) : (d1 << 16)), -ex);
                    const half2_t hp = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(f0, f1));
                    a[2 * kk] = hp[0];
                    a[2 * kk + 1] = hp[1];
                }
                if (it < items)  // (the quad's lanes share it < items: all four run the DPP sums)
                    *reinterpret_cast<half8_t *>(lds + L.xs + ((ci * 4 + p) * kWave + q4 * 16 + m) * 16u) = a;
                if (ZP) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        psum = __builtin_amdgcn_fdot2(half2_t{a[2 * kk], a[2 * kk + 1]},
                                                      half2_t{static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)},
                                                      psum, false);
                }
            }
            if (ZP) psum = quad_sum(psum);
            if (q4 == 0 && it < items) {
                reinterpret_cast<float *>(lds + L.ex)[ci * kSpTile + m] = ldexpf(1.0f, ex);
                if (ZP) reinterpret_cast<float *>(lds + L.sx)[ci * kSpTile + m] = psum;
            }
        }
    };
    convert();
    prime();

    // ---- table ----
    {
        int frac = 0;
#pragma unroll
        for (int i = 0; i < kSpTableLoads; ++i) {
            const int e = tid + i * kSpThreads;
            if (e < nent) {
                const int row = e / ngb;
                const int te = row * ts + (e - row * ngb);
                const float sc = bf16_to_f32(sv[i]);
                if (ZP) {
                    const float z = bf16_to_f32(zv[ZP ? i : 0]);
                    const float zi = fminf(fmaxf(__builtin_rintf(z), -1024.0f), 1024.0f);
                    const float zr = z - zi;
                    frac |= zr != 0.0f;
                    const uint32_t hl = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-(1024.0f + zi)));
                    const uint32_t hh = __builtin_bit_cast(uint16_t, static_cast<_Float16>(-(64.0f + zi)));
                    *reinterpret_cast<u32x4_t *>(lds + L.table + 16u * te) =
                        u32x4_t{__float_as_uint(sc), hl | (hl << 16), hh | (hh << 16), __float_as_uint(zr)};
                } else {
                    *reinterpret_cast<float *>(lds + L.table + 4u * te) = sc;
                }
            }
        }
        if (ZP) {
            const bool any = __builtin_amdgcn_ballot_w64(frac != 0) != 0;
            if (lane == 0) reinterpret_cast<int *>(lds + L.flags)[w] = any ? 1 : 0;
        }
    }
    sp_lds_barrier();  // (the weight loads of the ring stay in flight)
    bool frac_any = false;
    if (ZP) {
        const int *fl = reinterpret_cast<const int *>(lds + L.flags);
        int f = 0;
#pragma unroll
        for (int i = 0; i < kSpWaves; ++i) f |= fl[i];
        frac_any = f != 0;
    }

    // ---- the units ----
    floatx4_t acc[TW];
    half8_t A[4];
    floatx4_t ex4;
    auto read_chunk = [&](int ci) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            A[j] = *reinterpret_cast<const half8_t *>(lds + L.xs + ((ci * 4 + j) * kWave + lane) * 16u);
        ex4 = *reinterpret_cast<const floatx4_t *>(lds + L.ex + (ci * kSpTile + 4 * q) * 4u);
    };
    // (a unit past the wave's share -- ci >= ncb -- is computed on chunk ncb - 1's activations and
    // table entry with a zero scale: its loads read zeros, and it adds exactly nothing; computing
    // it keeps the ring's loop free of branches, whose joins made the compiler wait for every
    // outstanding load)
    const SpMasks spk = sp_masks();
    auto compute = [&](int ci, int i, const u32x4_t &wv, bool valid) {
        // the chunk's quantization group is (cb0 + ci) >> gshift
        const uint32_t te = static_cast<uint32_t>(16 * (w * TW + i) + n) * static_cast<uint32_t>(ts) +
                            static_cast<uint32_t>(((cb0 + ci) >> gshift) - gb0);
        float sc, zr = 0.0f;
        uint32_t zlo = 0xE408E408u, zhi = 0xD480D480u;  // -(1024 + 8), -(64 + 8) as fp16 pairs
        if (ZP) {
            const u32x4_t ent = *reinterpret_cast<const u32x4_t *>(lds + L.table + 16u * te);
            sc = __uint_as_float(ent.x);
            zlo = ent.y;
            zhi = ent.z;
            zr = __uint_as_float(ent.w);
        } else {
            sc = *reinterpret_cast<const float *>(lds + L.table + 4u * te);
        }
        sc = valid ? sc : 0.0f;
        floatx4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[j], sp_dequant8(wv[j], zlo, zhi, spk), d, 0, 0, 0);
        if (ZP && frac_any) {  // residual zero points, through the activations' sums
            const float *sxp = reinterpret_cast<const float *>(lds + L.sx) + ci * kSpTile + 4 * q;
#pragma unroll
            for (int r = 0; r < 4; ++r) d[r] = fmaf(-zr, sxp[r], d[r]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][r] = fmaf(ex4[r] * sc, d[r], acc[i][r]);
    };

    // one 16-token tile: the ring over the wave's units, then the tile's results
    auto run_tile = [&](int tt) {
#pragma unroll
        for (int i = 0; i < TW; ++i) acc[i] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
        int kb = 0;
        do {  // NU >= 1
#pragma unroll
            for (int u = 0; u < kSpRing; ++u) {
                const int k = kb + u;
                const int i = u % TW;  // kb is a multiple of TW
                const bool valid = k < NU;
                const int ci = valid ? k / TW : ncb - 1;
                if (i == 0) read_chunk(ci);
                compute(ci, i, ring[u], valid);
                phase_fence();
                wload(k + kSpRing, ring[u]);
                phase_fence();
            }
            kb += kSpRing;
        } while (kb < NU);

        // lane (n, q) holds tokens 4q .. 4q+3 of row 16 tile + n
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            const int row = 16 * (w * TW + i) + n;
            if (row >= R) continue;
            const int gr = r0 + row;
            const float bv = (S == 1 && bias) ? bf16_to_f32(bias[gr]) : 0.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int token = tt * kSpTile + 4 * q + r;
                if (token >= M) continue;
                if (S == 1)
                    store_out(y, static_cast<int64_t>(token) * ldy + gr, acc[i][r] + bv, out_f32 != 0);
                else
                    part[(static_cast<int64_t>(s) * M + token) * d_out + gr] = acc[i][r];
            }
        }
    };
    run_tile(0);
    // further token tiles (M > 16): the same steps, the weights read once per tile (a separate
    // loop: a branch around the first tile's prologue made the compiler wait for every
    // outstanding load at the top of the ring)
    const int TT = (M + kSpTile - 1) / kSpTile;
    for (int tt = 1; tt < TT; ++tt) {
        __syncthreads();  // every wave is done with the previous tile's activations
        xload(tt);
        convert();
        prime();
        sp_lds_barrier();
        run_tile(tt);
    }
    // the ring's last loads (zeros, out of range) have no memory traffic
}

// y[m][row] = bias[row] + sum over the slices s = 0, 1, ... of part[s][m][row], in that order.
// The slices' values are loaded 8 at a time before they are added (independent loads in flight,
// not a chain of S round trips).
__global__ void __launch_bounds__(256) gemv_split_reduce_kernel(
    const float *__restrict__ part, int S, int M, int d_out, const uint16_t *__restrict__ bias,
    void *__restrict__ y, int64_t ldy, int out_f32) {
    // (M d_out S 4 bytes < 2^31: the host's plan keeps the partial sums of a split that small)
    const uint32_t total = static_cast<uint32_t>(M) * static_cast<uint32_t>(d_out);
    const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int m = static_cast<int>(idx / static_cast<uint32_t>(d_out));
    const int row = static_cast<int>(idx - static_cast<uint32_t>(m) * static_cast<uint32_t>(d_out));
    // part[s][m][row]: the slices' partial sums of one output, kSpReduceBatch loads in flight at
    // once (past S they read out of range, zeros), added in slice order
    const rsrc_t rp = make_rsrc(part, static_cast<uint32_t>(S) * total * 4u);
    float v = 0.0f;
    for (int s0 = 0; s0 < S; s0 += kSpReduceBatch) {
        float t[kSpReduceBatch];
#pragma unroll
        for (int k = 0; k < kSpReduceBatch; ++k)
            t[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rp, (static_cast<uint32_t>(s0 + k) * total + idx) * 4u, 0, 0));
#pragma unroll
        for (int k = 0; k < kSpReduceBatch; ++k) v += t[k];
    }
    if (bias) v += bf16_to_f32(bias[row]);
    store_out(y, static_cast<int64_t>(m) * ldy + row, v, out_f32 != 0);
}

}  // namespace

// The split: TW tiles per wave, S column slices, XK activation items per thread. Chosen for
// 2..64 tokens on matrices with fewer than four 16-row tiles per compute unit and groups that
// hold whole 128-column chunks: about one workgroup per compute unit, with as many rows per
// workgroup as that allows (the activations of a slice are converted once per workgroup and
// serve its 16 TB rows).
SplitPlan plan_split(int64_t M, int64_t d_out, int64_t k_pad, int64_t span, int64_t n_groups) {
    SplitPlan p{};
    const int64_t cus = device_cu_count();
    const int64_t tiles = (d_out + 15) / 16;
    const int64_t C = (k_pad + 127) / 128;
    const bool forced = split_forced();
    if (M < 2 || M > 64) return p;
    if (tiles >= 4 * cus && !forced) return p;  // the few-token kernel serves those
    if (n_groups != 1 && span != 128 && span != 256) return p;
    // the activation stage and the second kernel cost several microseconds: the split pays off
    // from about 64 KiB of codes per compute unit (measured at 16 tokens: 3584 x 18944 19 us
    // against 30 us without it; 4608 x 3584 and 3584 x 3584, 26-32 KiB per unit, 12 and 10 us
    // against 10 and 9 us)
    if (d_out * (k_pad / 2) < 64 * 1024 * cus && !forced) return p;
    p.gshift = n_groups == 1 ? 30 : (span == 256 ? 1 : 0);
    p.tw = tiles >= 2 * kSpWaves * 16 ? 2 : 1;
    const int64_t TB = p.tw * kSpWaves;
    const int64_t slices = (tiles + TB - 1) / TB;
    int64_t S = cus / slices;
    if (S < 1) S = 1;
    if (S > C) S = C;
    for (; S <= C; ++S) {  // an activation stage of at most 4 items per thread, a table of at most 8
        const int64_t ncb = (C + S - 1) / S;
        const int64_t ngb = sp_groups(static_cast<int>(ncb), p.gshift);
        if (ncb * 64 > 4 * kSpThreads) continue;
        if (16 * TB * ngb > (int64_t)kSpTableLoads * kSpThreads) continue;
        if (sp_lds(static_cast<int>(ncb), static_cast<int>(TB), static_cast<int>(ngb), true).total >
            kSpLdsLimit)
            continue;
        p.S = static_cast<int>(S);
        p.xk = ncb * 64 <= kSpThreads ? 1 : ncb * 64 <= 2 * kSpThreads ? 2 : 4;
        p.slices = static_cast<int>(slices);
        p.ok = true;
        return p;
    }
    return SplitPlan{};
}

// Workspace: the partial sums [S][M][d_out] fp32.
size_t split_work_bytes(const SplitPlan &p, int64_t M, int64_t d_out) {
    return p.ok && p.S > 1 ? static_cast<size_t>(p.S) * M * d_out * sizeof(float) : 0;
}

namespace {

template <int TW, bool ZP, int XK>
hipError_t launch_split_t(const SplitPlan &p, const uint16_t *x, int64_t ldx, int64_t M,
                          int64_t d_in, const uint8_t *qweight, const uint16_t *scales,
                          const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                          int64_t k_pad, int64_t n_groups, void *work, void *y, int64_t ldy,
                          bool out_f32, hipStream_t stream) {
    const int C = static_cast<int>((k_pad + 127) / 128);
    const int ncb = (C + p.S - 1) / p.S;
    const size_t lds = sp_lds(ncb, TW * kSpWaves, sp_groups(ncb, p.gshift), ZP).total;
    float *part = static_cast<float *>(work);
    hipLaunchKernelGGL((gemv_split_kernel<TW, ZP, XK>), dim3(p.slices, p.S), dim3(kSpThreads),
                       lds, stream, x, ldx, static_cast<int>(M), static_cast<int>(d_in), qweight,
                       scales, zeros, bias, static_cast<int>(d_out), static_cast<int>(k_pad / 2),
                       static_cast<int>(n_groups), p.gshift, C, part, y, ldy, out_f32 ? 1 : 0);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.S == 1) return err;
    const int64_t total = M * d_out;  // one thread per output (M d_out < 2^31: host)
    hipLaunchKernelGGL(gemv_split_reduce_kernel, dim3(static_cast<int>((total + 255) / 256)),
                       dim3(256), 0, stream, part, p.S, static_cast<int>(M),
                       static_cast<int>(d_out), bias, y, ldy, out_f32 ? 1 : 0);
    return hipGetLastError();
}

template <int TW, bool ZP>
hipError_t launch_split_xk(const SplitPlan &p, const uint16_t *x, int64_t ldx, int64_t M,
                           int64_t d_in, const uint8_t *qweight, const uint16_t *scales,
                           const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                           int64_t k_pad, int64_t n_groups, void *work, void *y, int64_t ldy,
                           bool out_f32, hipStream_t stream) {
    if (p.xk == 1)
        return launch_split_t<TW, ZP, 1>(p, x, ldx, M, d_in, qweight, scales, zeros, bias, d_out,
                                         k_pad, n_groups, work, y, ldy, out_f32, stream);
    if (p.xk == 2)
        return launch_split_t<TW, ZP, 2>(p, x, ldx, M, d_in, qweight, scales, zeros, bias, d_out,
                                         k_pad, n_groups, work, y, ldy, out_f32, stream);
    return launch_split_t<TW, ZP, 4>(p, x, ldx, M, d_in, qweight, scales, zeros, bias, d_out,
                                     k_pad, n_groups, work, y, ldy, out_f32, stream);
}

}  // namespace

bool gemv_split_supported(const SplitPlan &p, int64_t M, int64_t d_in, int64_t k_pad,
                          int64_t ldx) {
    if (!p.ok || M < 2 || M > 64) return false;
    // 31-bit offsets: a workgroup's weight rows (lane offsets include the slice's first chunk,
    // and units past a share step one chunk further) and the activations
    if (int64_t(16) * p.tw * kSpWaves * (k_pad / 2) + 2 * (k_pad / 2) + 1024 >= (int64_t)kOutOfRange)
        return false;
    // the reduction's descriptor spans every partial sum
    if (int64_t(p.S) * M * p.slices * 16 * p.tw * kSpWaves * 4 >= (int64_t)kOutOfRange) return false;
    return d_in <= k_pad && (M * ldx + 1024) * 2 < (int64_t)kSpNoToken;
}

hipError_t launch_gemv_split(const SplitPlan &p, const uint16_t *x, int64_t M, int64_t ldx,
                             const uint8_t *qweight, const uint16_t *scales,
                             const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                             int64_t d_in, int64_t k_pad, int64_t n_groups, void *work, void *y,
                             int64_t ldy, bool out_f32, hipStream_t stream) {
    const bool zp = zeros != nullptr;
    if (p.tw == 2)
        return zp ? launch_split_xk<2, true>(p, x, ldx, M, d_in, qweight, scales, zeros, bias,
                                             d_out, k_pad, n_groups, work, y, ldy, out_f32, stream)
                  : launch_split_xk<2, false>(p, x, ldx, M, d_in, qweight, scales, zeros, bias,
                                              d_out, k_pad, n_groups, work, y, ldy, out_f32, stream);
    return zp ? launch_split_xk<1, true>(p, x, ldx, M, d_in, qweight, scales, zeros, bias, d_out,
                                         k_pad, n_groups, work, y, ldy, out_f32, stream)
              : launch_split_xk<1, false>(p, x, ldx, M, d_in, qweight, scales, zeros, bias, d_out,
                                          k_pad, n_groups, work, y, ldy, out_f32, stream);
}

}  // namespace w4
