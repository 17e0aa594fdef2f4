// decode_stream.hip -- persistent streaming decode GEMVs (W4A16 and W4A8) for gfx950.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "基础", "INT4 线性量化",
// "融合INT4反量化与矩阵乘"), [Orin] "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到
// 24 tok/s" (sections "模型尺寸和 decode 的真实瓶颈", "DP4A 做了什么", "INT32 accumulator 是否安全",
// "o2-all 和 o4-all 为什么能加速").
//
// Decode reads every packed weight once per token; the kernel is shaped after a plain HBM
// streaming read:
//   * a persistent grid (a few workgroups per CU) converts the activations once per workgroup
//     into LDS and then streams rows until the matrix is done;
//   * each wave owns batches of RW rows; lane l handles the 16-byte chunks l, l + 64, ... of a row
//     (T steps), so a load instruction reads 1 KiB of one row;
//   * a wave keeps a ring of NB small batches: while one is computed, the next NB - 1 are in
//     flight, and the batch just computed is refilled with the one NB ahead. Many short rounds
//     with a modest amount of data in flight per CU keep the memory latency low. The
//     vector-memory counter is in order and the compiler's waits must hold on every path, so no
//     load sits behind a branch: weights, scales and bias are read with raw buffer loads through
//     a descriptor that covers exactly the batch's valid rows, and a row, chunk or batch past
//     the end of the matrix gets an offset outside it -- the load returns zeros without touching
//     memory, and a store there is dropped;
//   * the activation chunk read from LDS is shared by the RW rows of a batch (the
//     rows-share-one-activation-load idea of [Orin o2-all 和 o4-all 为什么能加速]);
//   * rows are finished with DPP cross-lane adds, in a fixed order (deterministic).
#include "w4_device.h"
#include "w4_quant.h"
#include "w4_launch.h"

#include <type_traits>

namespace w4 {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kChunkCols = 32;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr size_t kLdsLimit = 64 * 1024;

// One (token, chunk) of bf16 activations: 16 fp16 pairs ordered like the nibble pairs of a
// packed u32 ((c0,c4), (c1,c5), (c2,c6), (c3,c7) per 8 columns) holding x * 2^-e exactly; the
// exponent e; and the fp32 sum of the scaled values (for zero-point residuals).
struct alignas(16) XChunk16 {
    uint32_t h[16];
    int e;
    float sum;
    int pad[2];
};

// One (token, chunk) of int8 activations: per 8 columns, the bytes of columns 0,2,4,6 and of
// 1,3,5,7 (matching (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F)); and the chunk's sum.
struct alignas(16) XChunk8 {
    uint32_t even[4];
    uint32_t odd[4];
    int qsum;
    int pad[3];
};

// Workgroup barrier for LDS-only dependencies, without a memory fence: the caller's LDS accesses
// are completed first (lgkmcnt(0)), but the weight loads of the ring stay in flight across it (a
// fenced barrier waits for every outstanding load). The empty asm statements keep the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Waves that share a SIMD are issued oldest first. Left alone, the older wave runs through its
// batches while the younger one waits, and the younger one's arithmetic piles up at the end,
// after the weight traffic has stopped. So a wave lowers its priority by one level for each
// quarter of its n batches it has done (k of them), and the wave that is behind goes first
// (measured on the 3584 x 18944 down projection: 8.9 against 9.3 us).
__device__ __forceinline__ void progress_priority(int k, int n) {
    const int q = (4 * k >= n) + (4 * k >= 2 * n) + (4 * k >= 3 * n);  // wave-uniform
    if (q == 0)
        __builtin_amdgcn_s_setprio(3);
    else if (q == 1)
        __builtin_amdgcn_s_setprio(2);
    else if (q == 2)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// Batch shape: RW rows per batch and NB batches in the ring. Measured on MI355X for the 7B
// shapes (3584 and 18944 columns), one row per batch and two buffers with 2-4 workgroups per CU
// (a few KiB in flight per wave) beat larger batches and deeper rings: more data in flight only
// lengthens every round trip.
struct Shape {
    int rw, nb;
};
constexpr Shape stream_shape(int /*T*/) { return Shape{1, 2}; }

// Wave-level bookkeeping shared by both kernels: batch b of this wave holds rows
// (wave_id + b * total_waves) * RW + [0, RW); b_last is the wave's last batch with a row in the
// matrix (-1: none). All values are wave-uniform 32-bit scalars (d_out <= 2^24): 64-bit
// compares would need vector registers, possibly ones a prefetch is still writing.
template <int RW>
struct Rows {
    int wave_id, total_waves, rows, b_last;
    __device__ __forceinline__ Rows(int wid, int64_t d_out, int waves_per_block) {
        wave_id = static_cast<int>(blockIdx.x) * waves_per_block + wid;
        total_waves = static_cast<int>(gridDim.x) * waves_per_block;
        rows = static_cast<int>(d_out);
        const int groups = (rows + RW - 1) / RW;
        b_last = wave_id < groups ? (groups - 1 - wave_id) / total_waves : -1;
    }
    __device__ __forceinline__ int row0(int b) const { return (wave_id + b * total_waves) * RW; }
    __device__ __forceinline__ int valid(int r0) const {
        const int v = rows - r0;
        return v < 0 ? 0 : (v > RW ? RW : v);
    }
};

// ---------------------------------------------------------------------------------------------
// W4A16
// ---------------------------------------------------------------------------------------------

// Long rows are cut into SEG segments of T steps: batch b of a wave is segment b % SEG of its
// row group b / SEG (NB is a multiple of SEG, so ring slot i always holds segment i % SEG), and
// the row's sums are carried from one segment to the next. A segment's loads take fewer
// registers than a whole row's, so more waves fit on a CU. BT threads per workgroup.
template <int MT, int T, int RW, int NB, bool ZP, int SEG, int BT>
__global__ void __launch_bounds__(BT) gemv_w4a16_stream_kernel(
    const uint16_t *__restrict__ x, int64_t ldx, int M, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int64_t d_out, int64_t d_in, int64_t k_pad,
    int chunk_group_shift, int64_t n_groups, void *__restrict__ y, int64_t ldy, int out_f32,
    int n_batches) {
    extern __shared__ XChunk16 xsh[];  // [MT][cpr + 1], record cpr of each token is zero
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t cpr = k_pad / kChunkCols;
    const int64_t row_bytes = k_pad / 2;
    const Rows<RW> R(wid, d_out, BT / kWave);

    // lane's chunk of step t: byte offsets of its codes in a row and of its group's scale (out of
    // range past the row end), and of its activation record in LDS (the token's zero record cpr
    // past the row end, so a chunk of zero codes adds nothing; a byte offset, so that reading it
    // takes no multiply in the loop)
    static_assert(NB % SEG == 0, "ring slots hold fixed segments");
    uint32_t wofs[SEG][T], gofs[SEG][T], xofs[SEG][T];
#pragma unroll
    for (int sg = 0; sg < SEG; ++sg)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t c = (int64_t)(sg * T + t) * kWave + lane;
            wofs[sg][t] = c < cpr ? static_cast<uint32_t>(c * 16) : kOutOfRange;
            gofs[sg][t] =
                c < cpr ? static_cast<uint32_t>((c >> chunk_group_shift) * 2) : kOutOfRange;
            xofs[sg][t] = static_cast<uint32_t>((c < cpr ? c : cpr) * sizeof(XChunk16));
        }

    // Everything a batch needs, including the per-row bias of the epilogue (16-bit values have
    // no scalar load, and a load issued later would wait behind the prefetch). The loaded values
    // stay raw, one register each, until the batch is computed: arithmetic on them at load time
    // would make the wave wait for the whole queue.
    struct Batch {
        u32x4_t w[RW][T];
        uint32_t sc[RW][T];
        uint32_t zr[ZP ? RW : 1][ZP ? T : 1];
        uint32_t bs[RW];
    };
    const uint32_t rb = static_cast<uint32_t>(row_bytes);
    const uint32_t gb = static_cast<uint32_t>(n_groups * 2);
    auto load_batch = [&](int b, int sg, Batch &dst) {  // row group b, segment sg
        const int row0 = R.row0(b);
        const int valid = R.valid(row0);
        const int64_t r0 = valid > 0 ? row0 : 0;
        const rsrc_t rw = make_rsrc(qweight + r0 * row_bytes, valid * rb);
        const rsrc_t rs = make_rsrc(scales + r0 * n_groups, valid * gb);
        const rsrc_t rz = make_rsrc(ZP ? zeros + r0 * n_groups : scales, ZP ? valid * gb : 0u);
        const rsrc_t rbias = make_rsrc(bias ? bias + r0 : scales, bias ? valid * 2u : 0u);
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            dst.bs[r] = __builtin_amdgcn_raw_buffer_load_b16(rbias, 2 * r, 0, 0);
#pragma unroll
            for (int t = 0; t < T; ++t) {
                dst.w[r][t] = __builtin_amdgcn_raw_buffer_load_b128(rw, wofs[sg][t] + r * rb, 0,
                                                                    kNonTemporal);
                dst.sc[r][t] =
                    __builtin_amdgcn_raw_buffer_load_b16(rs, gofs[sg][t] + r * gb, 0, 0);
                if (ZP)
                    dst.zr[ZP ? r : 0][ZP ? t : 0] =
                        __builtin_amdgcn_raw_buffer_load_b16(rz, gofs[sg][t] + r * gb, 0, 0);
            }
        }
    };

    // ---- activations: SI chunk loads per thread, issued before the weight batches so that
    // waiting for them does not wait for the weight loads. x rows are ldx apart with ldx % 8 == 0,
    // so an 8-column piece that starts before d_in lies inside its row; a piece at or past d_in,
    // and every piece of a thread past the last chunk, gets an out-of-range offset and reads as
    // zeros. (The host keeps the tile's offsets below 2^31.) ----
    constexpr int SI = (MT * T * SEG * kWave + BT - 1) / BT;  // >= ceil(MT * cpr / BT)
    const int n_chunks = MT * static_cast<int>(cpr);
    const int cpr_i = static_cast<int>(cpr);
    const int din = static_cast<int>(d_in);  // decode rows have d_in <= 65536
    const rsrc_t rx = make_rsrc(x, 0x7FFFFFFFu);
    uint4 xraw[SI][4];
#pragma unroll
    for (int si = 0; si < SI; ++si) {
        const int idx = static_cast<int>(threadIdx.x) + si * BT;
        const int m = MT == 1 ? 0 : idx / cpr_i;
        const int c = idx - m * cpr_i;
        const int mx = m < M ? m : M - 1;  // tokens of the tile past M repeat token M - 1
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int col = c * kChunkCols + 8 * p;
            const uint32_t off = idx < n_chunks && col < din
                                     ? static_cast<uint32_t>(((int64_t)mx * ldx + col) * 2)
                                     : kOutOfRange;
            xraw[si][p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
    }
    // The ring's first batches. With segmented (long) rows only the first is issued before the
    // activations are converted: the activation loads then wait behind less weight traffic, and
    // the arithmetic starts earlier (measured on the 3584 x 18944 down projection: 9.9 against
    // 10.3 us); the rest follow the barrier below.
    constexpr int K0 = SEG > 1 ? 1 : NB;
    Batch buf[NB];
#pragma unroll
    for (int i = 0; i < K0; ++i) {
        phase_fence();
        load_batch(i / SEG, i % SEG, buf[i]);
    }
    phase_fence();

    // ---- convert: each 32-column chunk is scaled by 2^-e with max|x 2^-e| in [2^14, 2^15):
    // bf16 values convert to fp16 exactly (8 of fp16's 11 significand bits) unless they are
    // below max * 2^-31 of their chunk ----
    // (a wave whose chunks all lie past the end skips the work: a wave-uniform branch that holds
    // no load, so the waits for the activation loads still leave the weight loads in flight)
    const bool ragged = (din & 7) != 0;  // the piece holding column d_in - 1 has columns past it
    const half2_t ones = {static_cast<half_t>(1.0f), static_cast<half_t>(1.0f)};
#pragma unroll
    for (int si = 0; si < SI; ++si) {
        if (si * BT + wid * kWave >= n_chunks) break;
        const int idx = static_cast<int>(threadIdx.x) + si * BT;
        const int m = MT == 1 ? 0 : idx / cpr_i;
        const int c = idx - m * cpr_i;
        uint32_t u[16];  // piece p, dword k: columns 8p + 2k (low half) and 8p + 2k + 1 (high)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            u[4 * p + 0] = xraw[si][p].x;
            u[4 * p + 1] = xraw[si][p].y;
            u[4 * p + 2] = xraw[si][p].z;
            u[4 * p + 3] = xraw[si][p].w;
        }
        if (__builtin_expect(ragged, 0)) {  // zero the columns at or past d_in
            // (kept a real branch: if-converted, the masks would cost every shape 64 VALU ops)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int col = c * kChunkCols + 2 * k;
                u[k] &= col + 1 < din ? 0xFFFFFFFFu : (col < din ? 0x0000FFFFu : 0u);
            }
        }
        // the largest magnitude, compared on the bf16 bit patterns (monotone in |x|)
        u16x2_t am = {0, 0};
#pragma unroll
        for (int k = 0; k < 16; ++k)
            am = __builtin_elementwise_max(am, __builtin_bit_cast(u16x2_t, u[k] & 0x7FFF7FFFu));
        const uint32_t amax_bits = am.x > am.y ? am.x : am.y;
        const float amax = __uint_as_float(amax_bits << 16);
        const int e = amax > 0.0f ? ilogbf(amax) - 14 : 0;
        XChunk16 rec;
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t a = u[4 * j + (i >> 1)], b = u[4 * j + 2 + (i >> 1)];
                const float xa = __uint_as_float((i & 1) ? (a & 0xFFFF0000u) : (a << 16));
                const float xb = __uint_as_float((i & 1) ? (b & 0xFFFF0000u) : (b << 16));
                half2_t h;
                h.x = static_cast<half_t>(ldexpf(xa, -e));  // column 8j + i, exact (v_ldexp)
                h.y = static_cast<half_t>(ldexpf(xb, -e));  // column 8j + i + 4
                rec.h[4 * j + i] = as_u32(h);
                if (ZP) sum = __builtin_amdgcn_fdot2(h, ones, sum, false);
            }
        }
        rec.e = e;
        rec.sum = sum;
        rec.pad[0] = rec.pad[1] = 0;
        if (idx < n_chunks) xsh[m * (cpr_i + 1) + c] = rec;
    }
    if (threadIdx.x < MT) {
        XChunk16 zero;
#pragma unroll
        for (int i = 0; i < 16; ++i) zero.h[i] = 0u;
        zero.e = 0;
        zero.sum = 0.0f;
        zero.pad[0] = zero.pad[1] = 0;
        xsh[(int64_t)threadIdx.x * (cpr + 1) + cpr] = zero;
    }
    lds_barrier();  // (the weight loads of the ring stay in flight)
#pragma unroll
    for (int i = K0; i < NB; ++i) {
        phase_fence();
        load_batch(i / SEG, i % SEG, buf[i]);
    }
    phase_fence();

    // ---- dequantize inside the dot products ([Lab5 融合INT4反量化与矩阵乘]):
    //   (w & 0x000F000F) | 0x6400_6400 = fp16 (1024 + c0, 1024 + c4), (w & 0x00F000F0) | ... =
    //   (1024 + 16 c1, 1024 + 16 c5), the same on w >> 8; one packed fp16 add/fma gives the
    //   exact integers (c - z), and v_dot2_f32_f16 multiplies them with the paired activations.
    const uint32_t kMask0 = 0x000F000Fu, kMask1 = 0x00F000F0u, kMagic = 0x64006400u;
    const half2_t one16 = {static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
    // results of a batch, stored only after the refill of its buffer has been issued: a load
    // issued after a store may reuse the store's data register and would first wait for it
    struct Out {
        float v[RW][MT];
    };
    float carry[RW][MT];  // a row's sums from its earlier segments
    auto compute_batch = [&](const Batch &bt, Out &out, int sg) {
        float acc[RW][MT];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = sg == 0 ? 0.0f : carry[r][m];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            half2_t xf[MT][16];
            int xe[MT];
            float xs[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const XChunk16 &rec = *reinterpret_cast<const XChunk16 *>(
                    reinterpret_cast<const unsigned char *>(xsh) +
                    static_cast<uint32_t>(m) * static_cast<uint32_t>((cpr + 1) * sizeof(XChunk16)) +
                    xofs[sg][t]);
#pragma unroll
                for (int i = 0; i < 16; ++i) xf[m][i] = as_half2(rec.h[i]);
                xe[m] = rec.e;
                xs[m] = rec.sum;
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const float s = bf16_to_f32(bt.sc[r][t]);
                half2_t nz0 = {static_cast<half_t>(-1032.0f), static_cast<half_t>(-1032.0f)};
                half2_t nz1 = {static_cast<half_t>(-72.0f), static_cast<half_t>(-72.0f)};
                float zres = 0.0f;
                if (ZP) {
                    const float z = bf16_to_f32(bt.zr[ZP ? r : 0][ZP ? t : 0]);
                    // zero points that are not integers of magnitude <= 1024 (w4_pack never
                    // makes one) split into such an integer and a residual applied through the
                    // chunk's activation sum
                    const bool zint = (z == __builtin_rintf(z)) && fabsf(z) <= 1024.0f;
                    const float zi = zint ? z : 0.0f;
                    zres = z - zi;
                    const half_t h0 = static_cast<half_t>(-(1024.0f + zi));
                    const half_t h1 = static_cast<half_t>(-(64.0f + zi));
                    nz0 = half2_t{h0, h0};
                    nz1 = half2_t{h1, h1};
                }
                float d0[MT], d1[MT];
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    d0[m] = 0.0f;
                    d1[m] = 0.0f;
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w0 = bt.w[r][t][j];
                    const uint32_t w8 = w0 >> 8;
                    const half2_t a0 = as_half2(and_or(w0, kMask0, kMagic)) + nz0;
                    const half2_t a1 = __builtin_elementwise_fma(
                        as_half2(and_or(w0, kMask1, kMagic)), one16, nz1);
                    const half2_t a2 = as_half2(and_or(w8, kMask0, kMagic)) + nz0;
                    const half2_t a3 = __builtin_elementwise_fma(
                        as_half2(and_or(w8, kMask1, kMagic)), one16, nz1);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        d0[m] = __builtin_amdgcn_fdot2(a0, xf[m][4 * j + 0], d0[m], false);
                        d1[m] = __builtin_amdgcn_fdot2(a1, xf[m][4 * j + 1], d1[m], false);
                        d0[m] = __builtin_amdgcn_fdot2(a2, xf[m][4 * j + 2], d0[m], false);
                        d1[m] = __builtin_amdgcn_fdot2(a3, xf[m][4 * j + 3], d1[m], false);
                    }
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float chunk = ZP ? (d0[m] + d1[m]) - zres * xs[m] : d0[m] + d1[m];
                    acc[r][m] = fmaf(ldexpf(s, xe[m]), chunk, acc[r][m]);
                }
            }
        }
        if (sg < SEG - 1) {
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) carry[r][m] = acc[r][m];
            return;
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float v = wave_sum_dpp(acc[r][m]);
                if (bias) v += bf16_to_f32(bt.bs[r]);
                out.v[r][m] = v;
            }
        }
    };
    // every lane stores the wave's (uniform) result; rows past d_out and tokens past M are out
    // of the descriptor's range and dropped
    const uint32_t out_elem = out_f32 ? 4u : 2u;
    auto store_batch = [&](int b, const Out &out) {
        const int row0 = R.row0(b);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool tok = m < M;
            const rsrc_t ry = make_rsrc(
                static_cast<char *>(y) + (tok ? (int64_t)m * ldy * out_elem : 0),
                tok ? static_cast<uint32_t>(R.rows) * out_elem : 0u);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int row = row0 + r;
                const uint32_t off =
                    row < R.rows ? static_cast<uint32_t>(row) * out_elem : kOutOfRange;
                if (out_f32)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out.v[r][m]), ry, off,
                                                          0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(
                        static_cast<uint16_t>(f32_to_bf16(out.v[r][m])), ry, off, 0, 0);
            }
        }
    };

    // The ring: fences keep each batch's arithmetic between its own loads (hoisting a later
    // batch's arithmetic would wait for that batch). n_batches is a multiple of NB, so the loop
    // has no exit between a prefetch and its use (a prefetch that is dead on some path would be
    // sunk past the fences). Batches past the wave's last row group are loaded (zeros, no
    // memory traffic) but not computed.
    // (b counts segments; the row group of batch b is b / SEG)
    Out out;
    const int b_last = (R.b_last + 1) * SEG - 1;
    int b = 0;
    do {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            progress_priority(b + i, b_last + 1);
            if (b + i <= b_last) compute_batch(buf[i], out, i % SEG);
            phase_fence();
            load_batch((b + i + NB) / SEG, i % SEG, buf[i]);
            phase_fence();
            if (i % SEG == SEG - 1 && b + i <= b_last) store_batch((b + i) / SEG, out);
        }
        b += NB;
    } while (b < n_batches);
}

// ---------------------------------------------------------------------------------------------
// W4A8
// ---------------------------------------------------------------------------------------------

// (segments of long rows and BT threads per workgroup: see the W4A16 kernel)
// FQ: the activations arrive as bf16 x ([M][ldq] elements) and are quantized here, token by
// token, with the rule of act_quant_int8 (w4_quant.h): every workgroup takes the token's maximum
// over the whole row and quantizes the chunks it stages, so q never goes through memory. The
// token scales are then written to s_x (if given) by workgroup 0. Otherwise they arrive as int8
// codes with their scales in s_x.
template <int MT, int T, int RW, int NB, int SEG, int BT, bool FQ>
__global__ void __launch_bounds__(BT) gemv_w4a8_stream_kernel(
    const void *__restrict__ act, int64_t ldq, int M, float *__restrict__ s_x,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ s_w,
    const uint16_t *__restrict__ bias, int64_t d_out, int64_t d_in, int64_t k_pad,
    void *__restrict__ y, int64_t ldy, int out_f32, int32_t *__restrict__ acc_out,
    int n_batches) {
    // [MT][cpr + 1] records (record cpr of each token is zero), then (FQ) [MT] token maxima
    extern __shared__ XChunk8 qsh[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t cpr = k_pad / kChunkCols;
    const int64_t row_bytes = k_pad / 2;
    const Rows<RW> R(wid, d_out, BT / kWave);

    static_assert(NB % SEG == 0, "ring slots hold fixed segments");
    uint32_t wofs[SEG][T];  // see the W4A16 kernel
    int xofs[SEG][T];
#pragma unroll
    for (int sg = 0; sg < SEG; ++sg)
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t c = (int64_t)(sg * T + t) * kWave + lane;
            wofs[sg][t] = c < cpr ? static_cast<uint32_t>(c * 16) : kOutOfRange;
            xofs[sg][t] = static_cast<int>(c < cpr ? c : cpr);
        }
    // per-row s_w and bias travel with the batch (see the W4A16 kernel)
    struct Batch {
        u32x4_t w[RW][T];
        uint32_t sw[RW];
        uint32_t bs[RW];
    };
    const uint32_t rb = static_cast<uint32_t>(row_bytes);
    auto load_batch = [&](int b, int sg, Batch &dst) {  // row group b, segment sg
        const int row0 = R.row0(b);
        const int valid = R.valid(row0);
        const int64_t r0 = valid > 0 ? row0 : 0;
        const rsrc_t rw = make_rsrc(qweight + r0 * row_bytes, valid * rb);
        const rsrc_t rsw = make_rsrc(s_w + r0, valid * 2u);
        const rsrc_t rbias = make_rsrc(bias ? bias + r0 : s_w, bias ? valid * 2u : 0u);
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            dst.sw[r] = __builtin_amdgcn_raw_buffer_load_b16(rsw, 2 * r, 0, 0);
            dst.bs[r] = __builtin_amdgcn_raw_buffer_load_b16(rbias, 2 * r, 0, 0);
#pragma unroll
            for (int t = 0; t < T; ++t)
                dst.w[r][t] = __builtin_amdgcn_raw_buffer_load_b128(rw, wofs[sg][t] + r * rb, 0,
                                                                    kNonTemporal);
        }
    };
    // activations and their scales first (see the W4A16 kernel), then the ring of batches
    float sx[MT];
    if (!FQ) {
#pragma unroll
        for (int m = 0; m < MT; ++m) sx[m] = s_x[m < M ? m : M - 1];
    }
    // (rows are ldq elements apart with ldq % 16 == 0 for int8 codes and ldq % 8 == 0 for bf16:
    // a 16-byte piece that starts before d_in lies inside its row; pieces past d_in and threads
    // past the last chunk read zeros)
    constexpr int SI = (MT * T * SEG * kWave + BT - 1) / BT;  // >= ceil(MT * cpr / BT)
    constexpr int NP = FQ ? 4 : 2;                            // 16-byte pieces per chunk
    constexpr int EB = FQ ? 2 : 1;                            // bytes per activation
    const int n_chunks = MT * static_cast<int>(cpr);
    const int cpr_i = static_cast<int>(cpr);
    const int din = static_cast<int>(d_in);
    const rsrc_t rx = make_rsrc(act, 0x7FFFFFFFu);  // the host keeps the offsets below 2^31
    uint4 qraw[SI][NP];
#pragma unroll
    for (int si = 0; si < SI; ++si) {
        const int idx = static_cast<int>(threadIdx.x) + si * BT;
        const int m = MT == 1 ? 0 : idx / cpr_i;
        const int c = idx - m * cpr_i;
        const int mx = m < M ? m : M - 1;  // tokens of the tile past M repeat token M - 1
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int col = c * kChunkCols + (16 / EB) * p;
            const uint32_t off = idx < n_chunks && col < din
                                     ? static_cast<uint32_t>(((int64_t)mx * ldq + col) * EB)
                                     : kOutOfRange;
            qraw[si][p] =
                __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
        }
    }
    constexpr int K0 = SEG > 1 ? 1 : NB;  // (as in the W4A16 kernel)
    Batch buf[NB];
#pragma unroll
    for (int i = 0; i < K0; ++i) {
        phase_fence();
        load_batch(i / SEG, i % SEG, buf[i]);
    }
    phase_fence();

    // FQ: each token's largest |x| over the row, on the bf16 magnitude bits (monotone in |x|)
    uint32_t *tmax = reinterpret_cast<uint32_t *>(qsh + MT * (cpr + 1));
    if (FQ) {
        if (threadIdx.x < MT) tmax[threadIdx.x] = 0u;
        lds_barrier();
#pragma unroll
        for (int si = 0; si < SI; ++si) {
            if (si * BT + wid * kWave >= n_chunks) break;
            const int idx = static_cast<int>(threadIdx.x) + si * BT;
            const int m = MT == 1 ? 0 : idx / cpr_i;
            const int c = idx - m * cpr_i;
            // (columns past d_in hold whatever follows in memory: masked without a branch)
            u16x2_t m2 = {0, 0};
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint4 &raw = qraw[si][k >> 2];
                const uint32_t d = (k & 3) == 0 ? raw.x : (k & 3) == 1 ? raw.y
                                   : (k & 3) == 2 ? raw.z : raw.w;
                const int left = din - (c * kChunkCols + 2 * k);  // columns of d before d_in
                const uint32_t keep = left >= 2 ? 0x7FFF7FFFu : (left == 1 ? 0x7FFFu : 0u);
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_t, d & keep));
            }
            uint32_t am = idx < n_chunks ? (m2[0] > m2[1] ? m2[0] : m2[1]) : 0u;
            if (MT == 1) {  // one token: a wave-wide maximum, then one atomic per wave
#pragma unroll
                for (int o = 32; o > 0; o >>= 1)
                    am = max(am, static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), o, kWave)));
                if (lane == 0) atomicMax(&tmax[0], am);
            } else if (idx < n_chunks) {
                atomicMax(&tmax[m], am);
            }
        }
        lds_barrier();
#pragma unroll
        for (int m = 0; m < MT; ++m) sx[m] = token_scale_int8(__uint_as_float(tmax[m] << 16));
        if (blockIdx.x == 0 && threadIdx.x < MT && static_cast<int>(threadIdx.x) < M && s_x)
            s_x[threadIdx.x] = token_scale_int8(__uint_as_float(tmax[threadIdx.x] << 16));
    }

    // permute to the nibble order ([Orin DP4A 做了什么]) and stage in LDS (a wave whose chunks
    // all lie past the end skips the work; see the W4A16 kernel)
    const bool ragged = (din & 15) != 0;  // the piece holding column d_in - 1 has bytes past it
#pragma unroll
    for (int si = 0; si < SI; ++si) {
        if (si * BT + wid * kWave >= n_chunks) break;
        const int idx = static_cast<int>(threadIdx.x) + si * BT;
        const int m = MT == 1 ? 0 : idx / cpr_i;
        const int c = idx - m * cpr_i;
        uint32_t u[8];
        if (FQ) {  // quantize the chunk: int8 codes of columns c * 32 .. + 31, in column order
            const float a = __uint_as_float(tmax[m] << 16);
            const float sc = token_scale_int8(a);
            const float rc = 1.0f / sc;  // correctly rounded
            // the codes of quantize_int8_fast, with its exact fallback taken once per chunk
            float t[kChunkCols];
            bool slow = !(fabsf(rc) < 0x1.0p126f);
#pragma unroll
            for (int e = 0; e < kChunkCols; ++e) {
                const uint4 &raw = qraw[si][e >> 3];
                const uint32_t d = ((e >> 1) & 3) == 0 ? raw.x : ((e >> 1) & 3) == 1 ? raw.y
                                   : ((e >> 1) & 3) == 2 ? raw.z : raw.w;
                const float xv = bf16_to_f32((e & 1) ? (d >> 16) : (d & 0xFFFFu));
                t[e] = quantize_int8_band(xv, rc, slow);
            }
            if (__builtin_expect(slow, 0)) {
#pragma unroll
                for (int e = 0; e < kChunkCols; ++e) {
                    const uint4 &raw = qraw[si][e >> 3];
                    const uint32_t d = ((e >> 1) & 3) == 0 ? raw.x : ((e >> 1) & 3) == 1 ? raw.y
                                       : ((e >> 1) & 3) == 2 ? raw.z : raw.w;
                    const float xv = bf16_to_f32((e & 1) ? (d >> 16) : (d & 0xFFFFu));
                    t[e] = static_cast<float>(quantize_int8(xv, sc));
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = 0u;
#pragma unroll
            for (int e = 0; e < kChunkCols; ++e) {
                const int qe = a != 0.0f && c * kChunkCols + e < din ? static_cast<int>(t[e]) : 0;
                u[e >> 2] |= (static_cast<uint32_t>(qe) & 0xFFu) << (8 * (e & 3));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint4 &raw = qraw[si][i >> 2];
                u[i] = (i & 3) == 0 ? raw.x : (i & 3) == 1 ? raw.y : (i & 3) == 2 ? raw.z : raw.w;
            }
        }
        if (!FQ && __builtin_expect(ragged, 0)) {  // zero the bytes at or past d_in
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int left = din - (c * kChunkCols + 4 * i);  // bytes before d_in: 0..4
                u[i] &= left >= 4 ? 0xFFFFFFFFu : (left <= 0 ? 0u : (1u << (8 * left)) - 1u);
            }
        }
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            sum = __builtin_amdgcn_sdot4(static_cast<int>(u[i]), 0x01010101, sum, false);
        XChunk8 rec;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rec.even[j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x06040200u);
            rec.odd[j] = __builtin_amdgcn_perm(u[2 * j + 1], u[2 * j], 0x07050301u);
        }
        rec.qsum = sum;
        rec.pad[0] = rec.pad[1] = rec.pad[2] = 0;
        if (idx < n_chunks) qsh[m * (cpr_i + 1) + c] = rec;
    }
    if (threadIdx.x < MT) {
        XChunk8 zero;
#pragma unroll
        for (int j = 0; j < 4; ++j) zero.even[j] = zero.odd[j] = 0u;
        zero.qsum = 0;
        zero.pad[0] = zero.pad[1] = zero.pad[2] = 0;
        qsh[(int64_t)threadIdx.x * (cpr + 1) + cpr] = zero;
    }
    lds_barrier();  // (the weight loads of the ring stay in flight)
#pragma unroll
    for (int i = K0; i < NB; ++i) {
        phase_fence();
        load_batch(i / SEG, i % SEG, buf[i]);
    }
    phase_fence();

    // sum_k (c - 8) q = sum_k c q - 8 sum_k q, exactly in int32 ([Orin INT32 accumulator 是否安全])
    struct Out {  // see the W4A16 kernel
        float v[RW][MT];
        int a[RW][MT];
    };
    int carry[RW][MT];  // a row's sums from its earlier segments
    auto compute_batch = [&](const Batch &bt, Out &out, int sg) {
        int acc[RW][MT];
#pragma unroll
        for (int r = 0; r < RW; ++r)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[r][m] = sg == 0 ? 0 : carry[r][m];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            uint32_t xe[MT][4], xo[MT][4];
            int qs[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const XChunk8 &rec = qsh[(int64_t)m * (cpr + 1) + xofs[sg][t]];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    xe[m][j] = rec.even[j];
                    xo[m][j] = rec.odd[j];
                }
                qs[m] = rec.qsum;
            }
#pragma unroll
            for (int r = 0; r < RW; ++r) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int lo = static_cast<int>(bt.w[r][t][j] & 0x0F0F0F0Fu);
                    const int hi = static_cast<int>((bt.w[r][t][j] >> 4) & 0x0F0F0F0Fu);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        acc[r][m] = __builtin_amdgcn_sdot4(lo, static_cast<int>(xe[m][j]),
                                                           acc[r][m], false);
                        acc[r][m] = __builtin_amdgcn_sdot4(hi, static_cast<int>(xo[m][j]),
                                                           acc[r][m], false);
                    }
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[r][m] -= 8 * qs[m];
            }
        }
        if (sg < SEG - 1) {
#pragma unroll
            for (int r = 0; r < RW; ++r)
#pragma unroll
                for (int m = 0; m < MT; ++m) carry[r][m] = acc[r][m];
            return;
        }
#pragma unroll
        for (int r = 0; r < RW; ++r) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int a = wave_sum_dpp(acc[r][m]);
                const float scale = bf16_to_f32(bt.sw[r]) * sx[m];
                float v = scale * static_cast<float>(a);
                if (bias) v += bf16_to_f32(bt.bs[r]);
                out.a[r][m] = a;
                out.v[r][m] = v;
            }
        }
    };
    const uint32_t out_elem = out_f32 ? 4u : 2u;  // see the W4A16 kernel
    auto store_batch = [&](int b, const Out &out) {
        const int row0 = R.row0(b);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool tok = m < M;
            const rsrc_t ry = make_rsrc(
                static_cast<char *>(y) + (tok ? (int64_t)m * ldy * out_elem : 0),
                tok ? static_cast<uint32_t>(R.rows) * out_elem : 0u);
            const rsrc_t ra = make_rsrc(acc_out ? acc_out + (tok ? (int64_t)m * d_out : 0) : y,
                                        acc_out && tok ? static_cast<uint32_t>(R.rows) * 4u : 0u);
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                const int row = row0 + r;
                const bool ok = row < R.rows;
                if (acc_out)
                    __builtin_amdgcn_raw_buffer_store_b32(
                        out.a[r][m], ra, ok ? static_cast<uint32_t>(row) * 4u : kOutOfRange, 0, 0);
                const uint32_t off = ok ? static_cast<uint32_t>(row) * out_elem : kOutOfRange;
                if (out_f32)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(out.v[r][m]), ry, off,
                                                          0, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b16(
                        static_cast<uint16_t>(f32_to_bf16(out.v[r][m])), ry, off, 0, 0);
            }
        }
    };

    Out out;  // the ring of the W4A16 kernel (b counts segments)
    const int b_last = (R.b_last + 1) * SEG - 1;
    int b = 0;
    do {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            progress_priority(b + i, b_last + 1);
            if (b + i <= b_last) compute_batch(buf[i], out, i % SEG);
            phase_fence();
            load_batch((b + i + NB) / SEG, i % SEG, buf[i]);
            phase_fence();
            if (i % SEG == SEG - 1 && b + i <= b_last) store_batch((b + i) / SEG, out);
        }
        b += NB;
    } while (b < n_batches);
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------

// Token tile of one launch: 1, 2 or 4 tokens; long rows take fewer tokens per launch (the
// per-token dot products and the ring of batches share the registers).
constexpr int kMaxT2 = 10, kMaxT4 = 6;  // largest step count served with 2 and 4 tokens
int stream_token_tile(int64_t M, int T) {
    if (M >= 3 && T <= kMaxT4) return 4;
    if (M >= 2 && T <= kMaxT2) return 2;
    return 1;
}


// Instantiated step counts (T >= chunks per row / 64; extra steps are masked).
constexpr int kSteps[] = {1, 2, 3, 4, 6, 8, 10, 12, 16};

int pick_steps(int64_t cpr) {
    for (int t : kSteps)
        if ((int64_t)t * kWave >= cpr) return t;
    return 0;
}

// Workgroups per CU of the persistent grid (measured on MI355X).
int stream_blocks_per_cu(int T, int seg, int64_t d_out) {
    if (seg > 1) return 1;
    if (T > 2) return 2;
    return d_out >= 32 * (int64_t)device_cu_count() ? 4 : 3;  // fewer rows: fewer workgroups
}

struct StreamPlan {
    int grid;
    int n_batches;
};

// T: steps per row; SEG: segments per row (n_batches counts segments)
// (bpc_div > 1: that many times fewer workgroups per CU, for kernels with a larger per-workgroup
// prologue that run with more waves per workgroup instead)
StreamPlan plan_stream(int64_t d_out, int T, int RW, int NB, int SEG = 1, int waves = kWaves,
                       int bpc_div = 1) {
    StreamPlan p{};
    const int64_t rows_per_round_per_block = (int64_t)waves * RW;
    int bpc = stream_blocks_per_cu(T, SEG, d_out) / bpc_div;
    if (bpc < 1) bpc = 1;
    int64_t blocks = (int64_t)device_cu_count() * bpc;
    const int64_t need = (d_out + rows_per_round_per_block - 1) / rows_per_round_per_block;
    if (blocks > need) blocks = need;
    p.grid = static_cast<int>(blocks);
    int64_t nb = (d_out + blocks * rows_per_round_per_block - 1) / (blocks * rows_per_round_per_block);
    nb *= SEG;
    nb = (nb + NB - 1) / NB * NB;  // the kernels' ring takes batches NB at a time
    p.n_batches = static_cast<int>(nb);
    return p;
}

template <int MT, int T>
hipError_t launch_w4a16_stream_t(bool zp, const uint16_t *x, int64_t ldx, int M,
                                 const uint8_t *qweight, const uint16_t *scales,
                                 const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                                 int64_t d_in, int64_t k_pad, int shift, int64_t n_groups,
                                 void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    constexpr Shape S = stream_shape(T);
    // one token on rows of 8 or more steps: two segments per row (see the kernel)
    constexpr int SEG = MT == 1 && T >= 8 ? 2 : 1;
    static_assert(T % SEG == 0 && S.nb % SEG == 0, "segments");
    const size_t lds = sizeof(XChunk16) * (size_t)MT * (size_t)(k_pad / kChunkCols + 1);
    auto launch = [&](auto bt) {
        constexpr int BT = decltype(bt)::value;
        const StreamPlan p = plan_stream(d_out, T, S.rw, S.nb, SEG, BT / kWave);
        if (zp)
            hipLaunchKernelGGL((gemv_w4a16_stream_kernel<MT, T / SEG, S.rw, S.nb, true, SEG, BT>),
                               dim3(p.grid), dim3(BT), lds, stream, x, ldx, M, qweight, scales,
                               zeros, bias, d_out, d_in, k_pad, shift, n_groups, y, ldy,
                               out_f32 ? 1 : 0, p.n_batches);
        else
            hipLaunchKernelGGL((gemv_w4a16_stream_kernel<MT, T / SEG, S.rw, S.nb, false, SEG, BT>),
                               dim3(p.grid), dim3(BT), lds, stream, x, ldx, M, qweight, scales,
                               zeros, bias, d_out, d_in, k_pad, shift, n_groups, y, ldy,
                               out_f32 ? 1 : 0, p.n_batches);
    };
    if (SEG > 1) {
        // segmented long rows: one workgroup per CU of 7 or 8 waves (the activations are
        // converted once per workgroup), whichever leaves fewer wave slots idle in the last
        // round of rows (C2 down: 3584 rows = 2 rounds of 256 x 7 waves)
        const int64_t cus = device_cu_count();
        auto idle = [&](int64_t w) { return (d_out + cus * w - 1) / (cus * w) * cus * w - d_out; };
        if (idle(7) < idle(8))
            launch(std::integral_constant<int, 7 * kWave>());
        else
            launch(std::integral_constant<int, 2 * kThreads>());
    } else {
        launch(std::integral_constant<int, kThreads>());
    }
    return hipGetLastError();
}

template <int MT>
hipError_t launch_w4a16_stream_mt(int T, bool zp, const uint16_t *x, int64_t ldx, int M,
                                  const uint8_t *qweight, const uint16_t *scales,
                                  const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                                  int64_t d_in, int64_t k_pad, int shift, int64_t n_groups,
                                  void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
#define W4_STREAM_CASE(TT)                                                                        \
    case TT:                                                                                      \
        if constexpr ((MT == 4 && TT > kMaxT4) || (MT == 2 && TT > kMaxT2))                       \
            return hipErrorInvalidValue;                                                          \
        else                                                                                      \
            return launch_w4a16_stream_t<MT, TT>(zp, x, ldx, M, qweight, scales, zeros, bias,     \
                                                 d_out, d_in, k_pad, shift, n_groups, y, ldy,     \
                                                 out_f32, stream);
    switch (T) {
        W4_STREAM_CASE(1)
        W4_STREAM_CASE(2)
        W4_STREAM_CASE(3)
        W4_STREAM_CASE(4)
        W4_STREAM_CASE(6)
        W4_STREAM_CASE(8)
        W4_STREAM_CASE(10)
        W4_STREAM_CASE(12)
        W4_STREAM_CASE(16)
        default:
            return hipErrorInvalidValue;
    }
#undef W4_STREAM_CASE
}

// LDS of the W4A8 kernel: the staged chunks, and (FQ) the token maxima
size_t w4a8_lds_bytes(int MT, int64_t k_pad, bool fq) {
    return sizeof(XChunk8) * (size_t)MT * (size_t)(k_pad / kChunkCols + 1) +
           (fq ? 16u * (size_t)((MT + 3) / 4) : 0u);
}

template <int MT, int T, bool FQ>
hipError_t launch_w4a8_stream_t(const void *act, int64_t ldq, int M, float *s_x,
                                const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                                int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                                bool out_f32, int32_t *acc, hipStream_t stream) {
    constexpr Shape S = stream_shape(T);
    constexpr int SEG = MT == 1 && T >= 8 ? 2 : 1;  // see launch_w4a16_stream_t
    static_assert(T % SEG == 0 && S.nb % SEG == 0, "segments");
    // 8-wave workgroups for segmented rows (see launch_w4a16_stream_t) and whenever the
    // workgroup quantizes the activations itself: a CU then quantizes the row half as often
    // (segmented rows: 7 or 8 waves, as in launch_w4a16_stream_t)
    constexpr bool wide = SEG > 1 || FQ;
    const size_t lds = w4a8_lds_bytes(MT, k_pad, FQ);
    auto launch = [&](auto bt) {
        constexpr int BT = decltype(bt)::value;
        const StreamPlan p =
            plan_stream(d_out, T, S.rw, S.nb, SEG, BT / kWave, FQ && SEG == 1 ? 2 : 1);
        hipLaunchKernelGGL((gemv_w4a8_stream_kernel<MT, T / SEG, S.rw, S.nb, SEG, BT, FQ>),
                           dim3(p.grid), dim3(BT), lds, stream, act, ldq, M, s_x, qweight, s_w,
                           bias, d_out, d_in, k_pad, y, ldy, out_f32 ? 1 : 0, acc, p.n_batches);
    };
    if (SEG > 1) {
        const int64_t cus = device_cu_count();
        auto idle = [&](int64_t w) { return (d_out + cus * w - 1) / (cus * w) * cus * w - d_out; };
        if (idle(7) < idle(8))
            launch(std::integral_constant<int, 7 * kWave>());
        else
            launch(std::integral_constant<int, 2 * kThreads>());
    } else {
        launch(std::integral_constant<int, wide ? 2 * kThreads : kThreads>());
    }
    return hipGetLastError();
}

template <int MT, bool FQ>
hipError_t launch_w4a8_stream_mt(int T, const void *act, int64_t ldq, int M, float *s_x,
                                 const uint8_t *qweight, const uint16_t *s_w,
                                 const uint16_t *bias, int64_t d_out, int64_t d_in,
                                 int64_t k_pad, void *y, int64_t ldy, bool out_f32, int32_t *acc,
                                 hipStream_t stream) {
#define W4_STREAM8_CASE(TT)                                                                       \
    case TT:                                                                                      \
        if constexpr ((MT == 4 && TT > kMaxT4) || (MT == 2 && TT > kMaxT2))                       \
            return hipErrorInvalidValue;                                                          \
        else                                                                                      \
            return launch_w4a8_stream_t<MT, TT, FQ>(act, ldq, M, s_x, qweight, s_w, bias, d_out,  \
                                                    d_in, k_pad, y, ldy, out_f32, acc, stream);
    switch (T) {
        W4_STREAM8_CASE(1)
        W4_STREAM8_CASE(2)
        W4_STREAM8_CASE(3)
        W4_STREAM8_CASE(4)
        W4_STREAM8_CASE(6)
        W4_STREAM8_CASE(8)
        W4_STREAM8_CASE(10)
        W4_STREAM8_CASE(12)
        W4_STREAM8_CASE(16)
        default:
            return hipErrorInvalidValue;
    }
#undef W4_STREAM8_CASE
}

}  // namespace

bool gemv_stream_supported(int64_t M, int64_t k_pad) {
    const int64_t cpr = k_pad / kChunkCols;
    if (pick_steps(cpr) == 0) return false;
    return sizeof(XChunk16) * (size_t)stream_token_tile(M, pick_steps(cpr)) * (size_t)(cpr + 1) <=
           kLdsLimit;
}

bool w4a8_stream_supported(int64_t M, int64_t k_pad, bool fused_quant) {
    const int64_t cpr = k_pad / kChunkCols;
    if (pick_steps(cpr) == 0) return false;
    return w4a8_lds_bytes(stream_token_tile(M, pick_steps(cpr)), k_pad, fused_quant) <=
           kLdsLimit;
}

hipError_t launch_gemv_stream(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                              const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                              int64_t d_out, int64_t d_in, int64_t k_pad, int chunk_group_shift,
                              int64_t n_groups, void *y, int64_t ldy, bool out_f32,
                              hipStream_t stream) {
    const int T = pick_steps(k_pad / kChunkCols);
    int tile = stream_token_tile(M, T);
    // the kernel addresses a tile's activations with 31-bit byte offsets; one token always fits
    if (((int64_t)(tile - 1) * ldx + k_pad) * 2 >= (int64_t)kOutOfRange) tile = 1;
    const size_t out_elem = out_f32 ? sizeof(float) : sizeof(uint16_t);
    const bool zp = zeros != nullptr;
    for (int64_t m0 = 0; m0 < M; m0 += tile) {
        const int mt = static_cast<int>(M - m0 < tile ? M - m0 : tile);
        const uint16_t *xm = x + m0 * ldx;
        void *ym = static_cast<char *>(y) + m0 * ldy * out_elem;
        hipError_t err;
        if (tile == 1)
            err = launch_w4a16_stream_mt<1>(T, zp, xm, ldx, mt, qweight, scales, zeros, bias,
                                            d_out, d_in, k_pad, chunk_group_shift, n_groups, ym,
                                            ldy, out_f32, stream);
        else if (tile == 2)
            err = launch_w4a16_stream_mt<2>(T, zp, xm, ldx, mt, qweight, scales, zeros, bias,
                                            d_out, d_in, k_pad, chunk_group_shift, n_groups, ym,
                                            ldy, out_f32, stream);
        else
            err = launch_w4a16_stream_mt<4>(T, zp, xm, ldx, mt, qweight, scales, zeros, bias,
                                            d_out, d_in, k_pad, chunk_group_shift, n_groups, ym,
                                            ldy, out_f32, stream);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

// act: int8 codes [M][ldq] with their token scales in s_x (fused_quant false), or bf16 x
// [M][ldq] quantized inside the kernel, the scales written to s_x if it is given (true).
hipError_t launch_w4a8_stream(const void *act, bool fused_quant, float *s_x, int64_t M,
                              int64_t ldq, const uint8_t *qweight, const uint16_t *s_w,
                              const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                              void *y, int64_t ldy, bool out_f32, int32_t *acc,
                              hipStream_t stream) {
    const int T = pick_steps(k_pad / kChunkCols);
    int tile = stream_token_tile(M, T);
    const int64_t eb = fused_quant ? 2 : 1;  // bytes per activation
    // the kernel addresses a tile's activations with 31-bit byte offsets; one token always fits
    if (((int64_t)(tile - 1) * ldq + k_pad) * eb >= (int64_t)kOutOfRange) tile = 1;
    const size_t out_elem = out_f32 ? sizeof(float) : sizeof(uint16_t);
    for (int64_t m0 = 0; m0 < M; m0 += tile) {
        const int mt = static_cast<int>(M - m0 < tile ? M - m0 : tile);
        const void *am_act = static_cast<const char *>(act) + m0 * ldq * eb;
        float *sm = s_x ? s_x + m0 : nullptr;
        void *ym = static_cast<char *>(y) + m0 * ldy * out_elem;
        int32_t *am = acc ? acc + m0 * d_out : nullptr;
        hipError_t err;
#define W4_W4A8_TILE(MTV)                                                                         \
    (fused_quant ? launch_w4a8_stream_mt<MTV, true>(T, am_act, ldq, mt, sm, qweight, s_w, bias,   \
                                                    d_out, d_in, k_pad, ym, ldy, out_f32, am,     \
                                                    stream)                                       \
                 : launch_w4a8_stream_mt<MTV, false>(T, am_act, ldq, mt, sm, qweight, s_w, bias,  \
                                                     d_out, d_in, k_pad, ym, ldy, out_f32, am,    \
                                                     stream))
        if (tile == 1)
            err = W4_W4A8_TILE(1);
        else if (tile == 2)
            err = W4_W4A8_TILE(2);
        else
            err = W4_W4A8_TILE(4);
#undef W4_W4A8_TILE
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace w4
