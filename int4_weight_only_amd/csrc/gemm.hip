// gemm.hip -- W4A16 prefill GEMM for gfx950 on the bf16 matrix cores.
//
// Pages: [Lab5] "Lab 5: Gemma4 端到端推理优化" (sections "Prefill和Decode分流": large M runs a
// dense matrix product after dequantization, amortized over many tokens; "融合INT4反量化与矩阵乘":
// no dense weight is written back to memory).  The TPU page ("Yeniden paketlenmiş QAT Gemma 4
// 26B-A4B ...", section "vLLM'in TPU backend'inde değişen ne oldu") dequantizes each weight chunk
// in fast on-chip memory before the multiply; here the on-chip memory is LDS.
//
// Exact weights as two bf16 halves.  A weight tile is dequantized on its way to LDS to the fp32
// value w = s * (c - z) (exact: an 8-bit scale times an integer of at most 8 bits, computed as
// fma(c, s, -(z * s)) with z * s exact), and split into
//     hi = w with the low 16 bits cleared,   lo = w - hi   (exact; at most 8 significant bits),
// both exact bf16 values with hi + lo = w.  The product runs as X * HI^T + X * LO^T on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation: twice the matrix work of a bf16 weight, but
// the activations stay untouched bf16 and no per-group fp32 rescale of the accumulators is
// needed, which at 32-column groups would cost as much vector time as the matrix product.
// (A zero point that is not an integer of magnitude <= 240 -- never produced by w4_pack -- makes w
// a rounded fp32 value and the split keeps its top 16 significant bits.)
//
// Tiling: 256 threads (4 waves, 2 x 2); block tile BM tokens x 128 output channels; K step 32
// (one MFMA deep; every 32-column step lies in one group).  Each wave owns (BM/2) x 64 outputs.
// LDS holds two stages of {x tile, hi tile, lo tile}; global loads run two steps ahead of the
// matrix work through two register sets.  Blocks are numbered so that each XCD (blocks are
// dealt to the 8 XCDs round-robin) works on consecutive output-channel tiles and shares their
// weights in its L2.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int BN = 128, BK = 32;
constexpr int kThreads = 256;
constexpr int kStride = BK + 8;  // bf16 elements per LDS row (padded against bank conflicts)
constexpr int kXcds = 8;

template <int BM>
struct Stage {
    uint16_t x[BM * kStride];
    uint16_t hi[BN * kStride];
    uint16_t lo[BN * kStride];
};

// Registers of one step's global loads: per thread BM/128 x-rows x 16 columns and one weight row
// x 16 codes, with that row's scale and zero point.
template <int BM>
struct Loaded {
    uint4 x[BM / 128][2];
    uint2 w;
    uint16_t s_bits, z_bits;  // raw bf16; converted only when stored (no early use of a load)
    int step;
};

// Mask of the bf16 pair at elements (e, e + 1) of a chunk with `left` valid elements.
__device__ __forceinline__ uint32_t keep_pair(int left, int e) {
    return left >= e + 2 ? 0xFFFFFFFFu : (left == e + 1 ? 0x0000FFFFu : 0u);
}

// The fp32 weights s * (c - z) of the 4 codes held as bytes in `b`, split into bf16 hi and lo
// halves; hi2/lo2 receive 2 dwords each (columns in byte order).
__device__ __forceinline__ void split4(uint32_t b, float s, float zs, uint32_t *hi2,
                                       uint32_t *lo2) {
    float w[4];
    w[0] = fmaf(static_cast<float>(b & 0xFFu), s, zs);
    w[1] = fmaf(static_cast<float>((b >> 8) & 0xFFu), s, zs);
    w[2] = fmaf(static_cast<float>((b >> 16) & 0xFFu), s, zs);
    w[3] = fmaf(static_cast<float>(b >> 24), s, zs);
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t u = __float_as_uint(w[e]);
        h[e] = u & 0xFFFF0000u;
        l[e] = __float_as_uint(w[e] - __uint_as_float(h[e]));  // exact, low 16 bits zero
    }
    hi2[0] = __builtin_amdgcn_perm(h[1], h[0], 0x07060302u);
    hi2[1] = __builtin_amdgcn_perm(h[3], h[2], 0x07060302u);
    lo2[0] = __builtin_amdgcn_perm(l[1], l[0], 0x07060302u);
    lo2[1] = __builtin_amdgcn_perm(l[3], l[2], 0x07060302u);
}

template <int BM, bool ZP>
__global__ void __launch_bounds__(kThreads) gemm_w4a16_kernel(
    const uint16_t *__restrict__ x, int M, int64_t ldx, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int d_out, int d_in, int64_t row_bytes,
    int steps_per_group, int n_groups, int n_steps, int tiles_m, int tiles_n,
    void *__restrict__ y, int64_t ldy, int out_f32) {
    constexpr int WM = BM / 2;   // rows of a wave tile
    constexpr int TM = WM / 16;  // 16-row MFMA tiles per wave
    constexpr int XR = BM / 128; // x rows loaded per thread
    __shared__ __attribute__((aligned(16))) Stage<BM> st[2];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int wm = wid >> 1, wn = wid & 1;

    // XCD-aware tile order: hardware block b runs on XCD b % 8; renumber so that the blocks of
    // one XCD are consecutive tiles, M fastest (the tokens tiles of one weight tile together).
    const int nblocks = tiles_m * tiles_n;
    const int b = static_cast<int>(blockIdx.x);
    int t = b;
    if (nblocks % kXcds == 0) t = (b % kXcds) * (nblocks / kXcds) + b / kXcds;
    const int tile_m = t % tiles_m, tile_n = t / tiles_m;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // loader roles: thread -> (row, 16-column half of the 32-column step)
    const int ld_row = tid >> 1;
    const int ld_half = tid & 1;
    const int wrow = n0 + ld_row;
    const bool wrow_ok = wrow < d_out;

    // Every load is unconditional (rows and columns are clamped into the arrays; data outside
    // them is masked when it is stored to LDS): a load behind a branch would make the compiler's
    // memory-counter waits drain the loads that run ahead.
    auto load_step = [&](int step, Loaded<BM> &L) {
        const int k0 = step * BK + 16 * ld_half;
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            const int xm = m0 + ld_row + 128 * r;
            const uint16_t *xp = x + static_cast<int64_t>(xm < M ? xm : M - 1) * ldx;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int col = k0 + 8 * p;
                L.x[r][p] = *reinterpret_cast<const uint4 *>(xp + (col < d_in ? col : 0));
            }
        }
        const int G = step / steps_per_group;
        const int wr = wrow_ok ? wrow : d_out - 1;
        L.w = *reinterpret_cast<const uint2 *>(qweight + static_cast<int64_t>(wr) * row_bytes +
                                               k0 / 2);
        const int64_t gi = static_cast<int64_t>(wr) * n_groups + G;
        L.s_bits = scales[gi];
        if (ZP) L.z_bits = zeros[gi];
        L.step = step;
    };

    auto store_step = [&](Loaded<BM> &L, Stage<BM> &S) {
        // Only the last token tile and the step that reaches d_in hold data to mask (a
        // block-uniform test): token rows >= M and columns >= d_in become 0.
        if (m0 + BM > M || (L.step + 1) * BK > d_in) {
#pragma unroll
            for (int r = 0; r < XR; ++r) {
                const int xm = m0 + ld_row + 128 * r;
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const int left = xm < M ? d_in - (L.step * BK + 16 * ld_half + 8 * p) : 0;
                    L.x[r][p].x &= keep_pair(left, 0);
                    L.x[r][p].y &= keep_pair(left, 2);
                    L.x[r][p].z &= keep_pair(left, 4);
                    L.x[r][p].w &= keep_pair(left, 6);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < XR; ++r) {
            uint16_t *xd = &S.x[(ld_row + 128 * r) * kStride + 16 * ld_half];
            *reinterpret_cast<uint4 *>(xd) = L.x[r][0];
            *reinterpret_cast<uint4 *>(xd + 8) = L.x[r][1];
        }
        const float sv = wrow_ok ? bf16_to_f32(L.s_bits) : 0.0f;
        const float zv = ZP ? bf16_to_f32(L.z_bits) : 8.0f;
        const float zs = -(zv * sv);
        // 16 codes: bytes of the even columns (w & 0x0F0F0F0F) and odd columns ((w >> 4) & ...)
        uint32_t hi[8], lo[8];
        const uint32_t wv[2] = {L.w.x, L.w.y};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t ev = wv[d] & 0x0F0F0F0Fu;
            const uint32_t od = (wv[d] >> 4) & 0x0F0F0F0Fu;
            // interleave to column order c0 c1 c2 c3 (bytes e0 o0 e1 o1) and c4..c7
            const uint32_t c03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);
            const uint32_t c47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);
            split4(c03, sv, zs, &hi[4 * d], &lo[4 * d]);
            split4(c47, sv, zs, &hi[4 * d + 2], &lo[4 * d + 2]);
        }
        uint16_t *hd = &S.hi[ld_row * kStride + 16 * ld_half];
        uint16_t *ldp = &S.lo[ld_row * kStride + 16 * ld_half];
        *reinterpret_cast<uint4 *>(hd) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *reinterpret_cast<uint4 *>(hd + 8) = make_uint4(hi[4], hi[5], hi[6], hi[7]);
        *reinterpret_cast<uint4 *>(ldp) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<uint4 *>(ldp + 8) = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    };

    floatx4_t acc[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int frag_row = lane & 15;
    const int frag_k = 8 * (lane >> 4);
    auto compute = [&](const Stage<BM> &S) {
        bf16x8_t a[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t *>(
                &S.x[(wm * WM + i * 16 + frag_row) * kStride + frag_k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int wr = (wn * 64 + j * 16 + frag_row) * kStride + frag_k;
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&S.hi[wr]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&S.lo[wr]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bh, acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bl, acc[i][j], 0, 0, 0);
        }
    };

    // One step: refill the free register set with step + 2 (the last steps reload the final
    // step, unconditionally), multiply from the current stage, then dequantize step + 1 into
    // the other stage (last read before the previous barrier; after the final step this writes
    // a stage nobody reads).
    auto run_step = [&](int step, Loaded<BM> &free_set, Loaded<BM> &next_set,
                        const Stage<BM> &cur, Stage<BM> &nxt) {
        load_step(step + 2 < n_steps ? step + 2 : n_steps - 1, free_set);
        compute(cur);
        store_step(next_set, nxt);
        __syncthreads();
    };

    Loaded<BM> R0, R1;
    load_step(0, R0);
    load_step(n_steps > 1 ? 1 : 0, R1);
    store_step(R0, st[0]);
    __syncthreads();

    int step = 0;
    for (; step + 1 < n_steps; step += 2) {
        run_step(step, R0, R1, st[0], st[1]);
        run_step(step + 1, R1, R0, st[1], st[0]);
    }
    if (step < n_steps) run_step(step, R0, R1, st[0], st[1]);

    // epilogue: D[i][j] of a 16x16 tile sits in lane j + 16 * (i / 4), element i % 4
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + frag_row;
        if (n >= d_out) continue;
        const float bv = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * WM + i * 16 + 4 * (lane >> 4) + r;
                if (m < M) store_out(y, static_cast<int64_t>(m) * ldy + n, acc[i][j][r] + bv,
                                     out_f32 != 0);
            }
        }
    }
}

template <int BM>
hipError_t launch_bm(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                     const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                     int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span, int64_t n_groups,
                     void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    const int steps_per_group = static_cast<int>(span / BK);
    const int n_steps = static_cast<int>(k_pad / BK);
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((d_out + BN - 1) / BN);
    if (static_cast<int64_t>(tiles_m) * tiles_n > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n));
    const int64_t row_bytes = k_pad / 2;
    if (zeros)
        hipLaunchKernelGGL((gemm_w4a16_kernel<BM, true>), grid, dim3(kThreads), 0, stream, x,
                           static_cast<int>(M), ldx, qweight, scales, zeros, bias,
                           static_cast<int>(d_out), static_cast<int>(d_in), row_bytes,
                           steps_per_group, static_cast<int>(n_groups), n_steps, tiles_m, tiles_n,
                           y, ldy, out_f32 ? 1 : 0);
    else
        hipLaunchKernelGGL((gemm_w4a16_kernel<BM, false>), grid, dim3(kThreads), 0, stream, x,
                           static_cast<int>(M), ldx, qweight, scales, zeros, bias,
                           static_cast<int>(d_out), static_cast<int>(d_in), row_bytes,
                           steps_per_group, static_cast<int>(n_groups), n_steps, tiles_m, tiles_n,
                           y, ldy, out_f32 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, void *y, int64_t ldy, bool out_f32, hipStream_t stream) {
    // 256-token tiles when they still give every compute unit two blocks, else 128.
    const int64_t tiles_n = (d_out + BN - 1) / BN;
    const int64_t blocks256 = ((M + 255) / 256) * tiles_n;
    if (M > 128 && blocks256 >= 2 * static_cast<int64_t>(device_cu_count()))
        return launch_bm<256>(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, k_pad, span,
                              n_groups, y, ldy, out_f32, stream);
    return launch_bm<128>(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, k_pad, span,
                          n_groups, y, ldy, out_f32, stream);
}

}  // namespace w4
