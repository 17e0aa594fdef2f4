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
// (one MFMA deep; every 32-column step lies in one group).  Each wave owns (BM/2) x 64 outputs,
// with the accumulators in VGPRs; two blocks share a compute unit.  Activations go from memory
// straight into a ring of three LDS stages (buffer_load ... lds), two steps ahead of the matrix
// work; packed weights go to registers, also two steps ahead, and are dequantized into one of
// two LDS stages while the current step multiplies.  One barrier per step, without a memory
// fence, so that loads stay in flight across it.  Blocks are numbered so that each XCD (blocks
// are dealt to the 8 XCDs round-robin) works on consecutive output-channel tiles and shares
// their weights in its L2.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int BN = 128, BK = 32;
constexpr int kThreads = 256;
constexpr int kXcds = 8;

// LDS rows are BK = 32 bf16 (64 bytes, four 16-byte chunks) with no padding; chunk c of row r is
// stored at chunk position c ^ ((r >> 2) & 3).  The 16 rows read by one 16-lane phase of a
// fragment load, and the 8 rows x 2 halves written by one phase of the tile stores, then fall
// into 16 different 16-byte bank groups.
__device__ __forceinline__ int lds_at(int row, int chunk) {
    return row * BK + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// One direct global->LDS load: 16 bytes per lane from `off` within the descriptor (0 when out of
// range) into LDS at `lds` + 16 * lane.
__device__ __forceinline__ void load_lds16(rsrc_t r, uint16_t *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                             off, 0, 0, 0);
}

// Block barrier without a memory fence.  The direct global->LDS loads of later steps stay in
// flight across it (a fenced barrier would drain them); the caller's own LDS stores are
// completed first (lgkmcnt(0)), and the loads of the stage read after the barrier have landed
// because the vector-memory counter is in order: they were issued before the weight loads that
// the caller has already waited for.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Registers of one step's weight loads (one row x 16 codes per thread, with that row's raw
// scale and zero point, converted only when stored so that nothing uses a load early), two steps
// ahead.
struct WLoad {
    uint2 w;
    uint16_t s_bits, z_bits;
};

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
__global__ void __launch_bounds__(kThreads, 2) gemm_w4a16_kernel(
    const uint16_t *__restrict__ x, int M, int64_t ldx, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int d_out, int d_in, int64_t row_bytes,
    int steps_per_group, int n_groups, int n_steps, int tiles_m, int tiles_n,
    void *__restrict__ y, int64_t ldy, int out_f32) {
    constexpr int WM = BM / 2;   // rows of a wave tile
    constexpr int TM = WM / 16;  // 16-row MFMA tiles per wave
    constexpr int XR = BM / 128; // x rows loaded per thread
    // Shared memory: a ring of three activation stages (filled two steps ahead by direct
    // global->LDS loads) and two stages of dequantized weight halves.  Every stage is an array of
    // its own and the step loop is unrolled so that each access names its array: the compiler
    // then sees that a direct load in flight does not touch the stage being read or written (it
    // would otherwise wait for the load before every such access).
    __shared__ __attribute__((aligned(16))) uint16_t sx0[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sx1[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sx2[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t shi[2][BN * BK];
    __shared__ __attribute__((aligned(16))) uint16_t slo[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wid >> 1, wn = wid & 1;

    // XCD-aware tile order: hardware block b runs on XCD b % 8; renumber so that the blocks of
    // one XCD are consecutive tiles, M fastest (the tokens tiles of one weight tile together).
    const int nblocks = tiles_m * tiles_n;
    const int b = static_cast<int>(blockIdx.x);
    int t = b;
    if (nblocks % kXcds == 0) t = (b % kXcds) * (nblocks / kXcds) + b / kXcds;
    const int tile_m = t % tiles_m, tile_n = t / tiles_m;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // Activations: direct global->LDS loads (buffer_load ... lds).  One instruction moves 16 rows
    // x 64 bytes of a step: lane l lands in LDS slot l (row l / 4, chunk position l % 4), so it
    // fetches the chunk that the swizzled layout keeps there.  Wave w owns rows
    // [w * BM / 4, (w + 1) * BM / 4) of the tile, XS slabs of 16 rows, each with a descriptor that
    // covers only the slab's rows below M: a row >= M, or a chunk starting at or beyond d_in, gets
    // an offset outside it and lands as zeros.  (Rows >= M only feed outputs that are never
    // stored; a chunk that straddles d_in is trimmed after it lands.)
    constexpr int XS = BM / 64;
    const int x_chunk = (lane & 3) ^ (lane >> 4);
    const uint32_t x_row_off = static_cast<uint32_t>(lane >> 2) * static_cast<uint32_t>(ldx) * 2u;
    rsrc_t x_rsrc[XS];
#pragma unroll
    for (int q = 0; q < XS; ++q) {
        const int grow0 = m0 + wid * (BM / 4) + q * 16;
        const int rows = grow0 < M ? (M - grow0 < 16 ? M - grow0 : 16) : 0;
        x_rsrc[q] = make_rsrc(rows > 0 ? x + static_cast<int64_t>(grow0) * ldx : x,
                              static_cast<uint32_t>(rows) * static_cast<uint32_t>(ldx) * 2u);
    }
    auto dma_x = [&](int step, uint16_t *stage) {
        const int col = step * BK + 8 * x_chunk;
        const uint32_t off = col < d_in ? x_row_off + 2u * static_cast<uint32_t>(col) : kOutOfRange;
#pragma unroll
        for (int q = 0; q < XS; ++q)
            load_lds16(x_rsrc[q], &stage[(wid * (BM / 4) + q * 16) * BK], off);
    };
    // Zero the columns >= d_in of the chunk that straddles d_in (only when d_in % 8 != 0, in the
    // one step that holds it), after this wave's loads of that stage have landed.
    auto trim_x = [&](int step, uint16_t *stage) {
        if ((d_in & 7) != 0 && d_in / BK == step) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            const int keep = d_in - (step * BK + 8 * x_chunk);  // valid columns of the chunk
            if (keep > 0 && keep < 8) {
                uint32_t m[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    m[e] = 2 * e + 2 <= keep ? 0xFFFFFFFFu : (2 * e + 1 == keep ? 0x0000FFFFu : 0u);
#pragma unroll
                for (int q = 0; q < XS; ++q) {
                    uint4 *p = reinterpret_cast<uint4 *>(&stage[(wid * (BM / 4) + q * 16) * BK + 8 * lane]);
                    uint4 v = *p;
                    v.x &= m[0];
                    v.y &= m[1];
                    v.z &= m[2];
                    v.w &= m[3];
                    *p = v;
                }
            }
        }
    };

    // loader roles for the weights: thread -> (row, 16-column half of the 32-column step)
    const int ld_row = tid >> 1;
    const int ld_half = tid & 1;
    const int wrow = n0 + ld_row;
    const bool wrow_ok = wrow < d_out;

    // Weight loads are unconditional (the row is clamped into the matrix and masked when
    // stored): a load behind a branch would make the compiler's memory-counter waits drain the
    // loads that run ahead.
    auto load_w = [&](int step, WLoad &L) {
        const int k0 = step * BK + 16 * ld_half;
        const int G = step / steps_per_group;
        const int wr = wrow_ok ? wrow : d_out - 1;
        L.w = *reinterpret_cast<const uint2 *>(qweight + static_cast<int64_t>(wr) * row_bytes +
                                               k0 / 2);
        const int64_t gi = static_cast<int64_t>(wr) * n_groups + G;
        L.s_bits = scales[gi];
        if (ZP) L.z_bits = zeros[gi];
    };

    // Weights of a loaded step -> exact hi/lo bf16 halves in a stage (straight-line vector code
    // that the scheduler can interleave with the matrix instructions of the current step).
    auto store_w = [&](const WLoad &L, int stage) {
        const float sv = wrow_ok ? bf16_to_f32(L.s_bits) : 0.0f;
        const float zv = ZP ? bf16_to_f32(L.z_bits) : 8.0f;
        const float zs = -(zv * sv);
        // 16 codes = two 16-byte chunks of the stage (8 columns per packed dword); per dword the
        // bytes of the even columns (w & 0x0F0F0F0F) and odd columns ((w >> 4) & 0x0F0F0F0F)
        const uint32_t wv[2] = {L.w.x, L.w.y};
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t ev = wv[d] & 0x0F0F0F0Fu;
            const uint32_t od = (wv[d] >> 4) & 0x0F0F0F0Fu;
            // interleave to column order c0 c1 c2 c3 (bytes e0 o0 e1 o1) and c4..c7
            const uint32_t c03 = __builtin_amdgcn_perm(od, ev, 0x05010400u);
            const uint32_t c47 = __builtin_amdgcn_perm(od, ev, 0x07030602u);
            uint32_t hi[4], lo[4];
            split4(c03, sv, zs, &hi[0], &lo[0]);
            split4(c47, sv, zs, &hi[2], &lo[2]);
            const int c = lds_at(ld_row, 2 * ld_half + d);
            *reinterpret_cast<uint4 *>(&shi[stage][c]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&slo[stage][c]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
    };

    floatx4_t acc[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // A lane reads row frag_row (+ multiples of 16) at k-chunk lane / 16 of every fragment.
    const int frag_row = lane & 15;
    const int frag_off = lds_at(frag_row, lane >> 4);
    auto compute = [&](const uint16_t *xstage, int wstage) {
        bf16x8_t a[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t *>(
                &xstage[(wm * WM + i * 16) * BK + frag_off]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int wr = (wn * 64 + j * 16) * BK + frag_off;
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&shi[wstage][wr]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&slo[wstage][wr]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bh, acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bl, acc[i][j], 0, 0, 0);
        }
    };

    // One step: start the activations of step + 2 into the free activation stage and the
    // weights of step + 2 into the free register set (the last steps reload the final step,
    // unconditionally), multiply from the current stages, and dequantize the weights of step + 1
    // into the other weight stage (last read before the previous barrier; after the final step
    // this writes a stage nobody reads).  Waiting for the weights of step + 1 also covers the
    // activations of step + 1, which were issued before them.
    const int last = n_steps - 1;
    auto run_step = [&](int step, uint16_t *xcur, uint16_t *xnext, uint16_t *xfree,
                        WLoad &free_set, const WLoad &next_set, int ws) {
        dma_x(step + 2 < n_steps ? step + 2 : last, xfree);
        load_w(step + 2 < n_steps ? step + 2 : last, free_set);
        // keep the loads ahead of the vector work on the previous set: a wait for that set placed
        // before them would have to drain every load in flight
        __builtin_amdgcn_sched_barrier(0);
        compute(xcur, ws);
        store_w(next_set, ws ^ 1);
        trim_x(step + 1, xnext);
        stage_barrier();
    };

    WLoad W0, W1;
    dma_x(0, sx0);
    load_w(0, W0);
    dma_x(n_steps > 1 ? 1 : 0, sx1);
    load_w(n_steps > 1 ? 1 : 0, W1);
    store_w(W0, 0);
    trim_x(0, sx0);
    __syncthreads();

    // steps 6i .. 6i + 5: activation stages rotate with period 3, weight sets with period 2
    int step = 0;
    for (; step + 5 < n_steps; step += 6) {
        run_step(step + 0, sx0, sx1, sx2, W0, W1, 0);
        run_step(step + 1, sx1, sx2, sx0, W1, W0, 1);
        run_step(step + 2, sx2, sx0, sx1, W0, W1, 0);
        run_step(step + 3, sx0, sx1, sx2, W1, W0, 1);
        run_step(step + 4, sx1, sx2, sx0, W0, W1, 0);
        run_step(step + 5, sx2, sx0, sx1, W1, W0, 1);
    }
    // the remaining 0..5 steps continue the same rotation
    if (step < n_steps) run_step(step, sx0, sx1, sx2, W0, W1, 0);
    if (step + 1 < n_steps) run_step(step + 1, sx1, sx2, sx0, W1, W0, 1);
    if (step + 2 < n_steps) run_step(step + 2, sx2, sx0, sx1, W0, W1, 0);
    if (step + 3 < n_steps) run_step(step + 3, sx0, sx1, sx2, W1, W0, 1);
    if (step + 4 < n_steps) run_step(step + 4, sx1, sx2, sx0, W0, W1, 0);
    // the last steps reloaded the final step: let those loads land before the block ends
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

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
