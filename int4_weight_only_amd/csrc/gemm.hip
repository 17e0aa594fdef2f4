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
// Tiling: 512 threads (8 waves, 2 x 4), one block per compute unit; block tile BM tokens x 256
// output channels; K step 32 (one MFMA deep; every 32-column step lies in one group).  Each wave
// owns (BM/2) x 64 outputs, with the accumulators in VGPRs.
//
// Everything a step reads from memory arrives by direct global->LDS loads (buffer_load ... lds),
// so that no wave ever waits for a load in its registers:
//   * activations: a ring of three stages, two steps ahead;
//   * packed weights and their scales (and zero points): chunks of four steps (64 bytes of every
//     weight row, four scales per row), double-buffered, one chunk ahead.
// The cost that bounds such a kernel on this part is the number of distinct cache lines its loads
// touch per step, not their bytes: a 256-row weight step touches 256 lines whichever way it is
// loaded, a four-step chunk touches the same lines once for four steps, and the 256-channel tile
// halves the activation lines per matrix instruction against a 128-channel tile.
// Each step dequantizes the next step's weights from the chunk into one of two LDS stages of
// exact hi/lo halves while the matrix cores work on the current one.  One barrier per step,
// without a memory fence, so that loads stay in flight across it.  Blocks are numbered so that
// each XCD (blocks are dealt to the 8 XCDs round-robin) works on consecutive tiles and shares
// their weights in its L2.
#include <type_traits>

#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int BN = 256, BK = 32;
constexpr int KC = 4;          // steps per weight chunk
constexpr int kThreads = 512;  // 8 waves
constexpr int kXcds = 8;
constexpr int kPeriod = 24;    // lcm of the stage rings: 3 activation, 2 weight, 2 chunk (x 4 steps)

// LDS layout of a [rows][BK = 32] bf16 tile: blocks of 16 rows (1 KiB), and inside a block the
// 16-byte chunk c (columns 8c .. 8c + 7) of row r at slot 16 c + r, chunk-major.  The matrix-core
// operand fragment of 16 rows x 32 columns (lane l: row l % 16, chunk l / 16) is then one
// contiguous 1 KiB read, lane l at byte 16 l, which the LDS serves at its full rate; a row-major
// tile (rows of 64 bytes), swizzled or not, serves the same fragment at half that rate.
__device__ __forceinline__ int lds_at(int row, int chunk) {
    return (row >> 4) * (16 * BK) + chunk * 128 + (row & 15) * 8;
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// Direct global->LDS loads: `bytes` (16: the 16 bytes at `off`; 2: the 16-bit value at `off`,
// zero-extended to a dword) per lane from the descriptor (zeros when out of range) into LDS at
// `lds` + bytes_per_slot * lane (16 or 4).
__device__ __forceinline__ void load_lds16(rsrc_t r, void *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void load_lds2(rsrc_t r, void *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 2, off, 0, 0, 0);
}

// s_waitcnt with lgkmcnt(0), expcnt(7) and vmcnt(N) (gfx9 encoding: vmcnt bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Block barrier without a memory fence, after this wave's LDS stores (lgkmcnt(0)) and all but
// its N most recent direct loads (vmcnt(N)) have completed.  The empty asm statements keep the
// compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    asm volatile("" ::: "memory");
    wait_vm_lgkm0<N>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

template <int BM, bool ZP, bool SW>
__global__ void __launch_bounds__(kThreads, 1) gemm_w4a16_kernel(
    const uint16_t *__restrict__ x, int M, int64_t ldx, const uint8_t *__restrict__ qweight,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const uint16_t *__restrict__ bias, int d_out, int d_in, int64_t row_bytes,
    int steps_per_group, int n_groups, int n_steps, int tiles_m, int tiles_n,
    void *__restrict__ y, int64_t ldy, int out_f32) {
    constexpr int WM = BM / 2;    // rows of a wave tile
    constexpr int TM = WM / 16;   // 16-row MFMA tiles per wave
    constexpr int XI = BM / 128;  // activation loads per wave per step (16 rows each)
    // chunk loads per wave per chunk (codes, scales, zeros: 2 each; with scale windows the codes
    // only)
    constexpr int CI = SW ? 2 : (ZP ? 6 : 4);
    // Shared memory, every stage an array of its own: the step loop is unrolled over the period
    // of all rings so that each access names its array, and the compiler then sees that a direct
    // load in flight does not touch the stage being read or written (it would otherwise wait for
    // the load before every such access).
    __shared__ __attribute__((aligned(16))) uint16_t sx0[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sx1[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sx2[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t shi0[BN * BK];
    __shared__ __attribute__((aligned(16))) uint16_t shi1[BN * BK];
    __shared__ __attribute__((aligned(16))) uint16_t slo0[BN * BK];
    __shared__ __attribute__((aligned(16))) uint16_t slo1[BN * BK];
    // weight chunk: 16 blocks of 16 rows; in block b the 16 bytes of row 16 b + r for step k of the
    // chunk at byte 1024 b + 256 k + 16 r
    __shared__ __attribute__((aligned(16))) uint8_t sq0[BN * KC * 16];
    __shared__ __attribute__((aligned(16))) uint8_t sq1[BN * KC * 16];
    // scale (zero point) bits of row 16 b + r for step k of the chunk in dword 64 b + 16 k + r
    __shared__ __attribute__((aligned(16))) uint32_t ss0[SW ? 1 : BN * KC];
    __shared__ __attribute__((aligned(16))) uint32_t ss1[SW ? 1 : BN * KC];
    // scale windows (SW): the bf16 scales of 8 consecutive groups of every row, row r at element
    // 8 r, a ring of three; waves 4..7 aim their (empty) window loads at a dummy
    __shared__ __attribute__((aligned(16))) uint16_t sw0[SW ? BN * 8 : 1];
    __shared__ __attribute__((aligned(16))) uint16_t sw1[SW ? BN * 8 : 1];
    __shared__ __attribute__((aligned(16))) uint16_t sw2[SW ? BN * 8 : 1];
    __shared__ __attribute__((aligned(16))) uint16_t swd[SW ? 64 * 8 : 1];
    __shared__ __attribute__((aligned(16))) uint32_t sz0[ZP ? BN * KC : 1];
    __shared__ __attribute__((aligned(16))) uint32_t sz1[ZP ? BN * KC : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wid >> 2, wn = wid & 3;

    // XCD-aware tile order: hardware block b runs on XCD b % 8; renumber so that the blocks of
    // one XCD are consecutive tiles, M fastest (the token tiles of one weight tile together).
    const int nblocks = tiles_m * tiles_n;
    const int b = static_cast<int>(blockIdx.x);
    int t = b;
    if (nblocks % kXcds == 0) t = (b % kXcds) * (nblocks / kXcds) + b / kXcds;
    const int tile_m = t % tiles_m, tile_n = t / tiles_m;
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    // Activations: one instruction moves 16 rows x 64 bytes of a step; lane l lands in LDS slot l
    // of a 16-row block, so it fetches row l % 16, chunk l / 16.  Wave w owns rows
    // [w * BM / 8, (w + 1) * BM / 8) of the tile, XI blocks of 16 rows, each with a descriptor
    // that covers only the block's rows below M: a row >= M, or a chunk starting at or beyond
    // d_in, gets an offset outside it and lands as zeros.  (Rows >= M only feed outputs that are
    // never stored; a chunk that straddles d_in is trimmed after it lands.)
    const int x_chunk = lane >> 4;
    const uint32_t x_row_off = static_cast<uint32_t>(lane & 15) * static_cast<uint32_t>(ldx) * 2u;
    rsrc_t x_rsrc[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int grow0 = m0 + wid * (BM / 8) + q * 16;
        const int rows = grow0 < M ? (M - grow0 < 16 ? M - grow0 : 16) : 0;
        x_rsrc[q] = make_rsrc(rows > 0 ? x + static_cast<int64_t>(grow0) * ldx : x,
                              static_cast<uint32_t>(rows) * static_cast<uint32_t>(ldx) * 2u);
    }
    auto dma_x = [&](int step, uint16_t *stage) {
        const int col = step * BK + 8 * x_chunk;
        const uint32_t off = col < d_in ? x_row_off + 2u * static_cast<uint32_t>(col) : kOutOfRange;
#pragma unroll
        for (int q = 0; q < XI; ++q)
            load_lds16(x_rsrc[q], &stage[(wid * (BM / 8) + q * 16) * BK], off);
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
                for (int q = 0; q < XI; ++q) {
                    uint4 *p = reinterpret_cast<uint4 *>(&stage[(wid * (BM / 8) + q * 16) * BK + 8 * lane]);
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

    // Weight chunks: wave w loads row blocks 2w and 2w + 1 (16 rows each) of the tile, each with
    // a descriptor that covers only its rows below d_out (rows beyond load zeros: zero codes and
    // a zero scale, so zero weights).  Codes: lane l fetches the 16 bytes of row l % 16 for step
    // l / 16 of the chunk (offsets past the row's end only occur in chunks beyond the last step,
    // whose contents are never used).  Scales and zero points: lane l fetches the 16-bit value of
    // row l % 16 for step l / 16, i.e. of group min(step / steps_per_group, n_groups - 1).
    rsrc_t q_rsrc[2], s_rsrc[2], z_rsrc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r0 = n0 + (2 * wid + h) * 16;
        const int rows = r0 < d_out ? (d_out - r0 < 16 ? d_out - r0 : 16) : 0;
        q_rsrc[h] = make_rsrc(rows > 0 ? qweight + static_cast<int64_t>(r0) * row_bytes : qweight,
                              static_cast<uint32_t>(rows * row_bytes));
        s_rsrc[h] = make_rsrc(rows > 0 ? scales + static_cast<int64_t>(r0) * n_groups : scales,
                              static_cast<uint32_t>(rows * n_groups * 2));
        if (ZP)
            z_rsrc[h] = make_rsrc(rows > 0 ? zeros + static_cast<int64_t>(r0) * n_groups : zeros,
                                  static_cast<uint32_t>(rows * n_groups * 2));
    }
    const uint32_t q_lane_off = static_cast<uint32_t>((lane & 15) * row_bytes + 16 * (lane >> 4));
    const uint32_t s_lane_row = static_cast<uint32_t>((lane & 15) * n_groups);
    auto dma_chunk = [&](int chunk, uint8_t *sq, uint32_t *ss, uint32_t *sz) {
        const int k0 = chunk * KC;
        const uint32_t qoff = q_lane_off + static_cast<uint32_t>(k0) * 16u;
        int g = (k0 + (lane >> 4)) / steps_per_group;
        g = g < n_groups ? g : n_groups - 1;
        const uint32_t soff = 2u * (s_lane_row + static_cast<uint32_t>(g));
#pragma unroll
        for (int h = 0; h < 2; ++h) load_lds16(q_rsrc[h], &sq[(2 * wid + h) * 1024], qoff);
        if (!SW) {
#pragma unroll
            for (int h = 0; h < 2; ++h) load_lds2(s_rsrc[h], &ss[(2 * wid + h) * 64], soff);
        }
        if (ZP) {
#pragma unroll
            for (int h = 0; h < 2; ++h) load_lds2(z_rsrc[h], &sz[(2 * wid + h) * 64], soff);
        }
    };

    // Scale windows (32-column groups, no zero points, n_groups % 8 == 0, 16-byte aligned scales):
    // one direct 16-byte load per lane brings the 8 scales of window w (groups 8 w .. 8 w + 7) of
    // one row -- waves 0..3 load 64 rows each, the other waves an empty load into a dummy, so
    // that every wave counts the same loads. A 256-row step then costs 32 lines instead of 64,
    // and 0.5 loads per wave instead of 4.
    rsrc_t w_rsrc = q_rsrc[0];
    uint32_t w_lane_off = kOutOfRange;
    if (SW) {
        const int r0 = n0 + 64 * (wid & 3);
        const int rows = r0 < d_out ? (d_out - r0 < 64 ? d_out - r0 : 64) : 0;
        w_rsrc = make_rsrc(rows > 0 ? scales + static_cast<int64_t>(r0) * n_groups : scales,
                           static_cast<uint32_t>(rows * n_groups * 2));
        if (wid < 4) w_lane_off = static_cast<uint32_t>(lane * n_groups * 2);
    }
    auto dma_window = [&](int window, uint16_t *buf) {
        const uint32_t off =
            wid < 4 ? w_lane_off + 16u * static_cast<uint32_t>(window) : kOutOfRange;
        load_lds16(w_rsrc, wid < 4 ? &buf[(wid & 3) * 64 * 8] : swd, off);
    };

    // Dequantizer roles: thread -> (row, 16-column half of the 32-column step); the 16 lanes of a
    // quarter wave take 16 consecutive rows and one half, so that their chunk reads and each of
    // their stage stores are contiguous in LDS.
    const int ld_row = (tid & 15) + 16 * (tid >> 5);
    const int ld_half = (tid >> 4) & 1;
    const int q_read = (ld_row >> 4) * 1024 + (ld_row & 15) * 16 + 8 * ld_half;
    const int s_read = (ld_row >> 4) * 64 + (ld_row & 15);

    // Step k of a chunk -> exact hi/lo bf16 halves in a weight stage.
    auto dequant = [&](int k, const uint8_t *sq, const uint32_t *ss, const uint32_t *sz,
                       const uint16_t *swb, int k8, uint16_t *shi, uint16_t *slo) {
        const uint2 wq = *reinterpret_cast<const uint2 *>(&sq[q_read + 256 * k]);
        const float sv = SW ? bf16_to_f32(swb[ld_row * 8 + k8]) : bf16_to_f32(ss[s_read + 16 * k]);
        const float zv = ZP ? bf16_to_f32(sz[s_read + 16 * k]) : 8.0f;
        const float zs = -(zv * sv);
        // 16 codes = two 16-byte chunks of the stage (8 columns per packed dword); per dword the
        // bytes of the even columns (w & 0x0F0F0F0F) and odd columns ((w >> 4) & 0x0F0F0F0F)
        const uint32_t wv[2] = {wq.x, wq.y};
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
            *reinterpret_cast<uint4 *>(&shi[c]) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
            *reinterpret_cast<uint4 *>(&slo[c]) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
    };

    floatx4_t acc[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // A lane reads row frag_row (+ multiples of 16) at k-chunk lane / 16 of every fragment.
    const int frag_row = lane & 15;
    const int frag_off = lds_at(frag_row, lane >> 4);  // = 8 * lane
    auto compute = [&](const uint16_t *xstage, const uint16_t *shi, const uint16_t *slo) {
        bf16x8_t a[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[i] = *reinterpret_cast<const bf16x8_t *>(
                &xstage[(wm * WM + i * 16) * BK + frag_off]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int wr = (wn * 64 + j * 16) * BK + frag_off;
            const bf16x8_t bh = *reinterpret_cast<const bf16x8_t *>(&shi[wr]);
            const bf16x8_t bl = *reinterpret_cast<const bf16x8_t *>(&slo[wr]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bh, acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bl, acc[i][j], 0, 0, 0);
        }
    };

    uint16_t *const sx[3] = {sx0, sx1, sx2};
    uint16_t *const shi[2] = {shi0, shi1};
    uint16_t *const slo[2] = {slo0, slo1};
    uint8_t *const sq[2] = {sq0, sq1};
    uint32_t *const ss[2] = {ss0, ss1};
    uint32_t *const sz[2] = {sz0, sz1};
    uint16_t *const swr[3] = {sw0, sw1, sw2};

    // Step s (P = s % kPeriod, known at compile time): start the activations of step s + 2 and,
    // at the first step of a chunk, the next chunk; multiply from the current stages; dequantize
    // step s + 1 from its chunk into the other weight stage (last read before the previous
    // barrier); then wait for what the next step reads and pass the barrier.
    //   vector-memory issue order: ... X(s+1) [CH(c+1) if s-1 opens chunk c] X(s+2) [CH if s opens]
    //   the next step reads X(s+1), and step 4c + 3 dequantizes from chunk c + 1; both are covered
    //   by waiting until only the loads issued after X(s+1) are in flight.
    // After the final step the loads run past the matrix (zeros or unused bytes) into stages
    // nobody reads.
    auto run_step = [&](int step, auto PP) {
        constexpr int P = decltype(PP)::value;
        constexpr int K = P % KC;
        constexpr int CB = (P / KC) % 2;  // chunk buffer of this step
        constexpr int CN = ((P + 1) / KC) % 2;  // chunk buffer of step s + 1
        dma_x(step + 2, sx[(P + 2) % 3]);
        if constexpr (K == 0) dma_chunk(step / KC + 1, sq[CB ^ 1], ss[CB ^ 1], sz[CB ^ 1]);
        // window w covers steps 8 w .. 8 w + 7; window w + 1 is loaded at step 8 w
        if constexpr (SW && P % 8 == 0) dma_window(step / 8 + 1, swr[(P / 8 + 1) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        compute(sx[P % 3], shi[P % 2], slo[P % 2]);
        dequant((P + 1) % KC, sq[CN], ss[CN], sz[CN], swr[((P + 1) / 8) % 3], (P + 1) % 8,
                shi[(P + 1) % 2], slo[(P + 1) % 2]);
        trim_x(step + 1, sx[(P + 1) % 3]);
        constexpr int N = XI + ((K == 0 || K == 1) ? CI : 0) +
                          (SW ? ((P % 8 == 0 || P % 8 == 1) ? 1 : 0) : 0);
        stage_barrier<N>();
    };

    // prologue: X(0), CH(0), [SW(0)], X(1); step 0's weights into stage 0
    dma_x(0, sx0);
    dma_chunk(0, sq0, ss0, sz0);
    if (SW) dma_window(0, sw0);
    dma_x(1, sx1);
    wait_vm_lgkm0<XI>();
    __syncthreads();
    dequant(0, sq0, ss0, sz0, sw0, 0, shi0, slo0);
    trim_x(0, sx0);
    __syncthreads();

    for (int s0 = 0; s0 < n_steps; s0 += kPeriod) {
        // the period unrolled; the final pass skips the steps from n_steps on (guards rather than
        // an exit per step: a loop with 24 exits costs the register allocator thousands of spills)
#define W4_STEP(p) \
        if (s0 + (p) < n_steps) run_step(s0 + (p), std::integral_constant<int, (p)>{});
        W4_STEP(0) W4_STEP(1) W4_STEP(2) W4_STEP(3) W4_STEP(4) W4_STEP(5)
        W4_STEP(6) W4_STEP(7) W4_STEP(8) W4_STEP(9) W4_STEP(10) W4_STEP(11)
        W4_STEP(12) W4_STEP(13) W4_STEP(14) W4_STEP(15) W4_STEP(16) W4_STEP(17)
        W4_STEP(18) W4_STEP(19) W4_STEP(20) W4_STEP(21) W4_STEP(22) W4_STEP(23)
#undef W4_STEP
    }
    // the loads that ran past the final step land before the block ends
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

template <int BM, bool SW>
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
    if (SW)
        hipLaunchKernelGGL((gemm_w4a16_kernel<BM, false, SW>), grid, dim3(kThreads), 0, stream, x,
                           static_cast<int>(M), ldx, qweight, scales, zeros, bias,
                           static_cast<int>(d_out), static_cast<int>(d_in), row_bytes,
                           steps_per_group, static_cast<int>(n_groups), n_steps, tiles_m, tiles_n,
                           y, ldy, out_f32 ? 1 : 0);
    else if (zeros)
        hipLaunchKernelGGL((gemm_w4a16_kernel<BM, true, false>), grid, dim3(kThreads), 0, stream, x,
                           static_cast<int>(M), ldx, qweight, scales, zeros, bias,
                           static_cast<int>(d_out), static_cast<int>(d_in), row_bytes,
                           steps_per_group, static_cast<int>(n_groups), n_steps, tiles_m, tiles_n,
                           y, ldy, out_f32 ? 1 : 0);
    else
        hipLaunchKernelGGL((gemm_w4a16_kernel<BM, false, false>), grid, dim3(kThreads), 0, stream, x,
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
    // 256-token tiles when they still give every compute unit a block, else 128.
    const int64_t tiles_n = (d_out + BN - 1) / BN;
    const int64_t blocks256 = ((M + 255) / 256) * tiles_n;
    const bool big = M > 128 && blocks256 >= static_cast<int64_t>(device_cu_count());
    // scale windows: symmetric 32-column groups with 16-byte aligned rows of scales
    const bool sw = zeros == nullptr && span == BK && n_groups % 8 == 0 &&
                    reinterpret_cast<uintptr_t>(scales) % 16 == 0;
#define W4_GEMM_LAUNCH(BMV, SWV)                                                                  \
    return launch_bm<BMV, SWV>(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, k_pad, span, \
                               n_groups, y, ldy, out_f32, stream);
    if (big) {
        if (sw) W4_GEMM_LAUNCH(256, true)
        W4_GEMM_LAUNCH(256, false)
    }
    if (sw) W4_GEMM_LAUNCH(128, true)
    W4_GEMM_LAUNCH(128, false)
#undef W4_GEMM_LAUNCH
}

}  // namespace w4
