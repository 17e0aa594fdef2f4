// gemm_w4a8.hip -- W4A8 prefill GEMM on the int8 matrix cores (gfx950), any number of tokens.
//
// Pages: [Orin] "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s" (sections "从 FP
// 线性层到 INT4 DP4A 的数学推导": y = s_W s_x sum (code - 8) q + b with int8 activations and an
// integer accumulator; "INT32 accumulator 是否安全": the int32 bound; "DP4A 做了什么": integer dot
// products of 4-bit codes against 8-bit operands), [Infra] "【infra之路】12-投机解码、量化与推理
// 引擎对比" (section 2.3: W8A8-style integer GEMMs with int32 accumulation at large batch).
//
// acc[m][n] = sum_{k < d_in} (code[n][k] - 8) q[m][k] is computed exactly as
// sum_k code q - 8 sum_k q on v_mfma_i32_16x16x64_i8: the 4-bit codes (0..15) are int8 operands as
// they are, and each token's sum of q is taken while its codes are staged. The epilogue is
// y = (s_W[n] s_x[m]) acc + b[n] in fp32, as in the W4A8 GEMV.
//
// Tiling: a block of WGM x WGN waves owns 64 WGM tokens x 128 WGN weight rows; each wave owns
// 64 tokens x 128 rows (4 x 8 MFMA tiles, the weight rows as the MFMA's M so that a lane's four
// results are four neighbouring outputs of one token). K runs in steps of 128 columns through
// two LDS stages:
//   * activations: every thread loads 16-column pieces of the tile's rows (8 neighbouring threads
//     cover one row's 128 bytes), adds them into its token sums, and stores the even columns and
//     the odd columns of each 32-column chunk apart: row = [chunk 0 even 16 B | chunk 0 odd 16 B |
//     chunk 1 ...], 144 bytes apart (16 B of padding keep 16 neighbouring rows on distinct banks);
//   * weights: the packed bytes are stored as they are (64 B per row and step, rows 80 bytes
//     apart); a lane reads 16 B (32 codes) of a row and splits them into the low nibbles
//     (w & 0x0F0F0F0F: the even columns) and the high ones ((w >> 4) & 0x0F0F0F0F: the odd), the
//     operands of two MFMAs whose partners are the token's even and odd columns.
// The next step's global loads are in flight while the current stage feeds the MFMAs. Loads are
// raw buffer loads: a token past M or a row past d_out reads zeros, and in the last step the
// activation bytes at and past d_in are masked to zero (act_quant_int8 leaves them unset), which
// also cancels whatever weight bytes meet them.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kG8Step = 128;     // columns per K step
constexpr int kG8AStride = 144;  // LDS bytes per token row of a stage
constexpr int kG8WStride = 80;   // LDS bytes per weight row of a stage
constexpr int kG8TM = 4;         // 16-token MFMA tiles per wave
constexpr int kG8Xcds = 8;

// A block barrier that waits for the LDS accesses only: the next step's global loads stay in
// flight across it (a plain __syncthreads also waits for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// WGM x WGN waves of 64 tokens x 16 TN weight rows each
template <int WGM, int WGN, int TN>
struct G8Shape {
    static constexpr int kThreads = kWave * WGM * WGN;
    static constexpr int kBM = 16 * kG8TM * WGM;  // tokens per block
    static constexpr int kBN = 16 * TN * WGN;     // weight rows per block
    static constexpr int kAL = kBM * 8 / kThreads;  // 16-byte activation pieces per thread
    static constexpr int kWL = kBN * 4 / kThreads;  // 16-byte weight pieces per thread
    static constexpr int kABytes = kBM * kG8AStride;
    static constexpr int kStage = kABytes + kBN * kG8WStride;
    static constexpr int kLds = 2 * kStage + kBM * 4;  // two stages, then the token sums
    static_assert(kAL * kThreads == kBM * 8 && kWL * kThreads == kBN * 4, "load split");
};

template <int WGM, int WGN, int TN, int MINW, bool RAGGED>
__global__ void __launch_bounds__(kWave * WGM * WGN, MINW) gemm_w4a8_kernel(
    const int8_t *__restrict__ q, int M, int64_t ldq, const float *__restrict__ s_x,
    const uint8_t *__restrict__ qweight, const uint16_t *__restrict__ s_w,
    const uint16_t *__restrict__ bias, int d_out, int d_in, int row_bytes, int n_steps,
    int tiles_m, int tiles_n, void *__restrict__ y, int64_t ldy, int out_f32, int vec_store,
    int32_t *__restrict__ acc_out) {
    using S = G8Shape<WGM, WGN, TN>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wid % WGM, wn = wid / WGM;
    const int r16 = lane & 15, kq = lane >> 4;

    // XCD-aware order: hardware block b runs on XCD b % 8; the blocks of one XCD take consecutive
    // tiles, tokens fastest, so that the blocks running together share weight and token tiles in
    // their L2.
    const int nblocks = tiles_m * tiles_n;
    const int b = static_cast<int>(blockIdx.x);
    int t = b;
    if (nblocks % kG8Xcds == 0) t = (b % kG8Xcds) * (nblocks / kG8Xcds) + b / kG8Xcds;
    const int mb = (t % tiles_m) * S::kBM;
    const int nb = (t / tiles_m) * S::kBN;

    const rsrc_t rq = make_rsrc(q, static_cast<uint32_t>(M) * static_cast<uint32_t>(ldq));
    const rsrc_t rw =
        make_rsrc(qweight, static_cast<uint32_t>(d_out) * static_cast<uint32_t>(row_bytes));

    // loader roles: activation piece i of this thread is row L / 8, columns 16 (L % 8) .. + 15 of
    // the step with L = i T + tid; weight piece i is row L / 4, bytes 16 (L % 4) .. + 15.
    uint32_t a_off[S::kAL], a_lds[S::kAL], w_off[S::kWL], w_lds[S::kWL];
    int a_col[S::kAL];
#pragma unroll
    for (int i = 0; i < S::kAL; ++i) {
        const int L = i * S::kThreads + tid, row = L >> 3, slot = L & 7;
        const int m = mb + row;
        a_off[i] = m < M ? static_cast<uint32_t>(m) * static_cast<uint32_t>(ldq) + 16u * slot
                         : kOutOfRange;
        a_col[i] = 16 * slot;
        a_lds[i] = row * kG8AStride + 32 * (slot >> 1) + 8 * (slot & 1);
    }
#pragma unroll
    for (int i = 0; i < S::kWL; ++i) {
        const int L = i * S::kThreads + tid, row = L >> 2, slot = L & 3;
        const int n = nb + row;
        w_off[i] = n < d_out
                       ? static_cast<uint32_t>(n) * static_cast<uint32_t>(row_bytes) + 16u * slot
                       : kOutOfRange;
        w_lds[i] = S::kABytes + row * kG8WStride + 16 * slot;
    }

    // The step's column offset goes into the scalar offset of the loads. Pieces past d_in are only
    // in the last step: their activation bytes are masked there (they may hold the next token's
    // codes, or read as zeros past the end of q), and the weight bytes they meet are multiplied by
    // those zeros whatever they hold (padding codes, the next row, zeros past the end).
    u32x4_t ra[S::kAL], rwt[S::kWL];
    auto gload = [&](int step) {
        const int c0 = step * kG8Step;
#pragma unroll
        for (int i = 0; i < S::kAL; ++i)
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, a_off[i], c0, 0);
#pragma unroll
        for (int i = 0; i < S::kWL; ++i)
            rwt[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[i], c0 / 2, 0);
    };

    int qs[S::kAL];  // this thread's share of each of its rows' sums of q
#pragma unroll
    for (int i = 0; i < S::kAL; ++i) qs[i] = 0;
    // when d_in % 128 != 0 the last step masks the activation bytes at and past d_in
    const int rag_step = RAGGED ? n_steps - 1 : -1;

    auto stage = [&](int step, int buf) {
        unsigned char *base = lds + buf * S::kStage;
#pragma unroll
        for (int i = 0; i < S::kAL; ++i) {
            uint32_t u[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
            if (RAGGED && step == rag_step) {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const int left = d_in - (step * kG8Step + a_col[i] + 4 * d);
                    u[d] &= left >= 4 ? 0xFFFFFFFFu : (left <= 0 ? 0u : (1u << (8 * left)) - 1u);
                }
            }
#pragma unroll
            for (int d = 0; d < 4; ++d)
                qs[i] = __builtin_amdgcn_sdot4(static_cast<int>(u[d]), 0x01010101, qs[i], false);
            const u32x2_t ev = {__builtin_amdgcn_perm(u[1], u[0], 0x06040200u),
                                __builtin_amdgcn_perm(u[3], u[2], 0x06040200u)};
            const u32x2_t od = {__builtin_amdgcn_perm(u[1], u[0], 0x07050301u),
                                __builtin_amdgcn_perm(u[3], u[2], 0x07050301u)};
            *reinterpret_cast<u32x2_t *>(base + a_lds[i]) = ev;
            *reinterpret_cast<u32x2_t *>(base + a_lds[i] + 16) = od;
        }
#pragma unroll
        for (int i = 0; i < S::kWL; ++i) *reinterpret_cast<u32x4_t *>(base + w_lds[i]) = rwt[i];
    };

    i32x4_t acc[TN][kG8TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < kG8TM; ++i) acc[j][i] = i32x4_t{0, 0, 0, 0};

    const uint32_t a_rd = (wm * 64 + r16) * kG8AStride + 32 * kq;
    const uint32_t w_rd = S::kABytes + (wn * 16 * TN + r16) * kG8WStride + 16 * kq;
    auto compute = [&](int buf) {
        const unsigned char *base = lds + buf * S::kStage;
        i32x4_t av[kG8TM][2];
        u32x4_t wv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j)
            wv[j] = *reinterpret_cast<const u32x4_t *>(base + w_rd + j * 16 * kG8WStride);
#pragma unroll
        for (int i = 0; i < kG8TM; ++i) {
            av[i][0] = *reinterpret_cast<const i32x4_t *>(base + a_rd + i * 16 * kG8AStride);
            av[i][1] = *reinterpret_cast<const i32x4_t *>(base + a_rd + i * 16 * kG8AStride + 16);
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {  // the even columns, then the odd ones
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const u32x4_t v = p == 0 ? wv[j] : wv[j] >> 4;
                const u32x4_t c = v & 0x0F0F0F0Fu;
                const i32x4_t wop = {static_cast<int>(c.x), static_cast<int>(c.y),
                                     static_cast<int>(c.z), static_cast<int>(c.w)};
#pragma unroll
                for (int i = 0; i < kG8TM; ++i)
                    acc[j][i] =
                        __builtin_amdgcn_mfma_i32_16x16x64_i8(wop, av[i][p], acc[j][i], 0, 0, 0);
            }
        }
    };

    gload(0);
    stage(0, 0);
    lds_barrier();
    for (int s = 0; s < n_steps; ++s) {
        const bool more = s + 1 < n_steps;
        if (more) gload(s + 1);
        compute(s & 1);
        if (more) stage(s + 1, (s + 1) & 1);
        lds_barrier();
    }

    // token sums: the 8 neighbouring threads of a row hold its 8 pieces
    int *qsum = reinterpret_cast<int *>(lds + 2 * S::kStage);
#pragma unroll
    for (int i = 0; i < S::kAL; ++i) {
        int v = qs[i];
        v += __shfl_xor(v, 1, kWave);
        v += __shfl_xor(v, 2, kWave);
        v += __shfl_xor(v, 4, kWave);
        if ((tid & 7) == 0) qsum[(i * S::kThreads + tid) >> 3] = v;
    }
    lds_barrier();

    // epilogue: acc[j][i] lane (r16, kq) holds rows nb + 16 TN wn + 16 j + 4 kq + r (r = 0..3) of
    // token mb + 64 wm + 16 i + r16
#pragma unroll
    for (int i = 0; i < kG8TM; ++i) {
        const int mloc = wm * 64 + 16 * i + r16;
        const int m = mb + mloc;
        if (m >= M) continue;
        const int tsum8 = 8 * qsum[mloc];
        const float sx = s_x[m];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = nb + wn * 16 * TN + 16 * j + 4 * kq;
            if (n >= d_out) continue;
            float v[4];
            int a[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                a[r] = acc[j][i][r] - tsum8;
                const int nr = n + r < d_out ? n + r : n;
                v[r] = (bf16_to_f32(s_w[nr]) * sx) * static_cast<float>(a[r]);
                if (bias) v[r] += bf16_to_f32(bias[nr]);
            }
            const int64_t o = static_cast<int64_t>(m) * ldy + n;
            if (vec_store && n + 3 < d_out) {
                if (out_f32) {
                    *reinterpret_cast<float4 *>(static_cast<float *>(y) + o) =
                        float4{v[0], v[1], v[2], v[3]};
                } else {
                    const uint32_t lo = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
                    const uint32_t hi = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
                    *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(y) + o) = u32x2_t{lo, hi};
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < d_out) store_out(y, o + r, v[r], out_f32 != 0);
            }
            if (acc_out) {
                const int64_t oa = static_cast<int64_t>(m) * d_out + n;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < d_out) acc_out[oa + r] = a[r];
            }
        }
    }
}

template <int WGM, int WGN, int TN, int MINW>
hipError_t launch_g8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                     const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                     int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                     bool out_f32, int32_t *acc, hipStream_t stream) {
    using S = G8Shape<WGM, WGN, TN>;
    const int tiles_m = static_cast<int>((M + S::kBM - 1) / S::kBM);
    const int tiles_n = static_cast<int>((d_out + S::kBN - 1) / S::kBN);
    const int n_steps = static_cast<int>((d_in + kG8Step - 1) / kG8Step);
    const size_t esz = out_f32 ? 4 : 2;
    const int vec = (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % (4 * esz) == 0);
    const dim3 grid(static_cast<unsigned>(tiles_m) * static_cast<unsigned>(tiles_n));
    auto kern = d_in % kG8Step != 0 ? gemm_w4a8_kernel<WGM, WGN, TN, MINW, true>
                                    : gemm_w4a8_kernel<WGM, WGN, TN, MINW, false>;
    hipLaunchKernelGGL(kern, grid, dim3(S::kThreads), S::kLds, stream, q, static_cast<int>(M),
                       ldq, s_x, qweight, s_w, bias, static_cast<int>(d_out),
                       static_cast<int>(d_in), static_cast<int>(k_pad / 2), n_steps, tiles_m,
                       tiles_n, y, ldy, out_f32 ? 1 : 0, vec, acc);
    return hipGetLastError();
}

}  // namespace

bool gemm_w4a8_supported(int64_t M, int64_t d_out, int64_t ldq, int64_t k_pad) {
    if (M < 1 || d_out < 1) return false;
    // 31-bit buffer offsets: the activations and the packed weights (plus one step past the row)
    if (M * ldq + kG8Step >= (int64_t)kOutOfRange) return false;
    if (d_out * (k_pad / 2) + kG8Step >= (int64_t)kOutOfRange) return false;
    // the grid's thread count stays below 2^31 (one thread per 128 outputs)
    return ((M + 127) / 128) * ((d_out + 255) / 256) * 256 < ((int64_t)1 << 31);
}

hipError_t launch_gemm_w4a8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                            const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                            int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                            bool out_f32, int32_t *acc, hipStream_t stream) {
    if (!gemm_w4a8_supported(M, d_out, ldq, k_pad)) return hipErrorInvalidValue;
    // 128 tokens x 256 rows per block (4 waves; two blocks per CU). Blocks of 256 x 256 (8 waves,
    // one per CU) measured no faster on the 7B prefill shapes, with or without the weight split
    // moved from the MFMA loop into the staging.
    return launch_g8<2, 2, 8, 2>(q, s_x, M, ldq, qweight, s_w, bias, d_out, d_in, k_pad, y, ldy,
                                 out_f32, acc, stream);
}

}  // namespace w4
