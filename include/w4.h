/*
 * w4.h -- C ABI of libw4.so: the group-wise INT4 weight-only quantized linear layer on MI355X
 * (gfx950).
 *
 *   y = x . W_hat^T (+ b),   W_hat[j][k] = s[j][G] * (code[j][k] - z[j][G]),  G = k / group_size
 *
 * Pages cited (title, then section):
 *   [Lab5]  "Lab 5: Gemma4 端到端推理优化"
 *   [Orin]  "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
 *   [Infra] "【infra之路】12-投机解码、量化与推理引擎对比"
 *   [QAT]   "Yeniden paketlenmiş QAT Gemma 4 26B-A4B, tek bir TPU v6e'de FP8 işlemenin 1.9 katı
 *            verimle sunuluyor"
 *
 * Conventions shared by every entry point
 *   - Array arguments are DEVICE pointers owned by the caller.  The library never allocates,
 *     frees or retains device memory and keeps no state between calls (thread-safe; calls on one
 *     stream are ordered by that stream).  The linear layers and the codecs need no scratch
 *     memory (partial sums meet in LDS); GPTQ's factor and column loop take caller-owned work
 *     buffers.  The one exception is w4_gptq_quantize_noalloc, for callers that cannot
 *     allocate: it keeps its work buffer in a device array of the library (see there).
 *   - bf16 values travel as uint16_t bit patterns.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream).  Calls enqueue kernels and return without synchronizing.
 *   - Arguments are validated on the host before anything is enqueued.  A failed check returns
 *     a nonzero w4_status and enqueues nothing; a failed launch returns W4_ERR_HIP and the HIP
 *     error text is kept in w4_last_hip_error() (per host thread).
 *   - Outputs are overwritten, never accumulated into.  Inputs and outputs must not overlap.
 *   - Identical inputs give bitwise-identical outputs (no floating-point atomics).
 *   - Inputs must be finite; NaN/Inf inputs are not checked and give unspecified results.
 *
 * Packed weight format [Lab5 INT4 线性量化], [Lab5 融合INT4反量化与矩阵乘]
 *   k_pad    = ceil(d_in / group_size) * group_size   (group_size in {32, 64, 128, 256})
 *            = ceil(d_in / 32) * 32 with one group per row   (group_size == 0)
 *   n_groups = k_pad / group_size   (1 when group_size == 0)
 *   qweight  uint8 [d_out][k_pad/2]: two 4-bit codes per byte, column 2i in the low nibble and
 *            column 2i+1 in the high nibble.  Rows are output channels.
 *   scales   bf16 [d_out][n_groups]
 *   zeros    bf16 [d_out][n_groups] for W4_ASYM; absent (NULL) for W4_SYM, whose zero point is
 *            the constant 8 (signed levels -8..7 stored as codes 0..15).
 *   Padded columns k >= d_in carry the zero code and decode to exactly 0.
 */
#ifndef W4_H
#define W4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4_OK = 0,
    W4_ERR_NULL = 1,        /* a required pointer is NULL, or zeros given/missing for the mode */
    W4_ERR_SHAPE = 2,       /* a size is < 1, or a leading dimension is smaller than its row  */
    W4_ERR_GROUP = 3,       /* group_size not in {0, 32, 64, 128, 256}                        */
    W4_ERR_ALIGN = 4,       /* a pointer or leading dimension breaks the alignment rules       */
    W4_ERR_RANGE = 5,       /* a size beyond the limits stated for the entry point             */
    W4_ERR_UNSUPPORTED = 6, /* valid arguments this entry point does not serve (e.g. M > 64)   */
    W4_ERR_HIP = 7          /* a HIP launch or query failed; see w4_last_hip_error()           */
} w4_status;

enum { W4_SYM = 0, W4_ASYM = 1 };         /* quantization mode                      */
enum { W4_OUT_BF16 = 0, W4_OUT_F32 = 1 }; /* element type of y                      */

/* Upper bounds checked by every entry point (W4_ERR_RANGE beyond them). */
#define W4_MAX_DIM ((int64_t)1 << 24)  /* d_out, d_in, M, K                      */
#define W4_MAX_W4A8_D_IN ((int64_t)1 << 20) /* keeps sum(code * q) within int32: 2^20*15*127 < 2^31 */
#define W4_GEMV_MAX_M 64
#define W4_DECODE_MAX_D_IN ((int64_t)1 << 16) /* d_in of the decode (M <= 64) entry points     */
#define W4_MAX_GPTQ_D_IN 8192 /* the GPTQ factorization holds d_in x d_in fp32 matrices      */

/*
 * w4_packed_layout -- host-only size query (no GPU work).
 * [Lab5 INT4 线性量化]: the input dimension is padded to a whole number of groups.
 * Writes k_pad, n_groups and the byte size of qweight (d_out * k_pad / 2) for the given shape.
 * Any output pointer may be NULL.  Errors: W4_ERR_SHAPE, W4_ERR_GROUP, W4_ERR_RANGE.
 */
int w4_packed_layout(int64_t d_out, int64_t d_in, int group_size, int64_t *k_pad,
                     int64_t *n_groups, size_t *qweight_bytes);

/*
 * w4_pack -- round-to-nearest (RTN) quantization of an fp32 weight into the packed format.
 * [Lab5 INT4 线性量化]: per (output row, group):
 *   W4_SYM : s = bf16(max|r| / 7), z = 8
 *   W4_ASYM: s = bf16((max r - min r) / 15), z = bf16(round(-min r / s))
 *   code = clip(round(r / s + z), 0, 15), with the stored bf16 s and z; round = ties-to-even.
 * Statistics run over the padded group (pads are 0), so pads encode to z and decode to 0.
 * A group whose bf16 scale is 0 is stored as s = +0, z = +0 (ASYM) and all codes equal to z.
 * The fp32 steps are single IEEE operations in this order:  a/7 (or (mx-mn)/15), bf16 rounding,
 * (-mn)/s, rint, bf16 rounding, then per element  r/s, +z, rint, clamp.
 *   w        fp32 [d_out][ldw], ldw >= d_in, 4-byte aligned
 *   qweight  uint8 [d_out][k_pad/2], 16-byte aligned
 *   scales   bf16 [d_out][n_groups];  zeros bf16 [d_out][n_groups] iff mode == W4_ASYM, else NULL
 */
int w4_pack(const float *w, int64_t d_out, int64_t d_in, int64_t ldw, int group_size, int mode,
            uint8_t *qweight, uint16_t *scales, uint16_t *zeros, void *stream);

/*
 * GPTQ -- quantization that compensates each column's rounding error in the columns after it,
 * producing the packed format of w4_pack.  [Lab5 从 RTN 到 GPTQ]:
 *   objective  min_Q ||X W^T - X Q^T||_F^2 over calibration activations X [N][d_in];
 *   H = (2/N) X^T X; dead columns (H_ii = 0) get H_ii = 1 and zero weights; H += alpha mean(diag H) I;
 *   H^-1 = U^T U (U upper triangular); columns in order: q_i = the code of w_i (the group's scale
 *   and zero by w4_pack's rule from the current, already updated weights of the group at its first
 *   column), e_i = (w_i - q_i) / U_ii, W[:, i:] -= e_i U[i, i:];
 *   L_pred = 1/2 sum_i ||w_i - q_i||^2 / U_ii^2.
 * Everything runs in fp32, as on the page.  Three calls, each enqueued on `stream`:
 *
 * w4_gptq_hessian -- h = (2/N) X^T X.
 *   x  bf16 [N][ldx], ldx >= d_in, only k < d_in read;  h  fp32 [d_in][d_in] (written in full)
 *
 * w4_gptq_factor -- dead columns, damping, and U with (H + lambda I)^-1 = U^T U.
 *   h     fp32 [d_in][d_in], in: the Hessian; destroyed (its lower triangle is worked in place)
 *   alpha the damping factor (the reference uses 0.01), >= 0; with alpha = 0 the Hessian must be
 *         positive definite (N >= d_in calibration rows in general position), else U holds NaN
 *   u     fp32 [d_in][d_in], out: U (zeros below the diagonal)
 *   work  fp32 [d_in][d_in], scratch (the reverse Cholesky factor V, H = V V^T, U = V^-1)
 *   dead  uint8 [d_in], out: 1 for dead columns
 *   The factorization launches about 2 d_in small kernels (an offline step).
 *
 * w4_gptq_quantize -- the column loop.
 *   w        fp32 [d_out][ldw], in: the weights; destroyed (the error-updated working copy)
 *   u, dead  from w4_gptq_factor (dead may be NULL: no dead columns)
 *   group_size, mode, qweight, scales, zeros: as for w4_pack
 *   work     fp32 [d_out][32], scratch (a block's errors)
 *   row_loss fp32 [d_out] or NULL: each row's share of L_pred
 * Limits: d_in <= W4_MAX_GPTQ_D_IN (W4_ERR_RANGE).
 */
int w4_gptq_hessian(const uint16_t *x, int64_t N, int64_t d_in, int64_t ldx, float *h,
                    void *stream);
int w4_gptq_factor(float *h, int64_t d_in, float alpha, float *u, float *work, uint8_t *dead,
                   void *stream);
int w4_gptq_quantize(float *w, int64_t d_out, int64_t d_in, int64_t ldw, const float *u,
                     const uint8_t *dead, int group_size, int mode, uint8_t *qweight,
                     uint16_t *scales, uint16_t *zeros, float *work, float *row_loss,
                     void *stream);

/*
 * w4_gptq_quantize_noalloc -- w4_gptq_quantize without the `work` argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The block errors live in a device array of the library,
 * W4_GPTQ_NOALLOC_MAX_ROWS rows of 32 floats (8 MiB), which each GPU holds from the first call on
 * it until the process ends. Every call on one GPU shares that array: calls that overlap on one
 * GPU (other streams, other host threads) race and give unspecified results; serialize them.
 * The call allocates nothing. d_out > W4_GPTQ_NOALLOC_MAX_ROWS returns W4_ERR_RANGE; every other
 * argument and result is that of w4_gptq_quantize.
 */
#define W4_GPTQ_NOALLOC_MAX_ROWS ((int64_t)1 << 16)
int w4_gptq_quantize_noalloc(float *w, int64_t d_out, int64_t d_in, int64_t ldw, const float *u,
                             const uint8_t *dead, int group_size, int mode, uint8_t *qweight,
                             uint16_t *scales, uint16_t *zeros, float *row_loss, void *stream);

/*
 * w4_qat_repack -- pack a weight trained on the 4-bit grid (a QAT export stored in bf16) without
 * re-quantizing it: the g32 symmetric format of w4_pack (group_size = 32, W4_SYM).
 * [QAT "Yeniden nicelendirme değil, yeniden paketleme"]: per row and group of 32 columns,
 *   a = max|r|; for m = 1 .. 8 the step a / m is kept if it reproduces the whole group, i.e.
 *   every v = r / (a / m) (fp32) is within 1/16 of a level l = rint(v) in [-8, 7];
 *   the kept levels give the codes l + 8 and the least-squares step s = sum r l / sum l^2
 *   (fp64 sums and quotient, rounded to fp32, stored as bf16).
 * A group no m reproduces is off the grid: it is packed by w4_pack's symmetric rule and m = 0 is
 * reported for it. An all-zero group has m = 1 and scale +0. Padded columns decode to 0.
 *   w        bf16 [d_out][ldw], ldw >= d_in, ldw % 8 == 0, 16-byte aligned; only k < d_in is read
 *   qweight  uint8 [d_out][k_pad/2], k_pad = ceil(d_in/32)*32, 16-byte aligned
 *   scales   bf16 [d_out][k_pad/32]
 *   m_out    uint8 [d_out][k_pad/32] or NULL: the m kept per group, 0 for groups off the grid
 * The result is bit-identical to the CPU reference of the same rule.
 */
int w4_qat_repack(const uint16_t *w, int64_t d_out, int64_t d_in, int64_t ldw, uint8_t *qweight,
                  uint16_t *scales, uint8_t *m_out, void *stream);

/*
 * w4_gemv -- W4A16 decode linear for 1 <= M <= 64 token rows, weights read once per call.
 * [Lab5 Prefill和Decode分流] (the small-M decode path), [Lab5 融合INT4反量化与矩阵乘]
 * (dequantize in registers inside the product, never a dense weight in memory),
 * [Orin 模型尺寸和 decode 的真实瓶颈] (y_j = sum_i W_ji x_i + b_j).
 *   x        bf16 [M][ldx], ldx >= d_in, ldx % 8 == 0, 16-byte aligned; only k < d_in is used
 *   qweight, scales, zeros, group_size: the packed format above (zeros NULL iff symmetric)
 *   bias     bf16 [d_out] or NULL
 *   y        [M][ldy], ldy >= d_out, element type out_dtype (W4_OUT_BF16 / W4_OUT_F32),
 *            naturally aligned.  Accumulation is fp32; the bf16 output is the round-to-nearest-
 *            even image of the fp32 result of the same call.
 * M > 64 returns W4_ERR_UNSUPPORTED (use w4_gemm); d_in <= W4_DECODE_MAX_D_IN = 65536 (else
 * W4_ERR_RANGE; w4_gemm serves any d_in up to W4_MAX_DIM).
 */
int w4_gemv(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
            int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *stream);

/*
 * w4_gemv_ws -- w4_gemv with a caller-provided workspace, for 2 <= M <= 64 token rows.
 * [Lab5 Prefill和Decode分流] (the small-M path reads every weight once per step),
 * [Lab5 Linear形状采样] (the projections of a decoder layer: q/k/v and o have few rows, down has
 * few rows and long ones).
 * On matrices with fewer than four 16-row tiles per compute unit (d_out < 64 * CUs) and long
 * rows (at least 64 KiB of codes per compute unit; groups of 128 or 256 columns or one per row),
 * the reduction over d_in is split over column slices that run on different compute units: each
 * slice converts only its own columns of the activations and stores fp32 partial sums in `work`,
 * and a second kernel adds the slices in slice order (so the result is deterministic).  Other
 * shapes run the w4_gemv path.
 *   work        device memory of at least w4_gemv_work_bytes(M, d_out, d_in, group_size) bytes,
 *               16-byte aligned, owned by the caller; its contents on entry do not matter and
 *               are left undefined.  Calls that share a workspace must be ordered (one stream,
 *               or events).  May be NULL when that size is 0.
 *   work_bytes  its size in bytes
 *   the other arguments as for w4_gemv, with the same result within the tolerance.
 * Returns W4_ERR_NULL for a missing workspace, W4_ERR_RANGE for one that is too small,
 * W4_ERR_ALIGN for a misaligned one, and otherwise the codes of w4_gemv.
 */
int w4_gemv_ws(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
               const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
               int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *work,
               size_t work_bytes, void *stream);

/*
 * w4_gemv_work_bytes -- the workspace w4_gemv_ws needs for these sizes (0: none; also 0 for
 * arguments w4_gemv_ws rejects): S * M * d_out * 4 bytes of partial sums for S column slices
 * (S <= d_in / 128 + 1).  It depends only on its arguments and the device's compute-unit count.
 */
size_t w4_gemv_work_bytes(int64_t M, int64_t d_out, int64_t d_in, int group_size);

/*
 * w4_gemv_glu -- the gate/up half of the MLP with its gate fused into the epilogue:
 *   h[m][j] = SiLU(g[m][j]) * u[m][j],  SiLU(v) = v / (1 + exp(-v)),
 *   g = x W_gate^T (+ b_gate),  u = x W_up^T (+ b_up),
 * [Lab5 基础] (FFN(x) = W_down [SiLU(W_gate x) (.) (W_up x)]), [Orin 后续还能继续优化什么] (the
 * SwiGLU kernel boundary). One launch reads the fused weight once and writes only h.
 *   qweight, scales, zeros: a packed weight of 2 d_ff rows, the gate rows [0, d_ff) then the
 *            up rows [d_ff, 2 d_ff) (w4_pack of the stacked gate and up weights)
 *   bias     bf16 [2 d_ff] (gate biases, then up biases) or NULL
 *   y        [M][ldy], ldy >= d_ff: h, as fp32 or its round-to-nearest-even bf16 image
 *   the other arguments as for w4_gemv.
 * Served by the int8 matrix-core decode kernel: 1 <= M <= 4 tokens, group_size 128 or 256, or
 * 0 with k_pad a multiple of 128, and k_pad <= 32768 / M (its activation stage); other arguments
 * return W4_ERR_UNSUPPORTED (use w4_gemv on the fused weight and apply the gate separately).
 * d_in <= W4_DECODE_MAX_D_IN (W4_ERR_RANGE beyond).
 */
int w4_gemv_glu(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_ff,
                int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *stream);

/*
 * w4_gemm -- W4A16 prefill linear for any M >= 1 (the arguments of w4_gemv, and the same
 * result within the tolerance).
 * [Lab5 Prefill和Decode分流] (large M: dequantize once per tile and run a dense matrix product).
 * Weight tiles are dequantized on chip to the fp32 values s (code - z), split into two bf16
 * halves whose sum is exact, and multiplied on the bf16 matrix cores with fp32 accumulation.
 * No dense weight is written to memory.
 */
int w4_gemm(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
            int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *stream);

/*
 * act_quant_int8 -- per-token dynamic symmetric int8 quantization of activations.
 * [Orin 从 FP 线性层到 INT4 DP4A 的数学推导], [Infra 2.2 量化的基本概念]:
 *   s_x[m] = max_k |x[m][k]| / 127 (fp32),  q[m][k] = clip(round(x[m][k] / s_x[m]), -127, 127)
 * round = ties-to-even, the division is one correctly rounded fp32 division.  A token whose
 * values are all zero gets s_x = 0 and q = 0.
 *   x      bf16 [M][ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned
 *   q      int8 [M][ldq], ldq >= K, ldq % 16 == 0, 16-byte aligned; q[m][k] for k < K only
 *   s_x    fp32 [M]
 *   q_sum  int32 [M] = sum_k q[m][k], or NULL
 */
int act_quant_int8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, int64_t ldq,
                   float *s_x, int32_t *q_sum, void *stream);

/*
 * w4a8_gemv -- W4A8 decode linear: int4 weights x int8 activations into an int32 accumulator.
 * [Orin 从 FP 线性层到 INT4 DP4A 的数学推导], [Orin INT32 accumulator 是否安全]:
 *   acc[m][j] = sum_{k < d_in} (code[j][k] - 8) * q[m][k]          (exact, int32)
 *   y[m][j]   = s_w[j] * s_x[m] * acc[m][j] + b[j]                  (fp32)
 * Weights are a per-row symmetric pack (w4_pack with group_size = 0, W4_SYM); s_w is that pack's
 * scales array.  1 <= M <= 64 (W4_ERR_UNSUPPORTED beyond: use w4a8_gemm) and
 * d_in <= W4_DECODE_MAX_D_IN = 65536, the decode kernels' limit (W4_ERR_RANGE beyond: w4a8_gemm
 * serves d_in up to W4_MAX_W4A8_D_IN = 2^20, the bound that keeps every partial sum in int32).
 *   q        int8 [M][ldq], ldq >= d_in, ldq % 16 == 0, 16-byte aligned (from act_quant_int8)
 *   s_x      fp32 [M]
 *   qweight  uint8 [d_out][k_pad/2], k_pad = ceil(d_in/32)*32, 16-byte aligned
 *   s_w      bf16 [d_out];  bias bf16 [d_out] or NULL
 *   y        [M][ldy], ldy >= d_out, out_dtype as for w4_gemv
 *   acc      int32 [M][d_out] (dense), or NULL: the exact accumulators, for bit-exact checks
 */
int w4a8_gemv(const int8_t *q, const float *s_x, int64_t M, int64_t ldq, const uint8_t *qweight,
              const uint16_t *s_w, const uint16_t *bias, int64_t d_out, int64_t d_in, void *y,
              int64_t ldy, int out_dtype, int32_t *acc, void *stream);

/*
 * w4a8_linear -- the W4A8 decode linear with the activation quantization folded in: the result
 * of act_quant_int8 followed by w4a8_gemv, in one launch, without q in memory.
 * [Orin 从 FP 线性层到 INT4 DP4A 的数学推导] (s_x = max|x|/127, q = clamp(rint(x/s_x), +-127)),
 * [Orin INT32 accumulator 是否安全], and the kernel boundary between quantization and linear that
 * [Orin 后续还能继续优化什么] names for further fusion.
 *   x        bf16 [M][ldx], ldx >= d_in, ldx % 8 == 0, 16-byte aligned; only k < d_in is used
 *   qweight, s_w, bias, y, out_dtype, acc: as for w4a8_gemv
 *   s_x      fp32 [M] or NULL: receives the token scales
 * The codes, s_x and acc are bit-identical to those of act_quant_int8 + w4a8_gemv on the same x.
 * Limits: those of w4a8_gemv (1 <= M <= 64, d_in <= W4_DECODE_MAX_D_IN, W4_ERR_RANGE beyond).
 * Every workgroup quantizes the whole activation row it needs; rows longer than the kernel's
 * activation stage (k_pad > 32768) return W4_ERR_UNSUPPORTED: use the two calls.
 */
int w4a8_linear(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                const uint16_t *s_w, const uint16_t *bias, int64_t d_out, int64_t d_in, void *y,
                int64_t ldy, int out_dtype, float *s_x, int32_t *acc, void *stream);

/*
 * w4a8_gemm -- W4A8 prefill linear for any M >= 1: the arguments and the result of w4a8_gemv
 * (acc bit-identical, y within the same rounding), for token counts where the weight tile is
 * reused across many tokens.
 * [Orin 从 FP 线性层到 INT4 DP4A 的数学推导] (the integer form of the linear layer),
 * [Infra 2.3] (int8 products with int32 accumulation for the compute-bound large-batch case).
 * The codes (0..15) and the int8 activations are multiplied on the int8 matrix cores as they
 * are; sum_k 8 q[m][k] is subtracted per token from the int32 sums, so acc is exact.
 *   q, s_x, qweight, s_w, bias, y, out_dtype, acc: as for w4a8_gemv, with any M >= 1
 * Limits (W4_ERR_RANGE beyond them): M <= W4_MAX_DIM, d_in <= W4_MAX_W4A8_D_IN, M * ldq < 2^31
 * and d_out * k_pad / 2 < 2^31 (32-bit buffer offsets), ceil(M / 128) * ceil(d_out / 256) < 2^23
 * (the launch grid).
 */
int w4a8_gemm(const int8_t *q, const float *s_x, int64_t M, int64_t ldq, const uint8_t *qweight,
              const uint16_t *s_w, const uint16_t *bias, int64_t d_out, int64_t d_in, void *y,
              int64_t ldy, int out_dtype, int32_t *acc, void *stream);

/* Text for a w4_status value (static storage). */
const char *w4_status_string(int status);

/* Text of the last HIP error seen by this host thread ("" if none). */
const char *w4_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4_H */
