// w4_launch.h -- host-side launchers of the gfx950 kernels (called by the C ABI after the
// arguments have been validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

hipError_t launch_pack(const float *w, int64_t d_out, int64_t d_in, int64_t ldw, int64_t span,
                       int64_t n_groups, int64_t k_pad, int mode, uint8_t *qweight,
                       uint16_t *scales, uint16_t *zeros, hipStream_t stream);

hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                            int64_t ldq, float *s_x, int32_t *q_sum, hipStream_t stream);

// Decode W4A16 for 1 <= M <= 64 (no scratch memory).
hipError_t launch_gemv(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, void *y, int64_t ldy, bool out_f32, hipStream_t stream);

hipError_t launch_w4a8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                       const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                       bool out_f32, int32_t *acc, hipStream_t stream);

// Decode W4A16 for 2 <= M <= 64 on matrices with few rows per compute unit (groups of 128 or 256
// columns or one per row), the reduction dimension split over S column slices
// (decode_split.hip). With S > 1 the slices' fp32 partial sums go through a caller-provided
// workspace of split_work_bytes() bytes and a second kernel adds them.
bool split_forced();  // the test build's hook (always false in the product library)
struct SplitPlan {
    int tw, S, slices, xk, gshift;
    bool ok;
};
SplitPlan plan_split(int64_t M, int64_t d_out, int64_t k_pad, int64_t span, int64_t n_groups);
size_t split_work_bytes(const SplitPlan &p, int64_t M, int64_t d_out);
bool gemv_split_supported(const SplitPlan &p, int64_t M, int64_t d_in, int64_t k_pad,
                          int64_t ldx);
hipError_t launch_gemv_split(const SplitPlan &p, const uint16_t *x, int64_t M, int64_t ldx,
                             const uint8_t *qweight, const uint16_t *scales,
                             const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
                             int64_t d_in, int64_t k_pad, int64_t n_groups, void *work, void *y,
                             int64_t ldy, bool out_f32, hipStream_t stream);

// W4A8 with the activation quantization folded into the GEMV (bf16 x in; s_x out, nullable).
bool w4a8_linear_supported(int64_t M, int64_t k_pad);
hipError_t launch_w4a8_linear(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                              const uint16_t *s_w, const uint16_t *bias, int64_t d_out,
                              int64_t d_in, int64_t k_pad, void *y, int64_t ldy, bool out_f32,
                              float *s_x, int32_t *acc, hipStream_t stream);

// GPTQ (gptq.hip): Hessian, factorization of its damped inverse, column loop.
hipError_t launch_gptq_hessian(const uint16_t *x, int64_t N, int64_t d_in, int64_t ldx, float *h,
                               hipStream_t stream);
hipError_t launch_gptq_factor(float *h, int64_t d_in, float alpha, float *u, float *v,
                              uint8_t *dead, hipStream_t stream);
// The device address of this GPU's block-error array for w4_gptq_quantize_noalloc
// (kGqScratchRows rows of 32 floats).
constexpr int64_t kGqScratchRows = int64_t(1) << 16;
hipError_t gptq_scratch(float **ptr);
hipError_t launch_gptq_quantize(float *w, int64_t d_out, int64_t d_in, int64_t ldw,
                                const float *u, const uint8_t *dead, int64_t span, int mode,
                                uint8_t *qweight, uint16_t *scales, uint16_t *zeros,
                                int64_t n_groups, int64_t k_pad, float *ebuf, float *row_loss,
                                hipStream_t stream);

// Repack of bf16 weights on the 4-bit grid into the g32 symmetric format (qat_repack.hip).
bool qat_repack_supported(int64_t d_out, int64_t n_groups);
hipError_t launch_qat_repack(const uint16_t *w, int64_t d_out, int64_t d_in, int64_t ldw,
                             uint8_t *qweight, uint16_t *scales, uint8_t *m_out,
                             hipStream_t stream);

// W4A8 prefill GEMM on the int8 matrix cores (gemm_w4a8.hip), any M.
bool gemm_w4a8_supported(int64_t M, int64_t d_out, int64_t ldq, int64_t k_pad);
hipError_t launch_gemm_w4a8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                            const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                            int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                            bool out_f32, int32_t *acc, hipStream_t stream);

hipError_t launch_gemm(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                       const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                       int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, void *y, int64_t ldy, bool out_f32, hipStream_t stream);

// Persistent streaming decode GEMVs (decode_stream.hip).
bool gemv_stream_supported(int64_t M, int64_t k_pad);
bool w4a8_stream_supported(int64_t M, int64_t k_pad, bool fused_quant);
hipError_t launch_gemv_stream(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                              const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                              int64_t d_out, int64_t d_in, int64_t k_pad, int chunk_group_shift,
                              int64_t n_groups, void *y, int64_t ldy, bool out_f32,
                              hipStream_t stream);
// act: int8 codes [M][ldq] with their scales in s_x, or (fused_quant) bf16 x [M][ldq], quantized
// per token inside the kernel with the act_quant rule, the scales written to s_x if given.
hipError_t launch_w4a8_stream(const void *act, bool fused_quant, float *s_x, int64_t M,
                              int64_t ldq, const uint8_t *qweight, const uint16_t *s_w,
                              const uint16_t *bias, int64_t d_out, int64_t d_in, int64_t k_pad,
                              void *y, int64_t ldy, bool out_f32, int32_t *acc,
                              hipStream_t stream);

// Few-token decode on the fp16 matrix cores (decode_mfma.hip): activations converted inside
// each block, one pass over the weights for all tokens of a 16-token tile; no workspace.
// W4A8 decode for 2..64 tokens on the int8 matrix cores (decode_w4a8_mfma.hip): the weights are
// read once per 16 tokens; same y and acc as the streaming kernel
bool w4a8_tok_supported(int64_t M, int64_t d_out, int64_t d_in, int64_t k_pad, int64_t ldq);
hipError_t launch_w4a8_tok(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                           const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                           int64_t d_out, int64_t d_in, int64_t k_pad, void *y, int64_t ldy,
                           bool out_f32, int32_t *acc, hipStream_t stream);
bool gemv_mfma_supported(int64_t M, int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                         int64_t n_groups, int64_t ldx, bool zp);
hipError_t launch_gemv_mfma(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                            int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                            int64_t n_groups, void *y, int64_t ldy, bool out_f32,
                            hipStream_t stream);

// One to four tokens on the int8 matrix cores (decode_i8.hip): activations as exact integer
// digits prepared inside each block, raw codes as the other operand; no workspace.
// glu: the fused gate/up GEMV with the SiLU(gate) * up epilogue (2 d_out weight rows, d_out
// outputs).
bool gemv_i8_supported(int64_t M, int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                       int64_t n_groups, int64_t ldx, bool glu = false);
bool gemv_i8_preferred(int64_t M, int64_t d_out, int64_t k_pad);
hipError_t launch_gemv_i8(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                          const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                          int64_t d_out, int64_t d_in, int64_t k_pad, int64_t span,
                          int64_t n_groups, void *y, int64_t ldy, bool out_f32, bool glu,
                          hipStream_t stream);

// Number of compute units of the current device (cached per device).
int device_cu_count();

}  // namespace w4
