// abi.hip -- the extern "C" entry points of libw4.so: host-side argument validation, layout
// arithmetic and dispatch to the gfx950 kernels.  The contract of every entry point is stated in
// include/w4.h; nothing here allocates device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/w4.h"
#include "w4_launch.h"

namespace {

thread_local std::string g_last_hip_error;

int hip_fail(hipError_t err) {
    g_last_hip_error = hipGetErrorString(err);
    return W4_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_group(int g) { return g == 0 || g == 32 || g == 64 || g == 128 || g == 256; }

struct Layout {
    int64_t k_pad, n_groups, span;
};

Layout layout_of(int64_t d_in, int group_size) {
    Layout L{};
    const int64_t q = group_size > 0 ? group_size : 32;
    L.k_pad = (d_in + q - 1) / q * q;
    L.n_groups = group_size > 0 ? L.k_pad / group_size : 1;
    L.span = L.k_pad / L.n_groups;
    return L;
}

// The decode kernels keep one row's columns spread over at most 16 waves x 64 lanes x a few
// 32-column steps; this bounds d_in for the decode entry points (w4.h: W4_DECODE_MAX_D_IN).
constexpr int64_t kDecodeMaxDin = W4_DECODE_MAX_D_IN;

int check_dims(int64_t d_out, int64_t d_in) {
    if (d_out < 1 || d_in < 1) return W4_ERR_SHAPE;
    if (d_out > W4_MAX_DIM || d_in > W4_MAX_DIM) return W4_ERR_RANGE;
    return W4_OK;
}

int check_linear(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                 const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                 int64_t d_out, int64_t d_in, int group_size, const void *y, int64_t ldy,
                 int out_dtype) {
    (void)zeros;
    if (!x || !qweight || !scales || !y) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (M < 1 || ldx < d_in || ldy < d_out) return W4_ERR_SHAPE;
    if (M > W4_MAX_DIM || ldx > W4_MAX_DIM || ldy > W4_MAX_DIM) return W4_ERR_RANGE;
    if (!valid_group(group_size)) return W4_ERR_GROUP;
    if (out_dtype != W4_OUT_BF16 && out_dtype != W4_OUT_F32) return W4_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(qweight, 16)) return W4_ERR_ALIGN;
    if (!aligned(scales, 2) || (bias && !aligned(bias, 2))) return W4_ERR_ALIGN;
    if (!aligned(y, out_dtype == W4_OUT_F32 ? 4 : 2)) return W4_ERR_ALIGN;
    return W4_OK;
}

}  // namespace

extern "C" {

const char *w4_status_string(int status) {
    switch (status) {
        case W4_OK: return "ok";
        case W4_ERR_NULL: return "null pointer (or zeros given/missing for the quantization mode)";
        case W4_ERR_SHAPE: return "invalid shape or leading dimension";
        case W4_ERR_GROUP: return "group_size must be 0, 32, 64, 128 or 256";
        case W4_ERR_ALIGN: return "pointer or leading dimension breaks the alignment rules";
        case W4_ERR_RANGE: return "size beyond the supported range";
        case W4_ERR_UNSUPPORTED: return "arguments not served by this entry point";
        case W4_ERR_HIP: return "HIP error (see w4_last_hip_error)";
        default: return "unknown status";
    }
}

const char *w4_last_hip_error(void) { return g_last_hip_error.c_str(); }

int w4_packed_layout(int64_t d_out, int64_t d_in, int group_size, int64_t *k_pad,
                     int64_t *n_groups, size_t *qweight_bytes) {
    if (int st = check_dims(d_out, d_in)) return st;
    if (!valid_group(group_size)) return W4_ERR_GROUP;
    const Layout L = layout_of(d_in, group_size);
    if (k_pad) *k_pad = L.k_pad;
    if (n_groups) *n_groups = L.n_groups;
    if (qweight_bytes) *qweight_bytes = static_cast<size_t>(d_out) * static_cast<size_t>(L.k_pad / 2);
    return W4_OK;
}

int w4_pack(const float *w, int64_t d_out, int64_t d_in, int64_t ldw, int group_size, int mode,
            uint8_t *qweight, uint16_t *scales, uint16_t *zeros, void *stream) {
    if (!w || !qweight || !scales) return W4_ERR_NULL;
    if (mode != W4_SYM && mode != W4_ASYM) return W4_ERR_UNSUPPORTED;
    if ((mode == W4_ASYM) != (zeros != nullptr)) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (ldw < d_in) return W4_ERR_SHAPE;
    if (ldw > W4_MAX_DIM) return W4_ERR_RANGE;
    if (!valid_group(group_size)) return W4_ERR_GROUP;
    if (!aligned(w, 4) || !aligned(qweight, 16) || !aligned(scales, 2) ||
        (zeros && !aligned(zeros, 2)))
        return W4_ERR_ALIGN;
    const Layout L = layout_of(d_in, group_size);
    const hipError_t err = w4::launch_pack(w, d_out, d_in, ldw, L.span, L.n_groups, L.k_pad,
                                           mode, qweight, scales, zeros,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gptq_hessian(const uint16_t *x, int64_t N, int64_t d_in, int64_t ldx, float *h,
                    void *stream) {
    if (!x || !h) return W4_ERR_NULL;
    if (N < 1 || d_in < 1 || ldx < d_in) return W4_ERR_SHAPE;
    if (N > W4_MAX_DIM || d_in > W4_MAX_GPTQ_D_IN || ldx > W4_MAX_DIM) return W4_ERR_RANGE;
    if (!aligned(x, 2) || !aligned(h, 4)) return W4_ERR_ALIGN;
    const hipError_t err =
        w4::launch_gptq_hessian(x, N, d_in, ldx, h, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gptq_factor(float *h, int64_t d_in, float alpha, float *u, float *work, uint8_t *dead,
                   void *stream) {
    if (!h || !u || !work || !dead) return W4_ERR_NULL;
    if (d_in < 1) return W4_ERR_SHAPE;
    if (d_in > W4_MAX_GPTQ_D_IN) return W4_ERR_RANGE;
    if (!(alpha >= 0.0f) || !(alpha < 1e30f)) return W4_ERR_RANGE;
    if (!aligned(h, 4) || !aligned(u, 4) || !aligned(work, 4)) return W4_ERR_ALIGN;
    const hipError_t err =
        w4::launch_gptq_factor(h, d_in, alpha, u, work, dead, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gptq_quantize(float *w, int64_t d_out, int64_t d_in, int64_t ldw, const float *u,
                     const uint8_t *dead, int group_size, int mode, uint8_t *qweight,
                     uint16_t *scales, uint16_t *zeros, float *work, float *row_loss,
                     void *stream) {
    if (!w || !u || !qweight || !scales || !work) return W4_ERR_NULL;
    if (mode != W4_SYM && mode != W4_ASYM) return W4_ERR_UNSUPPORTED;
    if ((mode == W4_ASYM) != (zeros != nullptr)) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (ldw < d_in) return W4_ERR_SHAPE;
    if (d_in > W4_MAX_GPTQ_D_IN || ldw > W4_MAX_DIM) return W4_ERR_RANGE;
    if (!valid_group(group_size)) return W4_ERR_GROUP;
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(qweight, 4) || !aligned(scales, 2) ||
        (zeros && !aligned(zeros, 2)) || !aligned(work, 4) || (row_loss && !aligned(row_loss, 4)))
        return W4_ERR_ALIGN;
    const Layout L = layout_of(d_in, group_size);
    const hipError_t err = w4::launch_gptq_quantize(
        w, d_out, d_in, ldw, u, dead, L.span, mode, qweight, scales, zeros, L.n_groups, L.k_pad,
        work, row_loss, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gptq_quantize_noalloc(float *w, int64_t d_out, int64_t d_in, int64_t ldw, const float *u,
                             const uint8_t *dead, int group_size, int mode, uint8_t *qweight,
                             uint16_t *scales, uint16_t *zeros, float *row_loss, void *stream) {
    if (!w || !u || !qweight || !scales) return W4_ERR_NULL;
    if (mode != W4_SYM && mode != W4_ASYM) return W4_ERR_UNSUPPORTED;
    if ((mode == W4_ASYM) != (zeros != nullptr)) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (ldw < d_in) return W4_ERR_SHAPE;
    if (d_in > W4_MAX_GPTQ_D_IN || ldw > W4_MAX_DIM || d_out > W4_GPTQ_NOALLOC_MAX_ROWS)
        return W4_ERR_RANGE;
    if (!valid_group(group_size)) return W4_ERR_GROUP;
    if (!aligned(w, 4) || !aligned(u, 4) || !aligned(qweight, 4) || !aligned(scales, 2) ||
        (zeros && !aligned(zeros, 2)) || (row_loss && !aligned(row_loss, 4)))
        return W4_ERR_ALIGN;
    static_assert(W4_GPTQ_NOALLOC_MAX_ROWS == w4::kGqScratchRows, "the scratch array's rows");
    float *ebuf = nullptr;
    hipError_t err = w4::gptq_scratch(&ebuf);
    if (err != hipSuccess) return hip_fail(err);
    const Layout L = layout_of(d_in, group_size);
    err = w4::launch_gptq_quantize(w, d_out, d_in, ldw, u, dead, L.span, mode, qweight, scales,
                                   zeros, L.n_groups, L.k_pad, ebuf, row_loss,
                                   static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_qat_repack(const uint16_t *w, int64_t d_out, int64_t d_in, int64_t ldw, uint8_t *qweight,
                  uint16_t *scales, uint8_t *m_out, void *stream) {
    if (!w || !qweight || !scales) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (ldw < d_in) return W4_ERR_SHAPE;
    if (ldw > W4_MAX_DIM) return W4_ERR_RANGE;
    if (!aligned(w, 16) || ldw % 8 != 0 || !aligned(qweight, 16) || !aligned(scales, 2))
        return W4_ERR_ALIGN;
    if (!w4::qat_repack_supported(d_out, (d_in + 31) / 32)) return W4_ERR_RANGE;
    const hipError_t err = w4::launch_qat_repack(w, d_out, d_in, ldw, qweight, scales, m_out,
                                                 static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gemv(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
            int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *stream) {
    if (int st = check_linear(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, group_size,
                              y, ldy, out_dtype))
        return st;
    if (zeros && !aligned(zeros, 2)) return W4_ERR_ALIGN;
    if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
    if (d_in > kDecodeMaxDin) return W4_ERR_RANGE;
    const Layout L = layout_of(d_in, group_size);
    const hipError_t err =
        w4::launch_gemv(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, L.k_pad, L.span,
                        L.n_groups, y, ldy, out_dtype == W4_OUT_F32,
                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

size_t w4_gemv_work_bytes(int64_t M, int64_t d_out, int64_t d_in, int group_size) {
    if (M < 2 || M > W4_GEMV_MAX_M || check_dims(d_out, d_in) != W4_OK || d_in > kDecodeMaxDin ||
        !valid_group(group_size))
        return 0;
    const Layout L = layout_of(d_in, group_size);
    return w4::split_work_bytes(w4::plan_split(M, d_out, L.k_pad, L.span, L.n_groups), M, d_out);
}

int w4_gemv_ws(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
               const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
               int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *work,
               size_t work_bytes, void *stream) {
    if (int st = check_linear(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, group_size,
                              y, ldy, out_dtype))
        return st;
    if (zeros && !aligned(zeros, 2)) return W4_ERR_ALIGN;
    if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
    if (d_in > kDecodeMaxDin) return W4_ERR_RANGE;
    const Layout L = layout_of(d_in, group_size);
    const w4::SplitPlan p = w4::plan_split(M, d_out, L.k_pad, L.span, L.n_groups);
    const size_t need = w4::split_work_bytes(p, M, d_out);
    if (need > 0) {
        if (!work) return W4_ERR_NULL;
        if (work_bytes < need) return W4_ERR_RANGE;
        if (!aligned(work, 16)) return W4_ERR_ALIGN;
    }
    hipError_t err;
    if (w4::gemv_split_supported(p, M, d_in, L.k_pad, ldx))
        err = w4::launch_gemv_split(p, x, M, ldx, qweight, scales, zeros, bias, d_out, d_in,
                                    L.k_pad, L.n_groups, work, y, ldy,
                                    out_dtype == W4_OUT_F32, static_cast<hipStream_t>(stream));
    else
        err = w4::launch_gemv(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, L.k_pad,
                              L.span, L.n_groups, y, ldy, out_dtype == W4_OUT_F32,
                              static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gemm(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
            const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_out,
            int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *stream) {
    if (int st = check_linear(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, group_size,
                              y, ldy, out_dtype))
        return st;
    if (zeros && !aligned(zeros, 2)) return W4_ERR_ALIGN;
    const Layout L = layout_of(d_in, group_size);
    const hipError_t err =
        w4::launch_gemm(x, M, ldx, qweight, scales, zeros, bias, d_out, d_in, L.k_pad, L.span,
                        L.n_groups, y, ldy, out_dtype == W4_OUT_F32,
                        static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int act_quant_int8(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q, int64_t ldq,
                   float *s_x, int32_t *q_sum, void *stream) {
    if (!x || !q || !s_x) return W4_ERR_NULL;
    if (M < 1 || K < 1 || ldx < K || ldq < K) return W4_ERR_SHAPE;
    if (M > W4_MAX_DIM || K > W4_MAX_DIM || ldx > W4_MAX_DIM || ldq > W4_MAX_DIM)
        return W4_ERR_RANGE;
    if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(q, 16) || ldq % 16 != 0 || !aligned(s_x, 4) ||
        (q_sum && !aligned(q_sum, 4)))
        return W4_ERR_ALIGN;
    const hipError_t err =
        w4::launch_act_quant(x, M, K, ldx, q, ldq, s_x, q_sum, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4a8_gemv(const int8_t *q, const float *s_x, int64_t M, int64_t ldq, const uint8_t *qweight,
              const uint16_t *s_w, const uint16_t *bias, int64_t d_out, int64_t d_in, void *y,
              int64_t ldy, int out_dtype, int32_t *acc, void *stream) {
    if (!q || !s_x || !qweight || !s_w || !y) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (M < 1 || ldq < d_in || ldy < d_out) return W4_ERR_SHAPE;
    if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
    if (d_in > W4_MAX_W4A8_D_IN || d_in > kDecodeMaxDin || ldq > W4_MAX_DIM || ldy > W4_MAX_DIM)
        return W4_ERR_RANGE;
    if (out_dtype != W4_OUT_BF16 && out_dtype != W4_OUT_F32) return W4_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(qweight, 16) || !aligned(s_x, 4) ||
        !aligned(s_w, 2) || (bias && !aligned(bias, 2)) || (acc && !aligned(acc, 4)) ||
        !aligned(y, out_dtype == W4_OUT_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    const Layout L = layout_of(d_in, 0);
    const hipError_t err =
        w4::launch_w4a8(q, s_x, M, ldq, qweight, s_w, bias, d_out, d_in, L.k_pad, y, ldy,
                        out_dtype == W4_OUT_F32, acc, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4a8_gemm(const int8_t *q, const float *s_x, int64_t M, int64_t ldq, const uint8_t *qweight,
              const uint16_t *s_w, const uint16_t *bias, int64_t d_out, int64_t d_in, void *y,
              int64_t ldy, int out_dtype, int32_t *acc, void *stream) {
    if (!q || !s_x || !qweight || !s_w || !y) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (M < 1 || ldq < d_in || ldy < d_out) return W4_ERR_SHAPE;
    if (M > W4_MAX_DIM || d_in > W4_MAX_W4A8_D_IN || ldq > W4_MAX_DIM || ldy > W4_MAX_DIM)
        return W4_ERR_RANGE;
    if (out_dtype != W4_OUT_BF16 && out_dtype != W4_OUT_F32) return W4_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || ldq % 16 != 0 || !aligned(qweight, 16) || !aligned(s_x, 4) ||
        !aligned(s_w, 2) || (bias && !aligned(bias, 2)) || (acc && !aligned(acc, 4)) ||
        !aligned(y, out_dtype == W4_OUT_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    const Layout L = layout_of(d_in, 0);
    if (!w4::gemm_w4a8_supported(M, d_out, ldq, L.k_pad)) return W4_ERR_RANGE;
    const hipError_t err =
        w4::launch_gemm_w4a8(q, s_x, M, ldq, qweight, s_w, bias, d_out, d_in, L.k_pad, y, ldy,
                             out_dtype == W4_OUT_F32, acc, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4_gemv_glu(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias, int64_t d_ff,
                int64_t d_in, int group_size, void *y, int64_t ldy, int out_dtype, void *stream) {
    if (int st = check_linear(x, M, ldx, qweight, scales, zeros, bias, d_ff, d_in, group_size, y,
                              ldy, out_dtype))
        return st;
    if (zeros && !aligned(zeros, 2)) return W4_ERR_ALIGN;
    if (2 * d_ff > W4_MAX_DIM) return W4_ERR_RANGE;
    if (d_in > kDecodeMaxDin) return W4_ERR_RANGE;
    const Layout L = layout_of(d_in, group_size);
    if (!w4::gemv_i8_supported(M, d_ff, d_in, L.k_pad, L.span, L.n_groups, ldx, true))
        return W4_ERR_UNSUPPORTED;
    const hipError_t err =
        w4::launch_gemv_i8(x, M, ldx, qweight, scales, zeros, bias, d_ff, d_in, L.k_pad, L.span,
                           L.n_groups, y, ldy, out_dtype == W4_OUT_F32, true,
                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

int w4a8_linear(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                const uint16_t *s_w, const uint16_t *bias, int64_t d_out, int64_t d_in, void *y,
                int64_t ldy, int out_dtype, float *s_x, int32_t *acc, void *stream) {
    if (!x || !qweight || !s_w || !y) return W4_ERR_NULL;
    if (int st = check_dims(d_out, d_in)) return st;
    if (M < 1 || ldx < d_in || ldy < d_out) return W4_ERR_SHAPE;
    if (M > W4_GEMV_MAX_M) return W4_ERR_UNSUPPORTED;
    if (d_in > W4_MAX_W4A8_D_IN || d_in > kDecodeMaxDin || ldx > W4_MAX_DIM || ldy > W4_MAX_DIM)
        return W4_ERR_RANGE;
    if (out_dtype != W4_OUT_BF16 && out_dtype != W4_OUT_F32) return W4_ERR_UNSUPPORTED;
    if (!aligned(x, 16) || ldx % 8 != 0 || !aligned(qweight, 16) || !aligned(s_w, 2) ||
        (bias && !aligned(bias, 2)) || (s_x && !aligned(s_x, 4)) || (acc && !aligned(acc, 4)) ||
        !aligned(y, out_dtype == W4_OUT_F32 ? 4 : 2))
        return W4_ERR_ALIGN;
    const Layout L = layout_of(d_in, 0);
    if (!w4::w4a8_linear_supported(M, L.k_pad)) return W4_ERR_UNSUPPORTED;
    const hipError_t err =
        w4::launch_w4a8_linear(x, M, ldx, qweight, s_w, bias, d_out, d_in, L.k_pad, y, ldy,
                               out_dtype == W4_OUT_F32, s_x, acc, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4_OK : hip_fail(err);
}

}  // extern "C"

namespace w4 {

int device_cu_count() {
    static std::mutex mu;
    static std::vector<int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace w4
