/*
 * oracle.c -- plain, slow CPU oracle for the group-wise INT4 weight-only linear layer.
 *
 * TEST INFRASTRUCTURE ONLY. This library is loaded by the test-suite, by the smoke check and by
 * the CPU-baseline leg of the benchmark, and by nothing else. It shares no source, header,
 * table or helper with the GPU library; the product path never calls it.
 *
 * Pages this file follows (cited as [tag section]):
 *   [Lab5]  "Lab 5: Gemma4 端到端推理优化"  (Grapesea HPC101 notes)
 *   [Orin]  "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
 *   [Infra] "【infra之路】12-投机解码、量化与推理引擎对比"
 *   [QAT]   "Yeniden paketlenmiş QAT Gemma 4 26B-A4B, tek bir TPU v6e'de FP8 işlemenin 1.9 katı
 *            verimle sunuluyor"
 *
 * Precision.  The codec steps (weight packing, activation quantization) produce integer codes and
 * bf16/fp32 bit patterns, so they are written as explicit fp32 operation sequences (one IEEE op
 * per line, round-to-nearest-even, no contraction; build with -ffp-contract=off and without
 * fast-math).  The contractions are done in fp64 (W4A16) and int64 (W4A8), which is exact
 * for the products and leaves only the fp64 summation error.
 *
 * Every routine loops over the mathematical definition directly: no blocking, no fusion, no
 * reordering.  OpenMP only splits independent output rows across host threads.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_SYM 0
#define ORACLE_ASYM 1

/* ------------------------------------------------------------------------------------------ */
/* bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.  Rounding fp32 -> bf16 is     */
/* round-to-nearest, ties-to-even on the discarded 16 bits (inputs are finite).                 */
/* ------------------------------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lower = u & 0xFFFFu;
    uint32_t upper = u >> 16;
    /* nearest: round up when the discarded part exceeds one half, or equals one half and the
       kept part is odd (ties to even) */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
    return (uint16_t)upper;
}

/* element-wise over arrays (the same two conversions) */
void oracle_bf16_to_f32_array(const uint16_t *h, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f32(h[i]);
}

void oracle_f32_to_bf16_array(const float *f, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(f[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Packed layout.  [Lab5 INT4 线性量化]: parameters are shared per output channel and per       */
/* group_size input columns; the input dimension is padded up to a multiple of the group size.  */
/* group_size == 0 means one group spanning the whole (padded) row, the per-output-row scale of  */
/* [Orin 从 FP 线性层到 INT4 DP4A 的数学推导]; the row is then padded to a multiple of 32.        */
/* ------------------------------------------------------------------------------------------ */
int64_t oracle_k_pad(int64_t d_in, int group_size) {
    int64_t q = group_size > 0 ? group_size : 32;
    return ((d_in + q - 1) / q) * q;
}

int64_t oracle_n_groups(int64_t d_in, int group_size) {
    return group_size > 0 ? oracle_k_pad(d_in, group_size) / group_size : 1;
}

/* ------------------------------------------------------------------------------------------ */
/* O1: RTN pack.  [Lab5 INT4 线性量化]                                                          */
/*   q = clip(round(r/s + z), 0, 15),  r_hat = s (q - z)                                          */
/*   symmetric:  s = max|r| / 7, z = 8 (signed [-8,7] stored as code [0,15])                     */
/*   asymmetric: s = (r_max - r_min) / 15, z = round(-r_min / s)                                  */
/*   two codes per byte, the earlier column in the low nibble; padded columns are zeros of the   */
/*   group, so they encode to the zero code and decode to exactly 0.                             */
/* The scale used to encode is the stored bf16 scale (one s for encode and decode); likewise the */
/* stored bf16 zero point.  A zero scale encodes the whole group as its zero code.  Zero scales  */
/* and zero points are stored as +0.                                                             */
/* ------------------------------------------------------------------------------------------ */
void oracle_pack(const float *w, int64_t d_out, int64_t d_in, int64_t ldw, int group_size,
                 int mode, uint8_t *qweight, uint16_t *scales, uint16_t *zeros) {
    const int64_t k_pad = oracle_k_pad(d_in, group_size);
    const int64_t n_groups = oracle_n_groups(d_in, group_size);
    const int64_t g = k_pad / n_groups;

#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < d_out; ++j) {
        for (int64_t G = 0; G < n_groups; ++G) {
            const int64_t k0 = G * g;
            /* group statistics over the padded group (pads are 0.0f) */
            float amax = 0.0f, mx = 0.0f, mn = 0.0f;
            for (int64_t t = 0; t < g; ++t) {
                const int64_t k = k0 + t;
                const float r = k < d_in ? w[j * ldw + k] : 0.0f;
                const float a = fabsf(r);
                if (t == 0) {
                    amax = a;
                    mx = r;
                    mn = r;
                } else {
                    if (a > amax) amax = a;
                    if (r > mx) mx = r;
                    if (r < mn) mn = r;
                }
            }
            float s32, zf;
            if (mode == ORACLE_SYM) {
                s32 = amax / 7.0f;
                zf = 8.0f;
            } else {
                const float range = mx - mn;
                s32 = range / 15.0f;
                zf = 0.0f; /* set below once s is known */
            }
            s32 = s32 + 0.0f; /* a zero scale is stored as +0 */
            const uint16_t s_bits = oracle_f32_to_bf16(s32);
            const float s = oracle_bf16_to_f32(s_bits);
            uint16_t z_bits = 0;
            if (mode == ORACLE_ASYM) {
                if (s != 0.0f) {
                    const float neg_mn = -mn;
                    const float ratio = neg_mn / s;
                    zf = rintf(ratio);
                    zf = zf + 0.0f; /* a zero point of -0 is stored as +0 */
                } else {
                    zf = 0.0f;
                }
                z_bits = oracle_f32_to_bf16(zf);
                zf = oracle_bf16_to_f32(z_bits);
                zeros[j * n_groups + G] = z_bits;
            }
            scales[j * n_groups + G] = s_bits;

            for (int64_t t = 0; t < g; t += 2) {
                unsigned code[2];
                for (int e = 0; e < 2; ++e) {
                    const int64_t k = k0 + t + e;
                    const float r = k < d_in ? w[j * ldw + k] : 0.0f;
                    if (s == 0.0f) {
                        code[e] = (unsigned)zf;
                    } else {
                        float v = r / s;
                        v = v + zf;
                        v = rintf(v);
                        if (v < 0.0f) v = 0.0f;
                        if (v > 15.0f) v = 15.0f;
                        code[e] = (unsigned)v;
                    }
                }
                qweight[j * (k_pad / 2) + (k0 + t) / 2] = (uint8_t)(code[0] | (code[1] << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O2: unpack.  [Lab5 量化正确性修正]: the low and the high nibble of each byte are computed      */
/* independently from the untouched packed bytes and only then interleaved (low first).          */
/* ------------------------------------------------------------------------------------------ */
void oracle_unpack(const uint8_t *qweight, int64_t d_out, int64_t k_pad, uint8_t *codes) {
    const int64_t nb = k_pad / 2;
    for (int64_t j = 0; j < d_out; ++j) {
        for (int64_t i = 0; i < nb; ++i) {
            const uint8_t byte = qweight[j * nb + i];
            const uint8_t low = (uint8_t)(byte & 0x0F);
            const uint8_t high = (uint8_t)(byte >> 4);
            codes[j * k_pad + 2 * i] = low;
            codes[j * k_pad + 2 * i + 1] = high;
        }
    }
}

/* the code of column k of row j, read straight from the packed bytes */
static unsigned code_at(const uint8_t *qweight, int64_t k_pad, int64_t j, int64_t k) {
    const uint8_t byte = qweight[j * (k_pad / 2) + k / 2];
    return (k % 2 == 0) ? (unsigned)(byte & 0x0F) : (unsigned)(byte >> 4);
}

/* ------------------------------------------------------------------------------------------ */
/* O3: dequant.  [Lab5 INT4 线性量化]: r_hat = s (q - z).  In fp64 this is exact (an 8-bit      */
/* significand times a small integer).  Symmetric packs have z = 8 and no zeros array.           */
/* Output: w_hat[d_out][k_pad], pads included.                                                    */
/* ------------------------------------------------------------------------------------------ */
void oracle_dequant(const uint8_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                    int64_t d_out, int64_t d_in, int group_size, double *w_hat) {
    const int64_t k_pad = oracle_k_pad(d_in, group_size);
    const int64_t n_groups = oracle_n_groups(d_in, group_size);
    const int64_t g = k_pad / n_groups;
    for (int64_t j = 0; j < d_out; ++j) {
        for (int64_t k = 0; k < k_pad; ++k) {
            const int64_t G = k / g;
            const double s = (double)oracle_bf16_to_f32(scales[j * n_groups + G]);
            const double z = zeros ? (double)oracle_bf16_to_f32(zeros[j * n_groups + G]) : 8.0;
            const double q = (double)code_at(qweight, k_pad, j, k);
            w_hat[j * k_pad + k] = s * (q - z);
        }
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O4: W4A16 linear.  y[m][j] = sum_{k < d_in} x[m][k] * r_hat[j][k]  (+ b[j])                    */
/* [Lab5 融合INT4反量化与矩阵乘] (dequantize inside the product, never a stored dense weight) and */
/* [Orin 模型尺寸和 decode 的真实瓶颈] (y_j = sum_i W_ji x_i + b_j).  x and b are bf16 bit        */
/* patterns; y is fp64 [M][d_out].                                                                */
/* ------------------------------------------------------------------------------------------ */
void oracle_w4a16(const uint16_t *x, int64_t M, int64_t ldx, const uint8_t *qweight,
                  const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                  int64_t d_out, int64_t d_in, int group_size, double *y) {
    const int64_t k_pad = oracle_k_pad(d_in, group_size);
    const int64_t n_groups = oracle_n_groups(d_in, group_size);
    const int64_t g = k_pad / n_groups;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < d_out; ++j) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < d_in; ++k) {
                const int64_t G = k / g;
                const double s = (double)oracle_bf16_to_f32(scales[j * n_groups + G]);
                const double z =
                    zeros ? (double)oracle_bf16_to_f32(zeros[j * n_groups + G]) : 8.0;
                const double q = (double)code_at(qweight, k_pad, j, k);
                const double w_hat = s * (q - z);
                acc += (double)oracle_bf16_to_f32(x[m * ldx + k]) * w_hat;
            }
            if (bias) acc += (double)oracle_bf16_to_f32(bias[j]);
            y[m * d_out + j] = acc;
        }
    }
}

/* O4 on a list of (token, output row) pairs, for spot checks at sizes where the full product    */
/* is too slow on the host.  out[i] = y[tok[i]][row[i]].                                          */
void oracle_w4a16_points(const uint16_t *x, int64_t ldx, const uint8_t *qweight,
                         const uint16_t *scales, const uint16_t *zeros, const uint16_t *bias,
                         int64_t d_in, int group_size, const int64_t *tok, const int64_t *row,
                         int64_t n_points, double *out) {
    const int64_t k_pad = oracle_k_pad(d_in, group_size);
    const int64_t n_groups = oracle_n_groups(d_in, group_size);
    const int64_t g = k_pad / n_groups;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_points; ++i) {
        const int64_t m = tok[i], j = row[i];
        double acc = 0.0;
        for (int64_t k = 0; k < d_in; ++k) {
            const int64_t G = k / g;
            const double s = (double)oracle_bf16_to_f32(scales[j * n_groups + G]);
            const double z = zeros ? (double)oracle_bf16_to_f32(zeros[j * n_groups + G]) : 8.0;
            const double q = (double)code_at(qweight, k_pad, j, k);
            acc += (double)oracle_bf16_to_f32(x[m * ldx + k]) * (s * (q - z));
        }
        if (bias) acc += (double)oracle_bf16_to_f32(bias[j]);
        out[i] = acc;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O5: per-token dynamic int8 activation quantization.                                            */
/* [Orin 从 FP 线性层到 INT4 DP4A 的数学推导] and [Infra 2.2 量化的基本概念]:                     */
/*   s_x = max_i |x_i| / 127,  q_i = clip(round(x_i / s_x), -127, 127)                            */
/* fp32 throughout (x is bf16, so |x| and the max are exact).  An all-zero token has s_x = 0 and  */
/* q = 0.  q_sum[m] = sum_k q[m][k] (nullable), used to fold the nibble offset of 8.             */
/* ------------------------------------------------------------------------------------------ */
void oracle_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                      int64_t ldq, float *s_x, int32_t *q_sum) {
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            const float v = fabsf(oracle_bf16_to_f32(x[m * ldx + k]));
            if (v > a) a = v;
        }
        const float s = a / 127.0f;
        s_x[m] = s;
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k) {
            int qi = 0;
            if (a != 0.0f) {
                float v = oracle_bf16_to_f32(x[m * ldx + k]) / s;
                v = rintf(v);
                if (v < -127.0f) v = -127.0f;
                if (v > 127.0f) v = 127.0f;
                qi = (int)v;
            }
            q[m * ldq + k] = (int8_t)qi;
            sum += qi;
        }
        if (q_sum) q_sum[m] = (int32_t)sum;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O6: W4A8 linear.  [Orin 从 FP 线性层到 INT4 DP4A 的数学推导] and [Orin INT32 accumulator 是否 */
/* 安全]:  acc_j = sum_i qW_ji qx_i  with qW = code - 8 in [-8, 7], computed here in int64;        */
/* y_j = sW_j * s_x * acc_j + b_j in fp64.  Weights are a group_size = 0 symmetric pack, so        */
/* sW_j = bf16(max_i |W_ji| / 7).  Returns the number of accumulators outside int32 (0 normally). */
/* acc (nullable) receives the int32 value; y is fp64 [M][d_out].                                 */
/* ------------------------------------------------------------------------------------------ */
int64_t oracle_w4a8(const int8_t *q, const float *s_x, int64_t M, int64_t ldq,
                    const uint8_t *qweight, const uint16_t *s_w, const uint16_t *bias,
                    int64_t d_out, int64_t d_in, int32_t *acc, double *y) {
    const int64_t k_pad = oracle_k_pad(d_in, 0);
    int64_t overflow = 0;
#pragma omp parallel for schedule(static) reduction(+ : overflow)
    for (int64_t j = 0; j < d_out; ++j) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t a = 0;
            for (int64_t k = 0; k < d_in; ++k) {
                const int64_t wq = (int64_t)code_at(qweight, k_pad, j, k) - 8;
                a += wq * (int64_t)q[m * ldq + k];
            }
            if (a > INT32_MAX || a < INT32_MIN) overflow += 1;
            if (acc) acc[m * d_out + j] = (int32_t)a;
            double r = (double)oracle_bf16_to_f32(s_w[j]) * (double)s_x[m] * (double)a;
            if (bias) r += (double)oracle_bf16_to_f32(bias[j]);
            y[m * d_out + j] = r;
        }
    }
    return overflow;
}

/* ------------------------------------------------------------------------------------------ */
/* O7: the gate of the MLP.  [Lab5 基础]: FFN(x) = W_down [SiLU(W_gate x) (.) (W_up x)] with      */
/* SiLU(v) = v sigma(v) = v / (1 + exp(-v)).  Given the two linear outputs g = W_gate x (+ b_gate) */
/* and u = W_up x (+ b_up) (O4 of the two halves of a fused gate/up weight), h_i = SiLU(g_i) u_i,  */
/* in fp64.                                                                                       */
/* ------------------------------------------------------------------------------------------ */
void oracle_silu_mul(const double *g, const double *u, int64_t n, double *h) {
    for (int64_t i = 0; i < n; ++i) {
        const double sigma = 1.0 / (1.0 + exp(-g[i]));
        h[i] = g[i] * sigma * u[i];
    }
}

/* ------------------------------------------------------------------------------------------ */
/* O8: repack of a weight trained on the 4-bit grid (QAT), groups of 32 input columns.          */
/* [QAT "Yeniden nicelendirme değil, yeniden paketleme"]: each group of 32 bf16 weights         */
/* already sits on a 16-level grid (levels -8..7 times a step); the step is found by dividing   */
/* the group's largest magnitude by m = 1, 2, ..., 8 and keeping the first step that reproduces */
/* the whole group, then refined by least squares over the group's values.                     */
/* Readings (the page does not fix them):                                                       */
/*   - "reproduces": for every value r of the group, v = r / s_m (fp32) lies within 1/16 of an   */
/*     integer level l = rint(v) with -8 <= l <= 7 (bf16 weights carry up to 2^-9 relative      */
/*     rounding, so an on-grid value is at most about 1/32 of a level away);                    */
/*   - least squares with the levels fixed: s = sum r l / sum l^2 (the sums are exact in fp64; */
/*     the quotient is taken in fp64, rounded to fp32, then to bf16);                           */
/*   - codes are l + 8 (the symmetric format); padded columns are zeros of the group (level 0); */
/*   - an all-zero group: m = 1, s = +0, codes 8;                                               */
/*   - a group that no m reproduces is off the grid: it is packed by O1's symmetric rule        */
/*     (s = bf16(max|r| / 7)) and its m is reported as 0.                                        */
/* w: bf16 bit patterns [d_out][ldw]; qweight [d_out][k_pad/2], scales [d_out][n_groups],        */
/* m_out [d_out][n_groups] (nullable), with k_pad = ceil(d_in / 32) * 32.                       */
/* ------------------------------------------------------------------------------------------ */
void oracle_qat_repack(const uint16_t *w, int64_t d_out, int64_t d_in, int64_t ldw,
                       uint8_t *qweight, uint16_t *scales, uint8_t *m_out) {
    const int64_t k_pad = oracle_k_pad(d_in, 32);
    const int64_t n_groups = k_pad / 32;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < d_out; ++j) {
        for (int64_t G = 0; G < n_groups; ++G) {
            float r[32];
            float amax = 0.0f;
            for (int t = 0; t < 32; ++t) {
                const int64_t k = G * 32 + t;
                r[t] = k < d_in ? oracle_bf16_to_f32(w[j * ldw + k]) : 0.0f;
                const float a = fabsf(r[t]);
                if (a > amax) amax = a;
            }
            int level[32];
            int found = 0;
            if (amax == 0.0f) {
                found = 1;
                for (int t = 0; t < 32; ++t) level[t] = 0;
            } else {
                for (int m = 1; m <= 8 && !found; ++m) {
                    const float s_m = amax / (float)m;
                    int ok = 1;
                    for (int t = 0; t < 32 && ok; ++t) {
                        const float v = r[t] / s_m;
                        const float l = rintf(v);
                        const float dev = fabsf(v - l);
                        if (l < -8.0f || l > 7.0f || dev > 0.0625f) ok = 0;
                        level[t] = (int)l;
                    }
                    if (ok) found = m;
                }
            }
            uint16_t s_bits;
            unsigned code[32];
            if (found) {
                double num = 0.0, den = 0.0;
                for (int t = 0; t < 32; ++t) {
                    num += (double)r[t] * (double)level[t];
                    den += (double)(level[t] * level[t]);
                }
                const float s32 = den > 0.0 ? (float)(num / den) : 0.0f;
                s_bits = oracle_f32_to_bf16(s32 + 0.0f);
                for (int t = 0; t < 32; ++t) code[t] = (unsigned)(level[t] + 8);
            } else {
                /* off the grid: O1's symmetric rule on this group */
                const float s_rtn = amax / 7.0f;
                s_bits = oracle_f32_to_bf16(s_rtn + 0.0f);
                const float s = oracle_bf16_to_f32(s_bits);
                for (int t = 0; t < 32; ++t) {
                    if (s == 0.0f) {
                        code[t] = 8;
                    } else {
                        float c = r[t] / s;
                        c = c + 8.0f;
                        c = rintf(c);
                        if (c < 0.0f) c = 0.0f;
                        if (c > 15.0f) c = 15.0f;
                        code[t] = (unsigned)c;
                    }
                }
            }
            scales[j * n_groups + G] = s_bits;
            if (m_out) m_out[j * n_groups + G] = (uint8_t)found;
            for (int t = 0; t < 32; t += 2)
                qweight[j * (k_pad / 2) + (G * 32 + t) / 2] = (uint8_t)(code[t] | (code[t + 1] << 4));
        }
    }
}
