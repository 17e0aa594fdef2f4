// qat_repack.hip -- repack of bf16 weights trained on the 4-bit grid (QAT) into the packed format.
//
// Page: [QAT] "Yeniden paketlenmiş QAT Gemma 4 26B-A4B, tek bir TPU v6e'de FP8 işlemenin 1.9 katı
// verimle sunuluyor" (section "Yeniden nicelendirme değil, yeniden paketleme"): every group of 32
// weights of a QAT export already lies on 16 levels (-8..7) times a step. The step is recovered by
// dividing the group's largest magnitude by m = 1, 2, ..., 8 and keeping the first m whose step
// reproduces every value of the group, then refined by least squares over the group; dividing by
// 8 unconditionally re-rounds every group whose peak is not at level -8.
//
// The readings this file implements (they decide integers, so each is one fixed sequence of IEEE
// operations):
//   * a value r is reproduced by the step s_m = max|r| / m (fp32) when v = r / s_m (fp32) lies
//     within 1/16 of the integer l = rint(v) and -8 <= l <= 7;
//   * the refined step is sum r l / sum l^2 with the levels fixed: the sums are exact, the
//     quotient is taken in fp64, rounded to fp32 and then to bf16; the codes are l + 8;
//   * an all-zero group has m = 1, step +0 and codes 8; padded columns are zeros of the group;
//   * a group no m reproduces is packed by the symmetric RTN rule of w4_pack (s = bf16(max|r| /
//     7), code = clip(rint(r / s + 8), 0, 15)) and reports m = 0.
//
// One lane per group: 64 bytes of bf16 (loaded coalesced by the wave and passed through LDS), the
// search in registers, one 16-byte store of the 32 codes, one bf16 scale and (optionally) the
// group's m. The search skips the
// divisors that the group's smallest nonzero value already rules out, and tests values with a
// multiplication by the step's reciprocal, falling back to the division only where the two could
// decide differently; the decisions are those of the rule above, bit for bit.
#include "w4_device.h"
#include "w4_launch.h"

namespace w4 {

namespace {

constexpr int kQatThreads = 256;

__global__ void __launch_bounds__(kQatThreads) qat_repack_kernel(
    const uint16_t *__restrict__ w, int d_in, int64_t ldw, int n_groups, int64_t total,
    uint8_t *__restrict__ qweight, uint16_t *__restrict__ scales, uint8_t *__restrict__ m_out) {
    // Coalesced loads: the wave's 64 groups are 256 16-byte chunks; chunk q = 64 i + lane is
    // loaded by lane q % 64 in load i and written to LDS at [q / 4][q % 4] (80 bytes per group,
    // so that 16 neighbouring lanes read their groups from distinct banks).
    __shared__ __align__(16) unsigned char lds[kQatThreads / kWave][kWave * 80];
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int64_t gid0 = static_cast<int64_t>(blockIdx.x) * kQatThreads + wv * kWave;
    const int64_t gid = gid0 + lane;
    const int64_t j0 = gid0 / n_groups;
    const int G0 = static_cast<int>(gid0 - j0 * n_groups);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = kWave * i + lane;
        const unsigned gq = static_cast<unsigned>(G0) + static_cast<unsigned>(q >> 2);
        const int64_t jq = j0 + gq / static_cast<unsigned>(n_groups);
        const int k = 32 * static_cast<int>(gq % static_cast<unsigned>(n_groups)) + 8 * (q & 3);
        uint4 v = {0u, 0u, 0u, 0u};
        if (gid0 + (q >> 2) < total && k < d_in)
            v = *reinterpret_cast<const uint4 *>(w + jq * ldw + k);
        *reinterpret_cast<uint4 *>(&lds[wv][(q >> 2) * 80 + (q & 3) * 16]) = v;
    }
    __syncthreads();
    if (gid >= total) return;
    const int64_t j = gid / n_groups;
    const int G = static_cast<int>(gid - j * n_groups);
    const int k0 = 32 * G;

    float r[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 v = *reinterpret_cast<const uint4 *>(&lds[wv][lane * 80 + c * 16]);
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            r[8 * c + e] = __uint_as_float((e & 1) ? (d[e >> 1] & 0xFFFF0000u) : (d[e >> 1] << 16));
    }
    if (k0 + 32 > d_in) {  // the row's last group: columns past d_in are zeros
#pragma unroll
        for (int t = 0; t < 32; ++t)
            if (k0 + t >= d_in) r[t] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) amax = fmaxf(amax, fabsf(r[t]));

    // Candidate divisors. A value b of the group can be reproduced by the step a / m only if
    // b m / a is within 1/16 of an integer, so m is dropped when that certainly fails for the
    // smallest nonzero magnitude b: the estimate b (1/a) m is within 2^-18 of b / (a / m) for
    // |b| <= a, m <= 8, and the test below keeps a margin of 2^-12. (If 1/a is not finite, every m
    // stays a candidate.)
    float b = amax;
#pragma unroll
    for (int t = 0; t < 32; ++t) b = fminf(b, r[t] != 0.0f ? fabsf(r[t]) : amax);
    uint32_t cand = 0xFFu;
    if (amax > 0.0f) {
        const float rcp_a = 1.0f / amax;
        if (__builtin_isfinite(rcp_a)) {
            const float tb = b * rcp_a;
            cand = 0u;
#pragma unroll
            for (int m = 1; m <= 8; ++m) {
                const float v = tb * static_cast<float>(m);
                const float dev = fabsf(v - rintf(v));
                if (dev <= 0.0625f + 0x1p-12f && v <= 8.0625f + 0x1p-12f) cand |= 1u << (m - 1);
            }
        }
    }

    float level[32];
    int found = 0;
    if (amax == 0.0f) {
        found = 1;
#pragma unroll
        for (int t = 0; t < 32; ++t) level[t] = 0.0f;
    } else {
        // every lane tests its own lowest remaining candidate, so the lanes of a wave test
        // their groups together whatever m each one needs
        uint32_t left = cand;
        while (left != 0u) {
            const int m = __builtin_ctz(left) + 1;
            left &= left - 1u;
            const float s_m = amax / static_cast<float>(m);
            // v = r / s_m decides. r (1 / s_m) is within 2^-19 of it: unless some value's
            // estimate lies within 2^-14 of the 1/16 threshold (or the reciprocal is not finite),
            // the estimates give the same levels and the same decision (near a half-integer the two
            // may round apart, but both are then rejected); otherwise the group is tested again
            // with the division.
            const float rcp = 1.0f / s_m;
            float dev_max = 0.0f, l_max = 0.0f, l_min = 0.0f, near = 1.0f;
#pragma unroll
            for (int t = 0; t < 32; ++t) {
                const float v = r[t] * rcp;
                const float l = rintf(v);
                const float dev = fabsf(v - l);
                dev_max = fmaxf(dev_max, dev);
                near = fminf(near, fabsf(dev - 0.0625f));
                l_max = fmaxf(l_max, l);
                l_min = fminf(l_min, l);
                level[t] = l;
            }
            if (!__builtin_isfinite(rcp) || near <= 0x1p-14f) {
                dev_max = 0.0f;
                l_max = 0.0f;
                l_min = 0.0f;
#pragma unroll
                for (int t = 0; t < 32; ++t) {
                    const float v = r[t] / s_m;
                    const float l = rintf(v);
                    dev_max = fmaxf(dev_max, fabsf(v - l));
                    l_max = fmaxf(l_max, l);
                    l_min = fminf(l_min, l);
                    level[t] = l;
                }
            }
            if (dev_max <= 0.0625f && l_max <= 7.0f && l_min >= -8.0f) {
                found = m;
                break;
            }
        }
    }

    uint32_t s_bits;
    uint32_t packed[4] = {0u, 0u, 0u, 0u};
    if (found) {
        // sum r l is exact in fp32 in any order: every value with l != 0 lies within a factor
        // of 8.6 of the step, so the products (8 + 4 significant bits) span at most 19 bit
        // positions and 32 of them at most 24; sum l^2 is a small integer
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            num = fmaf(r[t], level[t], num);
            den = fmaf(level[t], level[t], den);
        }
        const float s32 =
            den > 0.0f ? static_cast<float>(static_cast<double>(num) / static_cast<double>(den))
                       : 0.0f;
        s_bits = f32_to_bf16(s32 + 0.0f);
#pragma unroll
        for (int t = 0; t < 32; ++t)
            packed[t >> 3] |= static_cast<uint32_t>(level[t] + 8.0f) << (4 * (t & 7));
    } else {
        s_bits = f32_to_bf16(amax / 7.0f + 0.0f);
        const float s = bf16_to_f32(s_bits);
#pragma unroll
        for (int t = 0; t < 32; ++t) {
            float c = 8.0f;
            if (s != 0.0f) c = fminf(fmaxf(rintf(r[t] / s + 8.0f), 0.0f), 15.0f);
            packed[t >> 3] |= static_cast<uint32_t>(c) << (4 * (t & 7));
        }
    }
    const int64_t k_pad = static_cast<int64_t>(n_groups) * 32;
    *reinterpret_cast<uint4 *>(qweight + j * (k_pad / 2) + 16 * G) =
        uint4{packed[0], packed[1], packed[2], packed[3]};
    scales[gid] = static_cast<uint16_t>(s_bits);
    if (m_out) m_out[gid] = static_cast<uint8_t>(found);
}

}  // namespace

bool qat_repack_supported(int64_t d_out, int64_t n_groups) {
    return (d_out * n_groups + kQatThreads - 1) / kQatThreads < ((int64_t)1 << 31);
}

hipError_t launch_qat_repack(const uint16_t *w, int64_t d_out, int64_t d_in, int64_t ldw,
                             uint8_t *qweight, uint16_t *scales, uint8_t *m_out,
                             hipStream_t stream) {
    const int64_t n_groups = (d_in + 31) / 32;
    if (!qat_repack_supported(d_out, n_groups)) return hipErrorInvalidValue;
    const int64_t total = d_out * n_groups;
    const dim3 grid(static_cast<unsigned>((total + kQatThreads - 1) / kQatThreads));
    hipLaunchKernelGGL(qat_repack_kernel, grid, dim3(kQatThreads), 0, stream, w,
                       static_cast<int>(d_in), ldw, static_cast<int>(n_groups), total, qweight,
                       scales, m_out);
    return hipGetLastError();
}

}  // namespace w4
