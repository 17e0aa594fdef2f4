"""Host-side check of the activation encoding of the int8 decode kernel (no GPU): per token and
128-column group, x is replaced by X 2^-S with X = rint(x 2^S) and max|x_g| 2^S in [2^(B-1), 2^B),
then the integer sums are exact. The per-element error is at most 2^-(B+1) 2^(e+1) <= max|x_g|
2^-B: it scales with the group's largest value, so an outlier channel in a group costs the other
columns of the group their precision.

Emulated here in numpy on C2-style rows (g128 symmetric, 0.1% weight outliers at +-0.5) with 1%
of the input channels scaled x3000 ([Infra] section 2.4: outliers concentrate in a few channels):
the earlier 20-bit grid (B = 20, three 7-bit digits) misses the tolerance
|y - y_ref| <= 2e-3 (1 + |y_ref|) on some rows, the 30-bit grid the kernel now uses (B = 30, four
signed base-256 digits) stays far inside it. y_ref is the oracle's O4."""
import numpy as np

import oracle
import workloads


def _emulate(x_bits, qw, sc, d_in, bits):
    x = oracle.bf16_to_f32(x_bits).astype(np.float64)[0, :d_in]
    codes = oracle.unpack(qw)[:, :d_in].astype(np.float64) - 8.0
    s = oracle.bf16_to_f32(sc).astype(np.float64)
    y = np.zeros(qw.shape[0])
    for G in range(0, d_in, 128):
        xg = x[G:G + 128]
        amax = np.max(np.abs(xg))
        if amax == 0.0:
            continue
        S = (bits - 1) - (np.frexp(amax)[1] - 1)  # max|x| 2^S in [2^(bits-1), 2^bits)
        X = np.rint(np.ldexp(xg, S))               # ties to even, as the fp32 rounding
        assert np.max(np.abs(X)) < 2.0 ** bits
        y += s[:, G // 128] * (codes[:, G:G + 128] @ X) * 2.0 ** -S
    return y


def test_outlier_channels_need_the_30_bit_grid():
    rows, d_in = 4096, 3584
    worst = {20: 0.0, 30: 0.0}
    over = {20: 0, 30: 0}
    for seed in range(3):
        w = workloads.weight(700 + seed, 0, rows, d_in)
        workloads.add_weight_outliers(w, 700 + seed, 0, 1e-3, 0.5)
        qw, sc, _ = oracle.pack(w, 128, oracle.SYM)
        x = workloads.activations(700 + seed, 1, 1, d_in, 0.01, 3000.0)
        y_ref = oracle.w4a16(x, qw, sc, None, None, d_in, 128)[0]
        bound = 2e-3 * (1.0 + np.abs(y_ref))
        for b in (20, 30):
            r = np.abs(_emulate(x, qw, sc, d_in, b) - y_ref) / bound
            worst[b] = max(worst[b], float(r.max()))
            over[b] += int(np.sum(r > 1.0))
    assert over[20] > 0 and worst[20] > 1.0, worst  # the old grid misses the bar
    assert over[30] == 0 and worst[30] < 1e-3, worst  # the new one: three orders inside it


def test_exact_for_values_within_22_binades_of_the_group_maximum():
    """bf16 carries 8 significant bits: X = x 2^S exactly whenever |x| >= 2^-22 max|x_g|."""
    rng = np.random.default_rng(5)
    g = rng.normal(size=128).astype(np.float32)
    g[3] = 3000.0
    g[7] = np.float32(3000.0 * 2.0 ** -22)
    xb = workloads.to_bf16_bits(g)
    xf = oracle.bf16_to_f32(xb).astype(np.float64)
    amax = np.max(np.abs(xf))
    S = 29 - (np.frexp(amax)[1] - 1)
    X = np.rint(np.ldexp(xf, S))
    exact = np.abs(xf) >= amax * 2.0 ** -22
    assert np.all(X[exact] == np.ldexp(xf[exact], S))
    assert np.all(np.abs(X * 2.0 ** -S - xf) <= amax * 2.0 ** -30)
