"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, not by the oracle itself.

Each test names the passage or the mathematical fact it checks.  Pages:
  [Lab5]  "Lab 5: Gemma4 端到端推理优化"
  [Orin]  "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
  [Infra] "【infra之路】12-投机解码、量化与推理引擎对比"
Kinds of pin: printed values (tests/golden), closed forms (on-grid weights whose codes and scales
are known exactly), invariants, brute force over all candidate codes, and library reductions.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

SYM, ASYM = oracle.SYM, oracle.ASYM


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _f32(v):
    return np.float32(v)


def _bf16_value(bits):
    """Decode bf16 bits with plain integer arithmetic (independent of the oracle's helper)."""
    b = int(bits)
    sign = -1.0 if b & 0x8000 else 1.0
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if e == 0:
        return sign * m * 2.0 ** (-133)
    return sign * (1.0 + m / 128.0) * 2.0 ** (e - 127)


# ------------------------------------------------------------------------------------------
# Nibble layout [Lab5 INT4 线性量化, 融合INT4反量化与矩阵乘], [Orin DP4A 做了什么]
# ------------------------------------------------------------------------------------------
def test_uint32_nibble_order_printed(golden_dir):
    g = _golden(golden_dir, "nibble_layout.json")
    word = int(g["uint32_hex"], 16)
    assert word == g["uint32_le"]
    row = np.frombuffer(np.uint32(word).tobytes(), dtype=np.uint8).reshape(1, 4)
    codes = oracle.unpack(row)
    assert codes.ravel().tolist() == g["codes_in_k_order"]


def test_all_byte_values_round_trip():
    row = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = oracle.unpack(row)
    # invariant: recombining the two codes of each byte gives the byte back
    re = (codes[0, 0::2].astype(np.int64) | (codes[0, 1::2].astype(np.int64) << 4))
    assert re.tolist() == list(range(256))
    assert codes.max() <= 15


def test_packed_row_bytes_printed(golden_dir):
    g = _golden(golden_dir, "packed_row_bytes.json")
    H = g["H"]
    w = workloads.weight(1, 0, 2, H)
    qw, sc, _ = oracle.pack(w, 128, SYM)
    assert qw.shape[1] == g["bytes_per_row"]["int4"]
    assert 2 * H == g["bytes_per_row"]["fp16"] and H == g["bytes_per_row"]["int8"]


def test_unpack_aliasing_regression():
    """[Lab5 量化正确性修正]: writing the low codes in place into the byte view before reading the
    high codes corrupts them; the oracle computes both nibbles from untouched bytes."""
    rng = np.random.default_rng(7)
    packed = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    good = oracle.unpack(packed)
    # emulate the faulty in-place interleave on one shared uint8 buffer
    buf = np.zeros((3, 128), dtype=np.uint8)
    buf[:, :64] = packed
    view = buf[:, :64]  # the "packed" view aliases the output storage
    buf[:, 0::2] = view & 0x0F
    buf[:, 1::2] = view >> 4
    assert not np.array_equal(buf, good)
    # the corrected form: independent low/high, then stack and flatten
    low, high = packed & 0x0F, packed >> 4
    fixed = np.stack((low, high), axis=-1).reshape(3, 128)
    assert np.array_equal(fixed, good)


# ------------------------------------------------------------------------------------------
# Closed forms: on-grid weights.  [Lab5 INT4 线性量化]
# ------------------------------------------------------------------------------------------
def _on_grid_group(codes, s, z):
    return np.array([(c - z) * s for c in codes], dtype=np.float32)


def test_asym_on_grid_codes_scales_zeros_exact():
    """Values r = s (c - z) with power-of-two s and every code 0..15 present round-trip exactly:
    s = (max - min)/15, z = round(-min/s), code = c, and each byte is c_even | c_odd << 4."""
    rng = np.random.default_rng(11)
    rows = []
    want_codes = []
    for j in range(6):
        s = 2.0 ** (-4 - j)
        z = [0, 3, 5, 8, 12, 15][j]
        c = np.concatenate([np.arange(16), rng.integers(0, 16, size=16)])
        rng.shuffle(c)
        rows.append(_on_grid_group(c, s, z))
        want_codes.append(c)
    w = np.stack(rows)
    qw, sc, zr = oracle.pack(w, 32, ASYM)
    for j in range(6):
        assert _bf16_value(sc[j, 0]) == 2.0 ** (-4 - j)
        assert _bf16_value(zr[j, 0]) == [0, 3, 5, 8, 12, 15][j]
        c = want_codes[j]
        assert qw[j].tolist() == [int(c[2 * i]) | (int(c[2 * i + 1]) << 4) for i in range(16)]
    wh = oracle.dequant(qw, sc, zr, 32, 32)
    assert np.array_equal(wh, w.astype(np.float64))


def test_sym_on_grid_divides_by_seven():
    """Symmetric: s = max|r| / 7 (not / 8), codes offset by 8; a group whose extreme is 7 s0 gets
    s = s0 exactly and codes c + 8 for r = c s0."""
    s0 = 2.0 ** -6
    c = np.array(list(range(-7, 8)) * 2 + [7, -7], dtype=np.int64)
    w = (c * s0).astype(np.float32).reshape(1, 32)
    qw, sc, _ = oracle.pack(w, 32, SYM)
    assert _bf16_value(sc[0, 0]) == s0
    codes = oracle.unpack(qw)[0]
    assert codes.tolist() == (c + 8).tolist()
    # the "max/8" rule would have given 7/8 s0 and moved every code
    assert 0 not in codes.tolist()


def test_zero_group_and_per_row_scale():
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 5] = 0.7
    qw, sc, _ = oracle.pack(w, 0, SYM)
    assert sc[0, 0] == 0 and oracle.unpack(qw)[0].tolist() == [8] * 64
    # per-row scale (group_size 0) for W4A8 [Orin 从 FP 线性层到 INT4 DP4A 的数学推导]
    assert abs(_bf16_value(sc[1, 0]) - 0.1) <= 0.1 * 2 ** -8
    qa, sa, za = oracle.pack(w, 0, ASYM)
    assert sa[0, 0] == 0 and za[0, 0] == 0 and oracle.unpack(qa)[0].tolist() == [0] * 64


# ------------------------------------------------------------------------------------------
# Scales against exact rationals; codes against brute force over all 16 candidates.
# ------------------------------------------------------------------------------------------
def _check_groups(w, qw, sc, zr, g, mode):
    d_out, d_in = w.shape
    kp = oracle.k_pad(d_in, g)
    ng = oracle.n_groups(d_in, g)
    gs = kp // ng
    codes = oracle.unpack(qw)
    wp = np.zeros((d_out, kp), dtype=np.float64)
    wp[:, :d_in] = w
    for j in range(d_out):
        for G in range(ng):
            seg = wp[j, G * gs:(G + 1) * gs]
            s = _bf16_value(sc[j, G])
            if mode == SYM:
                exact = Fraction(float(np.max(np.abs(seg)))) / 7
                z = 8.0
            else:
                exact = (Fraction(float(seg.max())) - Fraction(float(seg.min()))) / 15
                z = _bf16_value(zr[j, G])
            # bf16 rounding of an fp32 quotient: within half a bf16 ulp plus an fp32 ulp
            assert abs(Fraction(s) - exact) <= exact * Fraction(1, 256) * Fraction(1025, 1024)
            if mode == ASYM and s != 0:
                ratio = -Fraction(float(seg.min())) / Fraction(s)
                lo = int(np.floor(float(ratio)))
                assert z in (lo, lo + 1)
                frac = float(ratio - lo)
                if abs(frac - 0.5) > 1e-5:
                    assert z == (lo if frac < 0.5 else lo + 1)
            c = codes[j, G * gs:(G + 1) * gs].astype(np.float64)
            if s == 0:
                assert np.all(c == z)
                continue
            cand = s * (np.arange(16)[None, :] - z)  # every representable value of the group
            err = np.abs(seg[:, None] - cand)
            best = err.min(axis=1)
            mine = np.abs(seg - s * (c - z))
            # RTN: the chosen code is a nearest grid point (up to fp32 rounding of r/s + z)
            assert np.all(mine <= best + 4e-7 * s * (1 + np.abs(seg / s) + abs(z))), (j, G)
    return codes


@pytest.mark.parametrize("g", [32, 64, 128, 256, 0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_scales_and_codes_brute_force(g, mode):
    w = workloads.weight(5, g + mode, 12, 300)
    workloads.add_weight_outliers(w, 5, 99, 0.01, 0.5)
    qw, sc, zr = oracle.pack(w, g, mode)
    codes = _check_groups(w, qw, sc, zr, g, mode)
    if mode == SYM:
        # RTN with s = max|r|/7 never reaches code 0 (= -8)
        assert codes.min() >= 1


def test_extreme_entries_map_to_edge_codes():
    w = workloads.weight(6, 0, 64, 128)
    qs, ss, _ = oracle.pack(w, 128, SYM)
    cs = oracle.unpack(qs)
    qa, sa, za = oracle.pack(w, 128, ASYM)
    ca = oracle.unpack(qa)
    for j in range(64):
        i = int(np.argmax(np.abs(w[j])))
        assert cs[j, i] == (15 if w[j, i] > 0 else 1)
        assert ca[j, int(np.argmin(w[j]))] == 0
        assert ca[j, int(np.argmax(w[j]))] in (14, 15)


def test_unclipped_error_at_most_half_scale():
    """[Infra 2.2 量化的基本概念]: each value is off by at most scale/2 after round-to-nearest."""
    w = workloads.weight(8, 0, 32, 512)
    for mode in (SYM, ASYM):
        qw, sc, zr = oracle.pack(w, 64, mode)
        wh = oracle.dequant(qw, sc, zr, 512, 64)
        s = np.repeat(oracle.bf16_to_f32(sc).astype(np.float64), 64, axis=1)
        codes = oracle.unpack(qw)
        interior = (codes > 0) & (codes < 15)
        assert np.all(np.abs(wh - w)[interior] <= 0.5 * s[interior] * (1 + 1e-6))


# ------------------------------------------------------------------------------------------
# Padding [Lab5 INT4 线性量化]: padded columns decode to exactly zero.
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [SYM, ASYM])
@pytest.mark.parametrize("d_in,g", [(3600, 128), (100, 32), (70, 0), (200, 64)])
def test_padding_decodes_to_zero(mode, d_in, g):
    w = workloads.weight(9, d_in, 16, d_in)
    w += 0.05  # mostly positive groups: the pads are what pulls min to 0
    qw, sc, zr = oracle.pack(w, g, mode)
    kp = oracle.k_pad(d_in, g)
    assert kp > d_in
    codes = oracle.unpack(qw)
    wh = oracle.dequant(qw, sc, zr, d_in, g)
    assert np.all(wh[:, d_in:] == 0.0)
    ng = oracle.n_groups(d_in, g)
    gs = kp // ng
    last = (d_in - 1) // gs
    for j in range(16):
        z = 8 if mode == SYM else _bf16_value(zr[j, last])
        assert np.all(codes[j, d_in:] == z)
        if mode == ASYM:
            assert 0 <= z <= 15


# ------------------------------------------------------------------------------------------
# W4A16 contraction
# ------------------------------------------------------------------------------------------
def test_w4a16_basis_probes_exact():
    """x = e_k gives y[j] = r_hat[j][k] exactly (one exact product)."""
    w = workloads.weight(10, 0, 24, 96)
    for mode, g in ((SYM, 32), (ASYM, 32), (ASYM, 0)):
        qw, sc, zr = oracle.pack(w, g, mode)
        wh = oracle.dequant(qw, sc, zr, 96, g)
        for k in (0, 1, 31, 32, 33, 95):
            x = np.zeros((1, 96), dtype=np.uint16)
            x[0, k] = 0x3F80  # bf16 1.0
            y = oracle.w4a16(x, qw, sc, zr, None, 96, g)
            assert np.array_equal(y[0], wh[:, k])


def test_w4a16_library_reduction_tiny():
    """On small shapes the loop equals numpy's fp64 matmul of x and the decoded weight."""
    w = workloads.weight(12, 0, 40, 200)
    x = workloads.activations(12, 0, 5, 200)
    b = workloads.bias(12, 0, 40)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    bf = oracle.bf16_to_f32(b).astype(np.float64)
    for mode, g in ((SYM, 32), (ASYM, 64), (SYM, 0)):
        qw, sc, zr = oracle.pack(w, g, mode)
        wh = oracle.dequant(qw, sc, zr, 200, g)[:, :200]
        y = oracle.w4a16(x, qw, sc, zr, b, 200, g)
        assert np.allclose(y, xf @ wh.T + bf, rtol=0, atol=1e-12)
        pts = oracle.w4a16_points(x, qw, sc, zr, b, 200, g, [0, 4, 2], [0, 39, 17])
        assert np.array_equal(pts, y[[0, 4, 2], [0, 39, 17]])


def test_w4a16_constant_codes():
    """All codes equal to z give y = b exactly; x = 1 with codes z + 1 gives the sum of the
    scales over the real columns of each group."""
    d_out, d_in, g = 8, 100, 32
    kp, ng = oracle.k_pad(d_in, g), oracle.n_groups(d_in, g)
    sc = oracle.f32_to_bf16(np.linspace(0.01, 0.08, d_out * ng).reshape(d_out, ng))
    zr = oracle.f32_to_bf16(np.tile(np.arange(ng, dtype=np.float32) + 3, (d_out, 1)))
    x = workloads.activations(13, 0, 2, d_in)
    b = workloads.bias(13, 0, d_out)
    codes = np.repeat(oracle.bf16_to_f32(zr).astype(np.uint8), g, axis=1)
    qw = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    y = oracle.w4a16(x, qw, sc, zr, b, d_in, g)
    assert np.array_equal(y, np.tile(oracle.bf16_to_f32(b).astype(np.float64), (2, 1)))
    codes1 = codes + 1
    qw1 = (codes1[:, 0::2] | (codes1[:, 1::2] << 4)).astype(np.uint8)
    ones = np.full((1, d_in), 0x3F80, dtype=np.uint16)
    y1 = oracle.w4a16(ones, qw1, sc, zr, None, d_in, g)
    counts = np.array([min(g, d_in - G * g) for G in range(ng)], dtype=np.float64)
    want = (oracle.bf16_to_f32(sc).astype(np.float64) * counts).sum(axis=1)
    assert np.allclose(y1[0], want, rtol=1e-15, atol=0)


# ------------------------------------------------------------------------------------------
# Activation quantization [Orin 从 FP 线性层到 INT4 DP4A 的数学推导], [Infra 2.2, 2.4]
# ------------------------------------------------------------------------------------------
def test_act_quant_outlier_example_printed(golden_dir):
    g = _golden(golden_dir, "int8_activation_examples.json")["outlier_example"]
    x = workloads.to_bf16_bits(np.array([[g["max"], g["value"], -0.02, 0.0]], np.float32))
    q, s, qs = oracle.act_quant(x)
    assert abs(s[0] - g["scale_approx"]) < 5e-4
    assert q[0, 1] == g["code"] and q[0, 0] == 127
    deq = float(s[0]) * int(q[0, 1])
    assert abs(deq - g["dequant_approx"]) < 5e-4
    rel = abs(deq - g["value"]) / g["value"]
    assert abs(rel - g["relative_error_approx"]) < 0.01
    assert qs[0] == int(q[0].astype(np.int64).sum())


def test_act_quant_symmetric_example_printed(golden_dir):
    g = _golden(golden_dir, "int8_activation_examples.json")["symmetric_example"]
    x = workloads.activations(14, 0, 1, 4096)
    xf = oracle.bf16_to_f32(x)
    xf = xf / np.abs(xf).max() * np.float32(g["max"])
    x = workloads.to_bf16_bits(xf)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    q, s, _ = oracle.act_quant(x)
    assert abs(s[0] - g["scale_approx"]) < 1e-4
    err = np.abs(xf[0] - float(s[0]) * q[0])
    assert err.max() <= g["max_error_approx"] + 1e-4
    assert err.max() <= float(s[0]) / 2 * (1 + 1e-6)


def test_act_quant_brute_force_and_edges():
    x = workloads.activations(15, 0, 6, 333, outlier_frac=0.01, outlier_scale=20.0)
    x[3] = 0  # an all-zero token
    q, s, qs = oracle.act_quant(x)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    cand = np.arange(-127, 128, dtype=np.float64)
    for m in range(6):
        if m == 3:
            assert s[m] == 0 and not q[m].any() and qs[m] == 0
            continue
        a = np.abs(xf[m]).max()
        assert abs(Fraction(float(s[m])) - Fraction(a) / 127) <= Fraction(a) / 127 * 2 ** -23
        i = int(np.argmax(np.abs(xf[m])))
        assert abs(int(q[m, i])) == 127
        err = np.abs(xf[m][:, None] - float(s[m]) * cand[None, :])
        mine = np.abs(xf[m] - float(s[m]) * q[m])
        assert np.all(mine <= err.min(axis=1) + 1e-6 * float(s[m]))
        assert qs[m] == int(q[m].astype(np.int64).sum())


# ------------------------------------------------------------------------------------------
# W4A8 [Orin INT32 accumulator 是否安全]
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("H", [3584, 18944])
def test_w4a8_worst_case_accumulator_printed(golden_dir, H):
    g = _golden(golden_dir, "int32_accumulator.json")
    assert g["max_abs_weight_code"] * g["max_abs_activation_code"] == g["max_abs_product"]
    qw = np.zeros((2, H // 2), dtype=np.uint8)  # all codes 0, i.e. weight -8
    sw = oracle.f32_to_bf16(np.array([1.0, 0.5], np.float32))
    q = np.full((1, H), -127, dtype=np.int8)
    s_x = np.array([1.0], np.float32)
    acc, y, nov = oracle.w4a8(q, s_x, qw, sw, None, H)
    want = H * g["max_abs_product"]
    if H == g["H"]:
        assert want == g["worst_case_accumulator"]
    assert nov == 0 and acc[0].tolist() == [want, want]
    assert want < g["int32_max"]
    assert y[0].tolist() == [float(want), 0.5 * want]


def test_w4a8_brute_force_python_ints():
    rng = np.random.default_rng(16)
    d_out, d_in = 7, 90
    kp = oracle.k_pad(d_in, 0)
    codes = rng.integers(0, 16, size=(d_out, kp))
    codes[:, d_in:] = 8
    qw = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    q = rng.integers(-127, 128, size=(3, d_in)).astype(np.int8)
    sw = workloads.to_bf16_bits(rng.uniform(0.001, 0.01, d_out))
    b = workloads.bias(16, 0, d_out)
    s_x = np.array([0.01, 0.5, 2.0], np.float32)
    acc, y, _ = oracle.w4a8(q, s_x, qw, sw, b, d_in)
    for m in range(3):
        for j in range(d_out):
            a = sum((int(codes[j, k]) - 8) * int(q[m, k]) for k in range(d_in))
            assert acc[m, j] == a
            want = _bf16_value(sw[j]) * float(s_x[m]) * a + _bf16_value(b[j])
            assert abs(y[m, j] - want) <= 1e-12 * (1 + abs(want))


def test_w4a8_end_to_end_within_quantization_bound():
    """y approximates x W^T: the gap is bounded by the two quantization errors, each at most
    half a step [Infra 2.2]."""
    cfg = workloads.C5
    lin = cfg.linears[0]
    w = workloads.weight(17, 0, 64, lin.d_in)
    x = workloads.activations(17, 0, 1, lin.d_in, 0.01, 20.0)
    qw, sc, _ = oracle.pack(w, 0, SYM)
    q, s_x, _ = oracle.act_quant(x)
    acc, y, nov = oracle.w4a8(q, s_x, qw, sc[:, 0], None, lin.d_in)
    assert nov == 0
    xf = oracle.bf16_to_f32(x).astype(np.float64)[0]
    ref = w.astype(np.float64) @ xf
    sw = oracle.bf16_to_f32(sc[:, 0]).astype(np.float64)
    wh = oracle.dequant(qw, sc, None, lin.d_in, 0)[:, :lin.d_in]
    xq = float(s_x[0]) * q[0].astype(np.float64)
    bound = (np.abs(w - wh) * np.abs(xf)).sum(axis=1) + (np.abs(wh) * np.abs(xf - xq)).sum(axis=1)
    assert np.all(np.abs(y[0] - ref) <= bound * (1 + 1e-9) + 1e-9)
    assert np.all(np.abs(xf - xq) <= float(s_x[0]) / 2 * (1 + 1e-6))
    assert np.all(sw > 0)


# ------------------------------------------------------------------------------------------
# O7: the gate of the MLP [Lab5 基础]: FFN(x) = W_down [SiLU(W_gate x) (.) (W_up x)],
# SiLU(v) = v sigma(v)
# ------------------------------------------------------------------------------------------
def test_silu_mul_closed_forms():
    """sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so SiLU(+-ln 3) = +-ln 3 * {3/4, 1/4}; sigma(0) =
    1/2; the logistic function at 1 is 0.7310585786300049 (e / (1 + e))."""
    import math
    ln3 = math.log(3.0)
    g = np.array([ln3, -ln3, 0.0, 1.0, -1.0])
    h = oracle.silu_mul(g, np.ones_like(g))
    e = math.e
    want = [ln3 * 0.75, -ln3 * 0.25, 0.0, e / (1 + e), -1.0 / (1 + e)]
    assert np.allclose(h, want, rtol=1e-15, atol=0)
    assert abs(h[3] - 0.7310585786300049) <= 1e-16


def test_silu_mul_identities_and_limits():
    """SiLU(v) - SiLU(-v) = v (sigma(v) + sigma(-v) = 1); SiLU(v) -> v for large v and -> 0- for
    very negative v; h is linear in u; SiLU(v) >= -0.2785 (its minimum, at v = -1.2785)."""
    v = np.linspace(-30.0, 30.0, 601)
    one = np.ones_like(v)
    d = oracle.silu_mul(v, one) - oracle.silu_mul(-v, one)
    assert np.allclose(d, v, rtol=0, atol=1e-12)
    big = oracle.silu_mul(np.array([40.0, -40.0, -800.0]), np.ones(3))
    assert big[0] == 40.0 and -1e-15 < big[1] < 0.0 and big[2] == 0.0
    u = np.random.default_rng(7).normal(size=v.shape)
    assert np.allclose(oracle.silu_mul(v, 2.0 * u), 2.0 * oracle.silu_mul(v, u), rtol=1e-15)
    assert oracle.silu_mul(v, one).min() >= -0.27846454276107


def test_w4a16_silu_mul_takes_gate_then_up():
    """A fused gate/up weight is gate rows [0, H) then up rows [H, 2H): with x = e_k the result is
    SiLU(w_hat_gate[j][k]) * w_hat_up[j][k], computed here in Python floats from the dequantized
    weights (each row pair has distinct gate and up values, so swapped halves fail)."""
    import math
    H, d_in = 8, 64
    w = workloads.weight(41, 0, 2 * H, d_in)
    w[:H] *= 40.0  # gate values far from the up values
    qw, sc, zr = oracle.pack(w, 32, ASYM)
    wh = oracle.dequant(qw, sc, zr, d_in, 32)
    for k in (0, 5, 33, 63):
        x = np.zeros((1, d_in), dtype=np.uint16)
        x[0, k] = 0x3F80
        h = oracle.w4a16_silu_mul(x, qw, sc, zr, None, d_in, 32)[0]
        for j in range(H):
            g, u = float(wh[j, k]), float(wh[H + j, k])
            assert abs(h[j] - g / (1.0 + math.exp(-g)) * u) <= 1e-12 * (1.0 + abs(h[j]))


# ------------------------------------------------------------------------------------------
# O8: repack of weights trained on the 4-bit grid.  [QAT] "Yeniden paketlenmiş QAT Gemma 4
# 26B-A4B, tek bir TPU v6e'de FP8 işlemenin 1.9 katı verimle sunuluyor", section "Yeniden
# nicelendirme değil, yeniden paketleme": 32-wide groups of bf16 weights on levels -8..7 times a
# step; the step is the group maximum over the first m in 1..8 that reproduces the group,
# refined by least squares; the max/8 rule re-rounds groups whose peak is below level 8.
# ------------------------------------------------------------------------------------------
def _rne_bf16(vals):
    """fp32 -> bf16 bits, round to nearest even, with integer arithmetic on the fp32 bits."""
    u = np.asarray(vals, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)


def _bits_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def _grid_groups(rng, n, peaks, steps):
    """n groups of 32 levels in [-8, 7], each holding the level +-1 and its peak level (signed)."""
    lv = np.zeros((n, 32), dtype=np.int64)
    for i in range(n):
        p = peaks[i % len(peaks)]
        P = abs(p)
        row = rng.integers(-min(P, 8), min(P, 7) + 1, size=32)
        row = np.clip(row, -P, P if p > 0 else P - 1 if P == 8 else P)
        row[rng.integers(0, 32)] = p
        k = rng.integers(0, 32)
        while row[k] == p:
            k = rng.integers(0, 32)
        row[k] = 1 if rng.random() < 0.5 else -1
        lv[i] = row
    st = np.asarray([steps[i % len(steps)] for i in range(n)], dtype=np.float64)
    return lv, st


def _nibbles(qw):
    return np.stack([qw & 0xF, qw >> 4], axis=-1).reshape(qw.shape[0], -1)


@pytest.mark.parametrize("peak", [7, -8, -7, 5, -3, 2, 1, 6, -5])
def test_qat_repack_exact_grid_closed_form(peak):
    """Steps with at most 4 significant bits: every s l is an exact bf16, so the group's codes are
    its levels + 8, its m is the peak level's magnitude (a level +-1 rules out coarser m), and
    the least-squares step is the step itself."""
    rng = np.random.default_rng(80 + peak)
    steps = [0.125, 0.01171875, 3.0, 2.0 ** -20 * 1.5, 0.4375]
    lv, st = _grid_groups(rng, 10, [peak], steps)
    w = _rne_bf16((lv * st[:, None]).astype(np.float32))
    assert np.array_equal(_bits_f32(w).astype(np.float64), lv * st[:, None])  # exact on the grid
    qw, sc, m = oracle.qat_repack(w.reshape(1, -1))
    assert np.array_equal(_nibbles(qw)[0], (lv + 8).reshape(-1))
    assert np.array_equal(_bits_f32(sc[0]).astype(np.float64), st)
    assert np.all(m == abs(peak))
    # the round trip is exact
    assert np.array_equal(_bits_f32(sc[0])[:, None].astype(np.float64) * lv, _bits_f32(w).reshape(10, 32))


def test_qat_repack_bf16_rounded_grid():
    """Random bf16 steps: s l rounded to bf16, as a trained export stores it.  Every group is found
    on the grid with its own levels; the refined step is the generating step or a neighbouring bf16
    value, and most values come back bit for bit (the page reports 92.6%)."""
    rng = np.random.default_rng(81)
    n = 400
    steps = _bits_f32(rng.integers(0x3A00, 0x3D80, size=n).astype(np.uint16)).astype(np.float64)
    lv, st = _grid_groups(rng, n, [7, -8, 6, -7, 4, -5, 3], steps)
    w = _rne_bf16((lv * st[:, None]).astype(np.float32))
    qw, sc, m = oracle.qat_repack(w.reshape(4, -1))
    assert np.array_equal(_nibbles(qw).reshape(n, 32), lv + 8)
    assert np.all(m.reshape(-1) == np.abs(lv).max(axis=1))
    s = _bits_f32(sc.reshape(-1)).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(st)) - 7)
    assert np.all(np.abs(s - st) <= ulp)
    back = _rne_bf16((s[:, None] * lv).astype(np.float32))
    frac = np.mean(back == w.reshape(n, 32))
    assert frac >= 0.9, frac


def test_qat_repack_least_squares_step():
    """Levels fixed, the step is sum r l / sum l^2: with a peak of 7.03125 on a unit grid the
    maximum over 7 would give 1.0045 (bf16 1.0078125); the least-squares step rounds to 1.0."""
    lv = np.array([7, 1, -1, 3, -8, 2, 0, 5] * 4, dtype=np.int64)
    lv[8:] = np.resize([1, -2, 4, -3, 6, 0, -7, 2], 24)
    lv[4] = -5
    r = lv.astype(np.float64)
    r[0] = 7.03125  # bf16: 1.7578125 * 4
    w = _rne_bf16(r.astype(np.float32))
    assert np.array_equal(_bits_f32(w).astype(np.float64), r)
    qw, sc, m = oracle.qat_repack(w.reshape(1, -1))
    assert m[0, 0] == 7
    assert np.array_equal(_nibbles(qw)[0], lv + 8)
    ls = Fraction(0)
    for t in range(32):
        ls += Fraction(r[t]) * int(lv[t])
    ls /= int((lv * lv).sum())
    assert float(ls) == pytest.approx(1.0 + 0.03125 * 7 / int((lv * lv).sum()), rel=1e-12)
    assert _bits_f32(sc[0])[0] == 1.0
    assert np.float32(7.03125) / np.float32(7.0) > np.float32(1.00390625)  # max/7 would round up


def test_qat_repack_reproduces_where_max_over_8_rerounds():
    """A group whose peak is +7 steps: the max/8 rule takes the step 7/8 too small and moves
    values off their levels; the search keeps every value."""
    lv = np.array([7, -3, 1, 0, 5, -6, 2, -1] * 4, dtype=np.int64)
    r = (lv * 0.25).astype(np.float32)
    w = _rne_bf16(r)
    qw, sc, m = oracle.qat_repack(w.reshape(1, -1))
    s = _bits_f32(sc[0])[0]
    assert m[0, 0] == 7 and s == 0.25
    assert np.array_equal(s * (_nibbles(qw)[0].astype(np.float32) - 8), r)
    s8 = np.float32(np.abs(r).max() / 8)
    back8 = s8 * np.clip(np.rint(r / s8), -8, 7)
    assert np.count_nonzero(back8 != r) > 0


def test_qat_repack_off_grid_falls_back_to_rtn():
    """Groups off the grid (normal samples) report m = 0 and are packed by the symmetric RTN
    rule O1 applies to the same values."""
    rng = np.random.default_rng(82)
    r = rng.normal(0, 0.02, size=(3, 96)).astype(np.float32)
    w = _rne_bf16(r)
    qw, sc, m = oracle.qat_repack(w)
    assert np.all(m == 0)
    qw1, sc1, _ = oracle.pack(_bits_f32(w), 32, SYM)
    assert np.array_equal(qw, qw1) and np.array_equal(sc, sc1)


def test_qat_repack_tolerance_and_level_range():
    """A value 0.047 of a level off its level is still on the grid; 0.078 is not; a peak at
    +8 steps is not a level of the grid."""
    base = np.array([7, -3, 1, 0, 5, -6, 2, -1] * 4, dtype=np.float32)
    near, far, plus8 = base.copy(), base.copy(), base.copy()
    near[1] = -3.046875
    far[1] = -3.078125
    plus8[0] = 8.0
    w = _rne_bf16(np.stack([near, far, plus8]))
    assert np.array_equal(_bits_f32(w), np.stack([near, far, plus8]))
    qw, sc, m = oracle.qat_repack(w)
    assert m[:, 0].tolist() == [7, 0, 0]
    assert np.array_equal(_nibbles(qw)[0], base.astype(np.int64) + 8)


def test_qat_repack_zero_group_pads_and_stride():
    """An all-zero group (m = 1, scale +0, codes 8), a ragged last group whose pads are level 0,
    and columns past d_in (NaN here) that are never read."""
    d_in, ldw = 40, 48
    w = np.full((2, ldw), 0x7FC0, dtype=np.uint16)
    w[0, :d_in] = 0
    lv = np.array([3, -2, 1, 0, -1, 2, 3, -3], dtype=np.int64)
    w[1, :32] = _rne_bf16(np.resize(lv, 32).astype(np.float32) * 0.5)
    w[1, 32:d_in] = _rne_bf16(lv.astype(np.float32) * 0.125)
    qw, sc, m = oracle.qat_repack(w, d_in)
    assert qw.shape == (2, 32) and sc.shape == (2, 2)
    assert m[0].tolist() == [1, 1] and sc[0].tolist() == [0, 0]
    assert np.all(_nibbles(qw)[0] == 8)
    assert m[1].tolist() == [3, 3]
    assert _bits_f32(sc[1]).tolist() == [0.5, 0.125]
    codes = _nibbles(qw)[1]
    assert np.array_equal(codes[32:40], lv + 8) and np.all(codes[40:] == 8)


# ------------------------------------------------------------------------------------------
# O9: GPTQ.  [Lab5] "从 RTN 到 GPTQ": the layer objective ||X (W - Q)^T||_F^2, H = (2/N) X^T X,
# dead columns, damping lambda = alpha mean(diag H), H^-1 = U^T U, e_i = (w_i - q_i) / U_ii,
# W[:, i:] -= e_i U[i, i:], L_pred = 1/2 sum ||w_i - q_i||^2 / U_ii^2.
# ------------------------------------------------------------------------------------------
import oracle.gptq as gq  # noqa: E402


def _calib(seed, N, d_in, dead=()):
    """bf16 calibration activations with correlated channels (a few latent factors plus noise);
    the listed columns are zero in every row."""
    rng = np.random.default_rng(seed)
    lat = rng.normal(size=(N, max(1, d_in // 4)))
    mix = rng.normal(size=(lat.shape[1], d_in)) / 2.0
    x = lat @ mix + 0.3 * rng.normal(size=(N, d_in))
    x[:, list(dead)] = 0.0
    return _rne_bf16(x.astype(np.float32))


def _deq(codes, scales_bits, zeros_bits, d_in, span):
    """s (code - z) per column, from the stored bits (plain arithmetic)."""
    G = np.arange(d_in) // span
    s = _bits_f32(scales_bits)[:, G].astype(np.float64)
    z = _bits_f32(zeros_bits)[:, G].astype(np.float64) if zeros_bits is not None else 8.0
    return s * (codes[:, :d_in].astype(np.float64) - z)


@pytest.mark.parametrize("g,mode", [(32, SYM), (128, ASYM), (0, SYM)])
def test_gptq_predicted_loss_is_the_objective(g, mode):
    """With H = (2/N) X^T X + lambda I and the updates of the page, W - Q = E U row by row, so
    1/2 (W - Q) H (W - Q)^T = 1/2 sum e_i^2 = L_pred: L_pred equals
    (1/N) ||X (W - Q)^T||_F^2 + (lambda / 2) ||W - Q||_F^2, computed here from X, W and the packed
    result alone."""
    d_out, d_in, N = 24, 200, 96
    w = workloads.weight(90, g + mode, d_out, d_in)
    xb = _calib(90 + g, N, d_in)
    r = gq.gptq(w, xb, g, mode)
    kp = oracle.k_pad(d_in, g)
    span = kp // oracle.n_groups(d_in, g)
    q = _deq(r["codes"], r["scales"], r["zeros"], d_in, span)
    x = _bits_f32(xb).astype(np.float64)
    lam = 0.01 * np.mean(2.0 / N * np.sum(x * x, axis=0))
    d = w.astype(np.float64) - q
    obj = np.sum((x @ d.T) ** 2) / N + 0.5 * lam * np.sum(d * d)
    assert r["L_pred"] == pytest.approx(obj, rel=1e-8)


def test_gptq_diagonal_hessian_is_rtn():
    """Orthogonal calibration columns (X = I): H is diagonal, U is diagonal, nothing propagates,
    and GPTQ gives O1's codes and scales."""
    d_out, d_in = 16, 96
    w = workloads.weight(91, 0, d_out, d_in)
    xb = _rne_bf16(np.eye(d_in, dtype=np.float32))
    for g, mode in ((32, SYM), (32, ASYM), (0, SYM)):
        r = gq.gptq(w, xb, g, mode)
        qw, sc, zr = oracle.pack(w, g, mode)
        assert np.array_equal(r["qweight"], qw) and np.array_equal(r["scales"], sc)
        if mode == ASYM:
            assert np.array_equal(r["zeros"], zr)


def test_gptq_two_columns_obs_closed_form():
    """Two columns in one group: after q0, the optimal-brain-surgeon update of the textbook,
    w1' = w1 + (w0 - q0) H01 / H11 (damped H), and q1 = the code of w1' with the group's scale."""
    rng = np.random.default_rng(92)
    d_out, N = 64, 40
    w = rng.normal(0, 0.02, size=(d_out, 2)).astype(np.float32)
    xb = _calib(92, N, 2)
    r = gq.gptq(w, xb, 32, SYM)
    x = _bits_f32(xb).astype(np.float64)
    H = 2.0 / N * (x.T @ x)
    H += 0.01 * np.mean(np.diag(H)) * np.eye(2)
    s = _bits_f32(r["scales"][:, 0]).astype(np.float64)
    c0 = r["codes"][:, 0].astype(np.float64)
    q0 = s * (c0 - 8.0)
    w1p = w[:, 1].astype(np.float64) + (w[:, 0] - q0) * H[0, 1] / H[1, 1]
    s32 = _bits_f32(r["scales"][:, 0])
    c1 = np.clip(np.rint(w1p.astype(np.float32) / s32 + np.float32(8.0)), 0, 15)
    assert np.array_equal(r["codes"][:, 1], c1.astype(np.uint8))
    # column 0 itself is O1's code of w0 with the scale of the pair
    c0_rtn = np.clip(np.rint(w[:, 0] / s32 + np.float32(8.0)), 0, 15)
    assert np.array_equal(r["codes"][:, 0], c0_rtn.astype(np.uint8))


@pytest.mark.parametrize("seed", [93, 94, 95])
def test_gptq_beats_rtn_on_the_layer_objective(seed):
    """On correlated calibration activations GPTQ's ||X (W - Q)^T|| is below RTN's (the point of
    the section), with every result on the same grid of codes and scales."""
    d_out, d_in, N = 32, 256, 128
    w = workloads.weight(seed, 0, d_out, d_in)
    xb = _calib(seed, N, d_in)
    x = _bits_f32(xb).astype(np.float64)
    for g, mode in ((32, SYM), (128, ASYM)):
        r = gq.gptq(w, xb, g, mode)
        qw, sc, zr = oracle.pack(w, g, mode)
        span = oracle.k_pad(d_in, g) // oracle.n_groups(d_in, g)
        codes_rtn = np.stack([qw & 0xF, qw >> 4], axis=-1).reshape(d_out, -1)
        q_rtn = _deq(codes_rtn, sc, zr, d_in, span)
        q_gptq = _deq(r["codes"], r["scales"], r["zeros"], d_in, span)
        e_rtn = np.sum((x @ (w - q_rtn).T) ** 2)
        e_gptq = np.sum((x @ (w - q_gptq).T) ** 2)
        assert e_gptq < 0.9 * e_rtn, (g, mode, e_gptq, e_rtn)


def test_gptq_dead_column():
    """A column that is zero in every calibration row: its weights become 0 (the zero code), H's
    diagonal entry becomes 1 before damping, and the loss identity still holds."""
    d_out, d_in, N = 16, 64, 80
    w = workloads.weight(96, 0, d_out, d_in)
    xb = _calib(96, N, d_in, dead=(5, 40))
    r = gq.gptq(w, xb, 32, SYM)
    assert np.all(r["codes"][:, [5, 40]] == 8)
    assert r["dead"][[5, 40]].all() and r["dead"].sum() == 2
    x = _bits_f32(xb).astype(np.float64)
    diag = 2.0 / N * np.sum(x * x, axis=0)
    diag[[5, 40]] = 1.0
    lam = 0.01 * np.mean(diag)
    w0 = w.astype(np.float64)
    w0[:, [5, 40]] = 0.0
    q = _deq(r["codes"], r["scales"], None, d_in, 32)
    d = w0 - q
    obj = np.sum((x @ d.T) ** 2) / N + 0.5 * lam * np.sum(d * d) + 0.5 * np.sum(d[:, [5, 40]] ** 2)
    assert r["L_pred"] == pytest.approx(obj, rel=1e-8)


@pytest.mark.parametrize("g,mode", [(32, SYM), (128, ASYM), (0, SYM), (64, ASYM)])
def test_gptq_exported_decision_values_round_to_its_result(g, mode):
    """O9's diagnostic exports are the values its decisions round: every code is
    clip(rint(v), 0, 15) of the exported pre-rounding value (nonzero scales), every stored scale
    is the bf16 rounding of the exported fp32 scale, every stored zero point the integer nearest
    the exported -min / s. A ragged last group (136 columns) is included."""
    d_out, d_in = 48, 136
    w = workloads.weight(77, g + mode, d_out, d_in)
    xb = _calib(9, 96, d_in)
    r = gq.gptq(w, xb, g, mode)
    kp = oracle.k_pad(d_in, g)
    span = kp // oracle.n_groups(d_in, g)
    s = oracle.bf16_to_f32(r["scales"])[:, np.arange(d_in) // span]
    nz = s != 0.0
    dec = np.clip(np.rint(r["v"]), 0, 15)
    assert np.array_equal(dec[nz], r["codes"][:, :d_in][nz])
    assert np.array_equal(oracle.f32_to_bf16(r["s_pre"]), r["scales"])
    if mode == ASYM:
        assert np.array_equal(np.rint(r["z_pre"]), oracle.bf16_to_f32(r["zeros"]))
