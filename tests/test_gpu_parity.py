"""GPU parity: every entry point of libw4.so, called through the C ABI (the thin Python binding),
against the CPU oracle on the same seeded inputs.

Bars: packing, codes, int8 activations, their scales and the W4A8 int32 accumulators are
bit-exact; floating outputs satisfy |y - y_ref| <= 2e-3 (1 + |y_ref|) on the fp32 output, and
the bf16 output of a call equals the round-to-nearest-even image of its fp32 output.
"""
import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import oracle
import workloads
from tests.gpu_helpers import (assert_bf16_is_rne_of_f32, assert_close, dev, dev_bf16,
                               forced_decode_path, host, host_bits)

pytestmark = pytest.mark.gpu

SYM, ASYM = w4.W4_SYM, w4.W4_ASYM
F32, BF16 = w4.W4_OUT_F32, w4.W4_OUT_BF16


def _announce(*what):
    print("[case]", *what, flush=True)


def gpu_pack(w, g, mode):
    qw, sc, zr = w4.w4_pack(dev(w), g, mode)
    return qw, sc, zr


def check_pack_bit_exact(w, g, mode, what):
    _announce("pack", what, w.shape, g, mode)
    qw_o, sc_o, zr_o = oracle.pack(w, g, mode)
    qw, sc, zr = gpu_pack(w, g, mode)
    assert np.array_equal(host(qw), qw_o), f"{what}: packed codes differ"
    assert np.array_equal(host_bits(sc), sc_o), f"{what}: scales differ"
    if mode == ASYM:
        assert np.array_equal(host_bits(zr), zr_o), f"{what}: zero points differ"
    else:
        assert zr is None
    return (qw_o, sc_o, zr_o), (qw, sc, zr)


def check_linear(entry, x_bits, packed_host, packed_dev, bias_bits, d_in, g, what,
                 ldx=None, ldy=None):
    """Run `entry` with fp32 and bf16 outputs; compare with oracle O4."""
    _announce(entry, what, x_bits.shape, d_in, g)
    qw_o, sc_o, zr_o = packed_host
    qw, sc, zr = packed_dev
    M = x_bits.shape[0]
    xb = x_bits
    if ldx is not None and ldx > x_bits.shape[1]:
        xb = np.zeros((M, ldx), dtype=np.uint16)
        xb[:, :x_bits.shape[1]] = x_bits
        xb[:, x_bits.shape[1]:] = 0x7FC0  # NaN beyond the row: must never be read
    x = dev_bf16(xb)
    b = dev_bf16(bias_bits) if bias_bits is not None else None
    fn = getattr(w4, entry)
    d_out = qw.shape[0]
    if ldy is not None:
        out32 = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
        y32 = fn(x, qw, sc, zr, b, d_in, g, F32, out=out32)[:, :d_out]
    else:
        y32 = fn(x, qw, sc, zr, b, d_in, g, F32)
    y16 = fn(x, qw, sc, zr, b, d_in, g, BF16)
    torch.cuda.synchronize()
    y_ref = oracle.w4a16(x_bits, qw_o, sc_o, zr_o, bias_bits, d_in, g)
    y32h = host(y32)
    assert_close(y32h, y_ref, what)
    assert_bf16_is_rne_of_f32(y16, y32h, what)
    return y32h, y_ref


# ------------------------------------------------------------------------------------------
# w4_pack
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("g", [32, 64, 128, 256, 0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_pack_ragged_shapes(g, mode):
    for d_out, d_in in ((1, 1), (3, 33), (17, 100), (64, 3600), (5, 1000)):
        w = workloads.weight(21, d_in + g + mode, d_out, d_in)
        workloads.add_weight_outliers(w, 21, 7, 0.02, 0.5)
        check_pack_bit_exact(w, g, mode, f"ragged {d_out}x{d_in}")


def test_pack_edge_values():
    rng = np.random.default_rng(22)
    rows = []
    rows.append(np.zeros(128, np.float32))                        # all-zero group
    rows.append(np.full(128, 0.25, np.float32))                   # constant group
    rows.append(np.full(128, -3.0, np.float32))                   # constant negative group
    rows.append((rng.normal(0, 1e-39, 128)).astype(np.float32))   # denormal weights
    rows.append((rng.normal(0, 1e30, 128)).astype(np.float32))    # huge weights
    rows.append(((np.arange(128) % 16 - 7.5) / 16).astype(np.float32))  # exact ties r/s + z
    rows.append(np.linspace(1.0, 1.01, 128).astype(np.float32))   # far-from-zero group (z < 0)
    sz = np.zeros(128, np.float32)
    sz[::2] = -0.0
    rows.append(sz)                                               # signed zeros
    w = np.stack(rows)
    for g in (32, 128, 0):
        for mode in (SYM, ASYM):
            check_pack_bit_exact(w, g, mode, "edge values")


def test_pack_configs_full_size():
    cases = [(workloads.C1, 0), (workloads.C2, 0), (workloads.C2, 1), (workloads.C3, 0),
             (workloads.C3, 3), (workloads.C4, 1), (workloads.C5, 0), (workloads.C5, 1)]
    for cfg, li in cases:
        lin = cfg.linears[li]
        w = workloads.linear_weight(cfg, li)
        check_pack_bit_exact(w, lin.group_size, lin.mode, f"{cfg.key}/{lin.name}")
    lin = workloads.C3.extra[0]
    w = workloads.linear_weight(workloads.C3, 4, lin=lin)
    check_pack_bit_exact(w, lin.group_size, lin.mode, "C3/pad3600")


# ------------------------------------------------------------------------------------------
# GPTQ (fp32 on the GPU) against O9 (fp64): the Hessian elementwise, the factor by its identity
# and elementwise, the column loop by its codes, its loss identity and the layer objective
# ------------------------------------------------------------------------------------------
import oracle.gptq as gq  # noqa: E402


def _gptq_calib(seed, N, d_in, dead=()):
    """bf16 calibration activations with correlated channels (latent factors plus noise), the
    listed columns zero in every row (the tests' own generator)."""
    rng = np.random.default_rng(seed)
    lat = rng.normal(size=(N, max(1, d_in // 4)))
    x = lat @ (rng.normal(size=(lat.shape[1], d_in)) / 2.0) + 0.3 * rng.normal(size=(N, d_in))
    x[:, list(dead)] = 0.0
    return workloads.to_bf16_bits(x.astype(np.float32))


def _deq(codes, sc_bits, zr_bits, d_in, span):
    G = np.arange(d_in) // span
    s = oracle.bf16_to_f32(sc_bits)[:, G].astype(np.float64)
    z = oracle.bf16_to_f32(zr_bits)[:, G].astype(np.float64) if zr_bits is not None else 8.0
    return s * (codes[:, :d_in].astype(np.float64) - z)


@pytest.mark.parametrize("N,d_in", [(1, 1), (37, 100), (256, 300), (2048, 3584)])
def test_gptq_hessian(N, d_in):
    _announce("gptq_hessian", N, d_in)
    xb = _gptq_calib(70 + N, N, d_in)
    ldx = d_in + 8 - d_in % 8 if d_in % 8 else d_in + 8
    xp = np.full((N, ldx), 0x7FC0, dtype=np.uint16)  # NaN past d_in: never read
    xp[:, :d_in] = xb
    h = host(w4.gptq_hessian(dev_bf16(xp), d_in))
    ref = gq.hessian(xb)
    x = np.abs(oracle.bf16_to_f32(xb).astype(np.float64))
    bound = 2.0 / N * (x.T @ x) * 1e-5 + 1e-30
    assert np.all(np.abs(h - ref) <= bound)


@pytest.mark.parametrize("d_in,dead", [(1, ()), (64, (3,)), (300, (0, 299)), (1024, (7, 500))])
def test_gptq_factor(d_in, dead):
    """U from the GPU factorization against O9's (fp64 inverse and Cholesky of the same damped
    matrix), and the identity U^T U (H + lambda I) = I."""
    _announce("gptq_factor", d_in, dead)
    N = 2 * d_in + 8
    xb = _gptq_calib(71 + d_in, N, d_in, dead)
    href = gq.hessian(xb)
    hd, _, lam, dref = gq.prepare(href, np.zeros((1, d_in)), 0.01)
    uref = gq.inverse_factor(hd)
    h = torch.from_numpy(href.astype(np.float32)).cuda()
    u, deadg = w4.gptq_factor(h, 0.01)
    torch.cuda.synchronize()
    u = host(u).astype(np.float64)
    assert np.array_equal(host(deadg).astype(bool), dref)
    assert np.all(np.tril(u, -1) == 0.0)
    assert np.max(np.abs(u - uref)) <= 2e-3 * np.max(np.abs(uref))
    eye = u.T @ u @ hd
    assert np.max(np.abs(eye - np.eye(d_in))) <= 2e-3


# A decision of the column loop rounds a value: a code rounds v = w / s + z, a scale rounds the
# fp32 max|w| / 7 (or (max - min) / 15) to bf16, a zero point rounds -min / s. The GPU propagates
# the errors in fp32 and O9 in fp64; their weights differ by far less than these margins, so the
# two can only decide differently where O9's value is this close to a rounding tie.
TIE_V = 1e-3        # |v - (k + 1/2)|, in units of the group's step
TIE_S = 2.0 ** -16  # |s32 - bf16 midpoint| / s32
TIE_Z = 1e-3        # |-min / s - (k + 1/2)|


def _check_first_divergence(codes, sc_bits, zr_bits, r, d_in, span, mode, what):
    """Row by row, the GPU's codes, scales and zero points equal O9's up to the row's first
    divergence, and that divergence is a near-tie of the decision that diverged (see TIE_*).
    Returns the number of rows that diverge at all."""
    ref_codes, ref_sc, ref_zr = r["codes"], r["scales"], r["zeros"]
    diverged = 0
    for row in range(codes.shape[0]):
        cm = np.flatnonzero(codes[row, :d_in] != ref_codes[row, :d_in])
        gm = np.flatnonzero((sc_bits[row] != ref_sc[row]) |
                            ((zr_bits[row] != ref_zr[row]) if mode == ASYM else False))
        c0 = int(cm[0]) if cm.size else None
        g0 = int(gm[0]) if gm.size else None
        if c0 is None and g0 is None:
            continue
        diverged += 1
        if g0 is not None and (c0 is None or g0 * span <= c0):
            if sc_bits[row, g0] != ref_sc[row, g0]:
                s32 = np.float32(r["s_pre"][row, g0])
                mid = ((np.array([s32]).view(np.uint32) & 0xFFFF0000) | 0x8000).view(np.float32)[0]
                assert abs(float(s32) - float(mid)) <= TIE_S * float(s32), \
                    f"{what}: row {row} group {g0}: scales differ away from a bf16 tie ({s32!r})"
            else:
                zp = float(r["z_pre"][row, g0])
                assert abs(zp - (np.floor(zp) + 0.5)) <= TIE_Z, \
                    f"{what}: row {row} group {g0}: zero points differ away from a tie ({zp!r})"
        else:
            v = float(r["v"][row, c0])
            assert abs(v - (np.floor(v) + 0.5)) <= TIE_V, \
                f"{what}: row {row} column {c0}: codes differ away from a rounding tie (v = {v!r})"
    return diverged


@pytest.mark.parametrize("g,mode", [(32, SYM), (128, ASYM), (0, SYM), (64, ASYM)])
def test_gptq_quantize_against_oracle(g, mode):
    """The column loop on the oracle's U. Each row's codes, scales and zero points equal O9's up
    to the row's first divergence, which must be a near-tie of the decision that diverged (fp32
    against fp64 error propagation); after it, the rounding apart propagates its own exact error,
    so the codes may differ: still at most 2% overall. Also the loss identity of the GPU's own
    result, and the layer objective within 1% of O9's. d_in = 1000: the last 32-column block holds
    8 columns."""
    d_out, d_in, N = 256, 1000, 512
    _announce("gptq_quantize", d_out, d_in, g, mode)
    w = workloads.weight(72, g + mode, d_out, d_in)
    xb = _gptq_calib(72 + g, N, d_in, dead=(17,))
    r = gq.gptq(w, xb, g, mode)
    u = torch.from_numpy(np.ascontiguousarray(r["U"], dtype=np.float32)).cuda()
    dead = torch.from_numpy(r["dead"].astype(np.uint8)).cuda()
    qw, sc, zr, row_loss = w4.gptq_quantize(torch.from_numpy(w.copy()).cuda(), u, dead, g, mode)
    torch.cuda.synchronize()
    qw, sc = host(qw), host_bits(sc)
    zr = host_bits(zr) if zr is not None else None
    codes = oracle.unpack(qw)
    kp = oracle.k_pad(d_in, g)
    span = kp // oracle.n_groups(d_in, g)
    n_div = _check_first_divergence(codes, sc, zr, r, d_in, span, mode, f"g{g} mode{mode}")
    print(f"[gptq] g{g} mode{mode}: {n_div} of {d_out} rows diverge", flush=True)
    assert np.mean(codes[:, :d_in] == r["codes"][:, :d_in]) >= 0.98
    x = oracle.bf16_to_f32(xb).astype(np.float64)
    w0 = r["w"]
    q = _deq(codes, sc, zr, d_in, span)
    assert np.all(q[:, 17] == 0.0)  # the dead column
    qp = _deq(codes, sc, zr, kp, span)  # pads decode to 0
    assert np.all(qp[:, d_in:] == 0.0)
    d = w0 - q
    obj = np.sum((x @ d.T) ** 2) / N + 0.5 * r["lam"] * np.sum(d * d)
    assert float(np.sum(host(row_loss).astype(np.float64))) == pytest.approx(obj, rel=2e-3)
    d_ref = w0 - _deq(r["codes"], r["scales"], r["zeros"], d_in, span)
    e_gpu, e_ref = np.sum((x @ d.T) ** 2), np.sum((x @ d_ref.T) ** 2)
    assert abs(e_gpu - e_ref) <= 0.01 * e_ref
    # every code decodes within the grid of its group's stored scale and zero
    assert codes.max() <= 15


@pytest.mark.parametrize("g,mode", [(32, SYM), (32, ASYM), (128, SYM)])
def test_gptq_ragged_last_block(g, mode):
    """d_in = 136: four full 32-column blocks, then 8 columns (and, at g = 128, a group of 8 real
    columns and 120 pads) that receive the error propagated from every column before them. Each
    row's decisions equal O9's up to a near-tie divergence (a wrong propagation into the ragged
    block would make rows diverge there away from any tie), and at most 5% of the rows diverge
    at all.""" 
    d_out, d_in, N = 512, 136, 256
    _announce("gptq ragged last block", d_out, d_in, g, mode)
    w = workloads.weight(75, g + mode, d_out, d_in)
    xb = _gptq_calib(75 + g, N, d_in)
    r = gq.gptq(w, xb, g, mode)
    u = torch.from_numpy(np.ascontiguousarray(r["U"], dtype=np.float32)).cuda()
    qw, sc, zr, _ = w4.gptq_quantize(torch.from_numpy(w.copy()).cuda(), u, None, g, mode)
    torch.cuda.synchronize()
    codes = oracle.unpack(host(qw))
    sc = host_bits(sc)
    zr = host_bits(zr) if zr is not None else None
    kp = oracle.k_pad(d_in, g)
    span = kp // oracle.n_groups(d_in, g)
    n_div = _check_first_divergence(codes, sc, zr, r, d_in, span, mode, "ragged last block")
    assert n_div <= d_out // 20, n_div  # near-ties are rare: most rows agree everywhere
    assert np.all(codes[:, d_in:kp] == r["codes"][:, d_in:kp])  # pads: the zero code


def test_gptq_strided_weights_without_dead_flags():
    """A weight with a row stride past d_in (junk there, never read or used) and no dead-column
    flags: the same codes and scales as the dense call."""
    d_out, d_in, ldw, N = 100, 200, 232, 160
    w = workloads.weight(74, 0, d_out, d_in)
    xb = _gptq_calib(74, N, d_in)
    h = w4.gptq_hessian(dev_bf16(xb))
    u, dead = w4.gptq_factor(h, 0.01)
    torch.cuda.synchronize()
    assert int(dead.sum()) == 0
    wp = np.full((d_out, ldw), 1e30, dtype=np.float32)
    wp[:, :d_in] = w
    a = w4.gptq_quantize(torch.from_numpy(wp).cuda(), u, None, 64, ASYM, d_in)
    b = w4.gptq_quantize(torch.from_numpy(w.copy()).cuda(), u, dead, 64, ASYM)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert np.array_equal(host(x.view(torch.int16) if x.dtype == torch.bfloat16 else x),
                              host(y.view(torch.int16) if y.dtype == torch.bfloat16 else y))


def test_gptq_end_to_end_c4_qkv():
    """The whole path on the GPU at the C4 q/k/v shape (4608 x 3584, g32 SYM, 2048 calibration
    tokens): GPTQ's layer objective is below RTN's, and its loss identity holds."""
    cfg = workloads.C4
    lin = cfg.linears[0]
    _announce("gptq end to end", lin.d_out, lin.d_in)
    w = workloads.linear_weight(cfg, 0)
    xb = _gptq_calib(73, 2048, lin.d_in)
    wd = torch.from_numpy(w).cuda()
    qw, sc, _, row_loss = w4.gptq(wd, dev_bf16(xb), 32, SYM)
    qr, sr, _ = w4.w4_pack(wd, 32, SYM)
    torch.cuda.synchronize()
    x = torch.from_numpy(oracle.bf16_to_f32(xb)).cuda().double()
    wt = wd.double()

    def deq(qwt, sct):
        c = oracle.unpack(host(qwt))[:, :lin.d_in].astype(np.float64)
        s = np.repeat(oracle.bf16_to_f32(host_bits(sct)).astype(np.float64), 32, axis=1)
        return torch.from_numpy(s[:, :lin.d_in] * (c - 8.0)).cuda()

    d_g, d_r = wt - deq(qw, sc), wt - deq(qr, sr)
    e_g = float(((x @ d_g.T) ** 2).sum())
    e_r = float(((x @ d_r.T) ** 2).sum())
    assert e_g < 0.8 * e_r, (e_g, e_r)
    diag = 2.0 / 2048 * (x * x).sum(dim=0)
    lam = 0.01 * float(diag.mean())
    obj = e_g / 2048 + 0.5 * lam * float((d_g * d_g).sum())
    assert float(row_loss.double().sum()) == pytest.approx(obj, rel=5e-3)


# ------------------------------------------------------------------------------------------
# w4_qat_repack
# ------------------------------------------------------------------------------------------
def check_qat(w_bits, d_in, what):
    """w4_qat_repack against the oracle's O8: codes, scales and the kept m, bit for bit."""
    _announce("w4_qat_repack", what, w_bits.shape, d_in)
    qw_o, sc_o, m_o = oracle.qat_repack(w_bits, d_in)
    qw, sc, m = w4.w4_qat_repack(dev_bf16(w_bits), d_in, want_m=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(m), m_o), f"{what}: kept m differs"
    assert np.array_equal(host(qw), qw_o), f"{what}: codes differ"
    assert np.array_equal(host_bits(sc), sc_o), f"{what}: scales differ"
    return qw_o, sc_o, m_o


def _qat_edge_groups():
    """Groups on the edges of the rule: all zero, one value 0.047 and one 0.078 of a level off,
    a peak at +8 steps, a peak at -8, subnormal steps, a coarser grid (all levels even), and a
    group whose peak is rounded (the least-squares step differs from max / 7)."""
    base = np.array([7, -3, 1, 0, 5, -6, 2, -1] * 4, dtype=np.float32)
    rows = [np.zeros(32, np.float32)]
    near, far, plus8, minus8 = base.copy(), base.copy(), base.copy(), base.copy()
    near[1], far[1], plus8[0], minus8[2] = -3.046875, -3.078125, 8.0, -8.0
    rows += [near, far, plus8, minus8]
    rows += [base * np.float32(2.0 ** -130), base * np.float32(3 * 2.0 ** -127)]
    rows += [np.array([6, -4, 2, 0, 4, -2, 2, -6] * 4, np.float32) * np.float32(0.375)]
    peak = base.copy()
    peak[0] = 7.03125
    rows.append(peak)
    edge = base.copy()
    edge[1] = -3.0625  # exactly 1/16 of a level off: still on the grid
    rows.append(edge)
    tiny = base.copy()
    tiny[3] = 2.0 ** -12  # a nonzero value far below a level: no divisor is ruled out early
    rows.append(tiny)
    return workloads.to_bf16_bits(np.concatenate(rows).reshape(1, -1))


def test_qat_repack_ragged_and_edges():
    for i, (d_out, d_in, ldw) in enumerate([(1, 1, 8), (3, 40, 48), (17, 100, 104), (64, 1000, 1000),
                                            (5, 3600, 3616), (300, 4100, 4104)]):
        w = workloads.qat_grid_weight(61, i, d_out, ldw, off_grid_frac=0.1)
        w[:, d_in:] = 0x7FC0  # NaN past d_in: never read
        check_qat(w, d_in, f"{d_out}x{d_in} ldw={ldw}")
    w = _qat_edge_groups()
    qw, sc, m = check_qat(w, w.shape[1], "edge groups")
    assert m[0].tolist() == [1, 7, 0, 0, 8, 7, 7, 3, 7, 7, 7]


def test_qat_repack_c4_full_size():
    """The C4 q/k/v, gate/up (the benchmarked shape) and down shapes (g32), 1% of the groups off
    the grid."""
    for li in (0, 1, 2):
        lin = workloads.C4.linears[li]
        w = workloads.qat_grid_weight(workloads.C4.seed, li, lin.d_out, lin.d_in, 0.01)
        _, _, m = check_qat(w, lin.d_in, f"C4/{lin.name}")
        assert 0 < np.count_nonzero(m == 0) < m.size // 50


def test_qat_repack_feeds_the_linear():
    """The repacked weight is a g32 symmetric pack: w4_gemv and w4_gemm on it against O4 on the
    oracle's repack."""
    d_out, d_in = 200, 1000
    w = workloads.qat_grid_weight(62, 0, d_out, d_in, 0.05)
    qw_o, sc_o, _ = oracle.qat_repack(w, d_in)
    qw, sc = w4.w4_qat_repack(dev_bf16(w), d_in)
    for M in (1, 5, 130):
        x = workloads.activations(62, M, M, d_in)
        check_linear("w4_gemv" if M <= 64 else "w4_gemm", x, (qw_o, sc_o, None), (qw, sc, None),
                     None, d_in, 32, f"repacked M={M}")


# ------------------------------------------------------------------------------------------
# act_quant_int8
# ------------------------------------------------------------------------------------------
def check_act_quant(x_bits, what, K=None):
    _announce("act_quant", what, x_bits.shape)
    K = x_bits.shape[1] if K is None else K
    q_o, s_o, qs_o = oracle.act_quant(x_bits, K)
    q, s, qs = w4.act_quant_int8(dev_bf16(x_bits), K)
    torch.cuda.synchronize()
    assert np.array_equal(host(q)[:, :K], q_o), f"{what}: int8 codes differ"
    assert np.array_equal(host(s).view(np.uint32), s_o.view(np.uint32)), f"{what}: s_x differs"
    assert np.array_equal(host(qs), qs_o), f"{what}: q_sum differs"


def test_act_quant_configs():
    for li, lin in enumerate(workloads.C5.linears):
        x = workloads.linear_x(workloads.C5, li, 1)
        check_act_quant(x, f"C5/{lin.name}")
    x = workloads.activations(23, 0, 64, 1000, 0.01, 20.0)
    x[5] = 0
    check_act_quant(x, "64 tokens, ragged K, one zero token")


@pytest.mark.parametrize("M,K", [(2048, 3584), (300, 8192), (256, 8200), (260, 18944),
                                 (256, 20480), (300, 20490), (255, 10001)])
def test_act_quant_many_tokens(M, K):
    """The row widths and token counts around each workgroup shape of the kernel (256 threads
    caching 4 or 10 chunks, 1024 threads), the prefill sizes among them; ragged K."""
    x = workloads.activations(24, M + K, M, K, 0.01, 20.0)
    x[M // 2] = 0
    xp = np.full((M, (K + 7) // 8 * 8), 0x7FC0, dtype=np.uint16)  # NaN past K: never read
    xp[:, :K] = x
    check_act_quant(xp, f"M={M} K={K}", K)


def test_act_quant_all_bf16_patterns():
    """Every finite bf16 value, quantized against several fixed maxima."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f32(allbits)
    finite = np.isfinite(vals)
    rows = []
    for top in (1.0, 5.0, 127.0, 3.0e38, 1e-30, 2.0 ** -126):
        keep = allbits[finite & (np.abs(vals) <= top)]
        top_bits = workloads.to_bf16_bits(np.array([top], np.float32))
        rows.append(np.concatenate([top_bits, keep]))
    K = (max(len(r) for r in rows) + 7) // 8 * 8
    x = np.zeros((len(rows), K), dtype=np.uint16)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    check_act_quant(x, "all finite bf16 patterns")


# ------------------------------------------------------------------------------------------
# w4_gemv (decode, M <= 64) and w4_gemm (prefill)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
def test_linear_c1_tiny(entry):
    cfg = workloads.C1
    lin = cfg.linears[0]
    w = workloads.linear_weight(cfg, 0)
    ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, "C1")
    for M in cfg.tokens:
        x = workloads.linear_x(cfg, 0, M)
        check_linear(entry, x, ph, pd, None, lin.d_in, lin.group_size, f"C1 M={M}")
    b = workloads.bias(cfg.seed, 0, lin.d_out)
    x = workloads.linear_x(cfg, 0, 4)
    check_linear(entry, x, ph, pd, b, lin.d_in, lin.group_size, "C1 M=4 with bias")


@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
@pytest.mark.parametrize("g", [32, 64, 128, 256, 0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_linear_ragged(entry, g, mode):
    """Shapes that span several tiles with ragged tails in every dimension."""
    shapes = [(1, 1, 1), (3, 130, 100), (17, 257, 1000), (64, 200, 3600)]
    if entry == "w4_gemm":
        shapes += [(130, 131, 300), (257, 96, 64)]
    for M, d_out, d_in in shapes:
        w = workloads.weight(24, M + d_out + d_in + g, d_out, d_in)
        ph, pd = check_pack_bit_exact(w, g, mode, "ragged")
        x = workloads.activations(24, g + mode, M, d_in)
        b = workloads.bias(24, 1, d_out)
        ldx = (d_in + 7) // 8 * 8 + 8
        check_linear(entry, x, ph, pd, b, d_in, g, f"M={M} {d_out}x{d_in}", ldx=ldx,
                     ldy=d_out + 3)


@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
def test_linear_basis_probes_exact(entry):
    """x = e_k gives y[j] = w_hat[j][k] exactly in the fp32 output: pins nibble order, group
    index, scale and zero point of every probed column."""
    d_out, d_in = 96, 300
    w = workloads.weight(25, 0, d_out, d_in)
    for g, mode in ((32, SYM), (64, ASYM), (128, ASYM), (0, SYM)):
        ph, pd = check_pack_bit_exact(w, g, mode, "probe")
        wh = oracle.dequant(ph[0], ph[1], ph[2], d_in, g)
        cols = [0, 1, 2, 7, 8, 31, 32, 33, 63, 64, 127, 128, 255, 256, 299]
        x = np.zeros((len(cols), (d_in + 7) // 8 * 8), dtype=np.uint16)
        for i, k in enumerate(cols):
            x[i, k] = 0x3F80
        for chunk in (slice(0, 4), slice(0, len(cols))):
            xs = x[chunk]
            if entry == "w4_gemv" and xs.shape[0] > 64:
                continue
            y = getattr(w4, entry)(dev_bf16(xs), *pd, None, d_in, g, F32)
            got = host(y).astype(np.float64)
            want = wh[:, [cols[i] for i in range(len(cols))][chunk]].T
            assert np.array_equal(got, want), f"{entry} basis probe g={g} mode={mode}"


@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
def test_linear_padding_with_junk_activations(entry):
    """The d_in = 3600 layer, run with d_in := k_pad = 3712 on activations whose 112 pad columns
    hold 1e3: the result must still match the d_in = 3600 oracle, which is only possible if the
    kernel multiplies the pad columns by exact zeros."""
    cfg = workloads.C3
    lin = cfg.extra[0]
    w = workloads.linear_weight(cfg, 4, lin=lin)
    ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, "C3/pad3600")
    k_pad = oracle.k_pad(lin.d_in, lin.group_size)
    for M in cfg.tokens:
        x = workloads.linear_x(cfg, 4, M, lin=lin)
        check_linear(entry, x, ph, pd, None, lin.d_in, lin.group_size, f"pad3600 M={M}")
        xj = np.zeros((M, k_pad), dtype=np.uint16)
        xj[:, :lin.d_in] = x
        xj[:, lin.d_in:] = workloads.to_bf16_bits(np.array([1000.0], np.float32))[0]
        _announce(entry, "junk pads", M)
        y = getattr(w4, entry)(dev_bf16(xj), *pd, None, k_pad, lin.group_size, F32)
        y_ref = oracle.w4a16(x, ph[0], ph[1], ph[2], None, lin.d_in, lin.group_size)
        assert_close(host(y), y_ref, f"junk pads M={M}")


def test_gemv_c2_full_size():
    cfg = workloads.C2
    for li, lin in enumerate(cfg.linears):
        w = workloads.linear_weight(cfg, li)
        ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, f"C2/{lin.name}")
        x = workloads.linear_x(cfg, li, 1)
        check_linear("w4_gemv", x, ph, pd, None, lin.d_in, lin.group_size, f"C2/{lin.name}")


def test_gemv_c3_layers():
    """Each C3 shape (asymmetric g128) at M = 1, 8, 16, for the first and the last layer."""
    cfg = workloads.C3
    for layer in (0, cfg.repeat_layers - 1):
        for li, lin in enumerate(cfg.linears):
            w = workloads.linear_weight(cfg, li, layer=layer)
            ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode,
                                          f"C3/L{layer}/{lin.name}")
            for M in cfg.tokens:
                x = workloads.linear_x(cfg, li, M, layer=layer)
                check_linear("w4_gemv", x, ph, pd, None, lin.d_in, lin.group_size,
                             f"C3/L{layer}/{lin.name} M={M}")


def test_gemv_c3_gate_up_two_and_three_tokens():
    """The C3 gate/up shape at M = 2 and 3, which the library gives to the int8 digit kernel
    (tall matrix of short rows), through w4_gemv and w4_gemv_ws."""
    cfg = workloads.C3
    li = [lin.name for lin in cfg.linears].index("gate_up")
    lin = cfg.linears[li]
    w = workloads.linear_weight(cfg, li)
    ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, "C3/gate_up")
    for M in (2, 3):
        x = workloads.linear_x(cfg, li, M)
        check_linear("w4_gemv", x, ph, pd, None, lin.d_in, lin.group_size, f"C3/gate_up M={M}")
        check_linear("w4_gemv_ws", x, ph, pd, None, lin.d_in, lin.group_size,
                     f"C3/gate_up ws M={M}")


def test_gemv_all_token_counts():
    d_out, d_in, g = 200, 520, 64
    w = workloads.weight(26, 0, d_out, d_in)
    ph, pd = check_pack_bit_exact(w, g, ASYM, "M sweep")
    for M in (1, 2, 3, 4, 5, 7, 8, 9, 16, 31, 33, 63, 64):
        x = workloads.activations(26, M, M, d_in)
        check_linear("w4_gemv", x, ph, pd, None, d_in, g, f"M={M}")


def _stratified_tokens(rng, M, tile=128):
    """The first and last token, and one random token of every `tile` consecutive tokens: every
    token tile of the GEMMs (128 or 256 tokens) is compared with the oracle."""
    picks = [t0 + int(rng.integers(min(tile, M - t0))) for t0 in range(0, M, tile)]
    return np.unique(np.array([0, M - 1] + picks))


def _stratified_rows(rng, d_out, total, tile=128):
    """One random row of every `tile` consecutive output rows (every row tile of the GEMMs), and
    random further rows up to `total` (all rows when d_out <= total)."""
    if d_out <= total:
        return np.arange(d_out)
    picks = np.array([r0 + int(rng.integers(min(tile, d_out - r0))) for r0 in range(0, d_out, tile)])
    extra = rng.choice(d_out, size=max(0, total - picks.size), replace=False)
    return np.unique(np.concatenate([picks, extra]))


def test_gemm_c4_sampled_full_size():
    """C4 at its full size (M = 2048): the whole output is computed; one token of every 128-token
    tile and one row of every 128-row tile (plus random further rows, 4096 per token) are
    compared with the oracle, computed point by point."""
    cfg = workloads.C4
    rng = np.random.default_rng(404)
    for li, lin in enumerate(cfg.linears):
        w = workloads.linear_weight(cfg, li)
        ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, f"C4/{lin.name}")
        del w
        M = cfg.tokens[0]
        x = workloads.linear_x(cfg, li, M)
        _announce("w4_gemm", f"C4/{lin.name}", M)
        xd = dev_bf16(x)
        y32 = w4.w4_gemm(xd, *pd, None, lin.d_in, lin.group_size, F32)
        y16 = w4.w4_gemm(xd, *pd, None, lin.d_in, lin.group_size, BF16)
        torch.cuda.synchronize()
        y32h = host(y32)
        assert np.all(np.isfinite(y32h))
        assert_bf16_is_rne_of_f32(y16, y32h, f"C4/{lin.name}")
        for t in _stratified_tokens(rng, M):
            rows = _stratified_rows(rng, lin.d_out, 4096)
            ref = oracle.w4a16_points(x, ph[0], ph[1], ph[2], None, lin.d_in, lin.group_size,
                                      np.full(rows.size, t), rows)
            assert_close(y32h[t, rows], ref, f"C4/{lin.name} token {t}")


def test_gemm_scale_windows():
    """The GEMM's scale-window path (symmetric 32-column groups, n_groups % 8 == 0, 16-byte
    aligned scales): a row count that leaves the last wave's 64 rows mostly empty, a window count
    that is not a multiple of the ring, two token tiles; and the same weights with the scales at
    an address 2 bytes past alignment, which takes the general path."""
    M, d_out, d_in, g = 300, 200, 1280, 32
    w = workloads.weight(71, 0, d_out, d_in)
    ph, pd = check_pack_bit_exact(w, g, SYM, "scale windows")
    x = workloads.activations(71, 0, M, d_in)
    check_linear("w4_gemm", x, ph, pd, None, d_in, g, "scale windows")
    # scales 2 bytes past a 16-byte boundary
    ng = ph[1].shape[1]
    buf = torch.empty(d_out * ng + 8, dtype=torch.bfloat16, device="cuda")
    sc_off = buf[1:1 + d_out * ng].view(d_out, ng)
    sc_off.copy_(pd[1])
    assert sc_off.data_ptr() % 16 == 2
    check_linear("w4_gemm", x, ph, (pd[0], sc_off, None), None, d_in, g, "scale windows off16")


def test_gemm_matches_gemv_small_m():
    d_out, d_in, g = 300, 1024, 32
    w = workloads.weight(27, 0, d_out, d_in)
    _, pd = check_pack_bit_exact(w, g, SYM, "gemm vs gemv")
    x = dev_bf16(workloads.activations(27, 0, 8, d_in))
    a = host(w4.w4_gemv(x, *pd, None, d_in, g, F32))
    b = host(w4.w4_gemm(x, *pd, None, d_in, g, F32))
    assert_close(a, b.astype(np.float64), "gemm vs gemv")


@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
@pytest.mark.parametrize("g", [128, 64, 32])
def test_linear_zero_points_beyond_pack(entry, g):
    """Zero points that w4_pack never writes (non-integers, beyond the code range, negative,
    large) still follow w = s (c - z): every decode kernel (forced where one token would pick
    another) and the GEMM against the oracle, which takes z as given. Groups of 128, and of 64
    and 32 (several groups per 128-column chunk in the few-token kernel)."""
    d_out, d_in = 300, 1000
    w = workloads.weight(29, 0, d_out, d_in)
    ph, pd = check_pack_bit_exact(w, g, ASYM, "zero points beyond pack")
    rng = np.random.default_rng(29)
    zf = rng.choice(np.array([0.5, 7.25, -3.0, 20.0, 300.0, -1000.0, 7.0, 15.0], np.float32),
                    size=ph[2].shape)
    zb = workloads.to_bf16_bits(zf)
    ph2 = (ph[0], ph[1], zb)
    pd2 = (pd[0], pd[1], dev_bf16(zb))
    b = workloads.bias(29, 1, d_out)
    paths = (None, "i8", "stream") if entry == "w4_gemv" and g == 128 else (None,)
    for path in paths:
        with forced_decode_path(path):
            for M in (1, 2, 5, 16):
                x = workloads.activations(29, M, M, d_in)
                check_linear(entry, x, ph2, pd2, b, d_in, g, f"z beyond pack M={M} path={path}")


def _glu_bound(x_bits, ph, bias_bits, d_in, g):
    """Tolerance of h = SiLU(g) u, derived from the linear tolerance tau(v) = 2e-3 (1 + |v|) on g
    and u: |dh| <= max|SiLU'| tau(g) (|u| + tau(u)) + (|SiLU(g)| + max|SiLU'| tau(g)) tau(u),
    max|SiLU'| < 1.1, plus 2^-20 |h| for the fp32 epilogue (exp, division, products)."""
    y = oracle.w4a16(x_bits, ph[0], ph[1], ph[2], bias_bits, d_in, g)
    H = y.shape[1] // 2
    gr, ur = y[:, :H], y[:, H:]
    h_ref = oracle.silu_mul(gr, ur)
    tg, tu = 2e-3 * (1 + np.abs(gr)), 2e-3 * (1 + np.abs(ur))
    s = np.abs(oracle.silu_mul(gr, np.ones_like(gr)))
    bound = 1.1 * tg * (np.abs(ur) + tu) + (s + 1.1 * tg) * tu + 2.0 ** -20 * np.abs(h_ref)
    return h_ref, bound


def check_glu(w, x_bits, bias_bits, g, mode, what, ldx=None):
    _announce("w4_gemv_glu", what, w.shape, x_bits.shape, g, mode)
    ph, pd = check_pack_bit_exact(w, g, mode, what)
    d_in = w.shape[1]
    M = x_bits.shape[0]
    xb = x_bits
    if ldx is not None and ldx > d_in:
        xb = np.full((M, ldx), 0x7FC0, dtype=np.uint16)  # NaN past d_in: never read
        xb[:, :d_in] = x_bits
    x = dev_bf16(xb)
    b = dev_bf16(bias_bits) if bias_bits is not None else None
    h32 = w4.w4_gemv_glu(x, *pd, b, d_in, g, F32)
    h16 = w4.w4_gemv_glu(x, *pd, b, d_in, g, BF16)
    torch.cuda.synchronize()
    h_ref, bound = _glu_bound(x_bits, ph, bias_bits, d_in, g)
    h = host(h32).astype(np.float64)
    bad = np.abs(h - h_ref) > bound
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside the derived bound"
    assert_bf16_is_rne_of_f32(h16, host(h32), what)


def test_gemv_glu_c2_gate_up_full_size():
    """The C2 gate/up weight (37888 x 3584, g128 SYM, outliers) as a fused gate/up: h = SiLU of
    rows [0, 18944) times rows [18944, 37888)."""
    cfg = workloads.C2
    gu = cfg.linears[0]
    w = workloads.linear_weight(cfg, 0)
    x = workloads.linear_x(cfg, 0, 1)
    check_glu(w, x, None, gu.group_size, gu.mode, "C2 gate/up")


@pytest.mark.parametrize("g", [128, 256, 0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_gemv_glu_ragged(g, mode):
    """1-4 tokens, ragged d_ff and d_in (NaN past d_in), with and without bias."""
    for M, d_ff, d_in in ((1, 1, 100), (2, 37, 1000), (3, 130, 3600), (4, 300, 4100)):
        w = workloads.weight(43, M + d_ff + g, 2 * d_ff, d_in)
        x = workloads.activations(43, g + mode, M, d_in)
        b = workloads.bias(43, 1, 2 * d_ff) if M % 2 else None
        if oracle.k_pad(d_in, g) % 128:  # one group per row, rows not whole 128-column groups
            _, pd = check_pack_bit_exact(w, g, mode, "glu unsupported")
            xp = np.zeros((M, (d_in + 7) // 8 * 8), dtype=np.uint16)
            xp[:, :d_in] = x
            with pytest.raises(w4.W4Error) as err:
                w4.w4_gemv_glu(dev_bf16(xp), *pd, None, d_in, g, F32)
            assert err.value.status == 6  # W4_ERR_UNSUPPORTED, the documented limit
            continue
        check_glu(w, x, b, g, mode, f"M={M} d_ff={d_ff} d_in={d_in}",
                  ldx=(d_in + 7) // 8 * 8 + 8)


def test_linear_maximum_reduction_length():
    """d_in = 65536, the decode entry points' limit (and far past every config): the decode
    paths (one token, few tokens, both group modes), the gate epilogue, W4A8 (two calls and
    fused; |acc| reaches 65536 * 8 * 127 = 66.6 M, well inside int32) and the GEMM."""
    d_in, d_out = 65536, 48
    for g, mode in ((128, ASYM), (32, SYM)):
        w = workloads.weight(47, g, d_out, d_in)
        ph, pd = check_pack_bit_exact(w, g, mode, f"d_in=65536 g={g}")
        for M in (1, 5, 64):
            x = workloads.activations(47, M, M, d_in)
            check_linear("w4_gemv", x, ph, pd, None, d_in, g, f"d_in=65536 M={M} g={g}")
        x = workloads.activations(47, 99, 130, d_in)
        check_linear("w4_gemm", x, ph, pd, None, d_in, g, f"d_in=65536 M=130 g={g}")
    w = workloads.weight(48, 0, 2 * d_out, 16384)
    check_glu(w, workloads.activations(48, 1, 1, 16384), None, 128, ASYM, "glu d_in=16384")
    w = workloads.weight(49, 0, d_out, d_in)
    x = workloads.activations(49, 3, 3, d_in, 0.01, 20.0)
    check_w4a8(w, x, workloads.bias(49, 1, d_out), "w4a8 d_in=65536")


@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
def test_linear_deterministic(entry):
    d_out, d_in, g = 1000, 3584, 128
    w = workloads.weight(28, 0, d_out, d_in)
    _, pd = check_pack_bit_exact(w, g, ASYM, "determinism")
    x = dev_bf16(workloads.activations(28, 0, 16, d_in))
    fn = getattr(w4, entry)
    first = host(fn(x, *pd, None, d_in, g, F32))
    for _ in range(3):
        again = host(fn(x, *pd, None, d_in, g, F32))
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))


# ------------------------------------------------------------------------------------------
# the int8 matrix-core decode kernel, forced onto every shape it supports (by default it serves
# one token on wide matrices only)
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("g", [128, 256, 0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
@forced_decode_path("i8")
def test_gemv_int8_kernel_ragged(g, mode):
    """One to four tokens, ragged d_out and d_in (NaN past d_in in x), bias, strided x and y."""
    shapes = [(1, 1, 100), (3, 130, 100), (4, 257, 1000), (2, 200, 3600), (1, 700, 4100),
              (1, 33, 18944)]
    for M, d_out, d_in in shapes:
        w = workloads.weight(29, M + d_out + d_in + g, d_out, d_in)
        ph, pd = check_pack_bit_exact(w, g, mode, "int8 kernel")
        x = workloads.activations(29, g + mode, M, d_in)
        b = workloads.bias(29, 1, d_out)
        ldx = (d_in + 7) // 8 * 8 + 16
        check_linear("w4_gemv", x, ph, pd, b, d_in, g, f"int8 kernel M={M} {d_out}x{d_in}",
                     ldx=ldx, ldy=d_out + 5)


@forced_decode_path("i8")
def test_gemv_int8_kernel_junk_pads_and_determinism():
    """Pad columns of the d_in = 3600 layer run as real columns holding 1e3 must add exact
    zeros; repeated calls are bit-identical."""
    cfg = workloads.C3
    lin = cfg.extra[0]
    w = workloads.linear_weight(cfg, 4, lin=lin)
    ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, "int8 kernel pad3600")
    k_pad = oracle.k_pad(lin.d_in, lin.group_size)
    for M in (1, 4):
        x = workloads.linear_x(cfg, 4, M, lin=lin)
        xj = np.zeros((M, k_pad), dtype=np.uint16)
        xj[:, :lin.d_in] = x
        xj[:, lin.d_in:] = workloads.to_bf16_bits(np.array([1000.0], np.float32))[0]
        _announce("int8 kernel junk pads", M)
        xd = dev_bf16(xj)
        y = host(w4.w4_gemv(xd, *pd, None, k_pad, lin.group_size, F32))
        y_ref = oracle.w4a16(x, ph[0], ph[1], ph[2], None, lin.d_in, lin.group_size)
        assert_close(y, y_ref, f"int8 kernel junk pads M={M}")
        for _ in range(2):
            again = host(w4.w4_gemv(xd, *pd, None, k_pad, lin.group_size, F32))
            assert np.array_equal(y.view(np.uint32), again.view(np.uint32))


# ------------------------------------------------------------------------------------------
# w4a8_gemv
# ------------------------------------------------------------------------------------------
def check_w4a8(w, x_bits, bias_bits, what):
    _announce("w4a8", what, w.shape, x_bits.shape)
    d_out, d_in = w.shape
    ph, pd = check_pack_bit_exact(w, 0, SYM, what)
    q_o, s_o, _ = oracle.act_quant(x_bits, d_in)
    acc_o, y_ref, nov = oracle.w4a8(q_o, s_o, ph[0], ph[1][:, 0], bias_bits, d_in)
    assert nov == 0
    xpad = np.zeros((x_bits.shape[0], (d_in + 7) // 8 * 8), dtype=np.uint16)
    xpad[:, :d_in] = x_bits
    q, s, _ = w4.act_quant_int8(dev_bf16(xpad), d_in)
    b = dev_bf16(bias_bits) if bias_bits is not None else None
    y32, acc = w4.w4a8_gemv(q, s, pd[0], pd[1], b, d_in, F32, want_acc=True)
    y16 = w4.w4a8_gemv(q, s, pd[0], pd[1], b, d_in, BF16)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), acc_o), f"{what}: int32 accumulators differ"
    y32h = host(y32)
    assert_close(y32h, y_ref, what)
    assert_bf16_is_rne_of_f32(y16, y32h, what)
    check_w4a8_gemm(q_o, s_o, ph, pd, bias_bits, d_in, acc_o, y_ref, what)
    # the same linear with the quantization folded in (w4a8_linear), on a strided x whose columns
    # past d_in hold NaN: the token scales and the accumulators are those of the oracle's O5 -> O6
    _announce("w4a8_linear", what, w.shape, x_bits.shape)
    ldx = (d_in + 7) // 8 * 8 + 8
    xj = np.full((x_bits.shape[0], ldx), 0x7FC0, dtype=np.uint16)
    xj[:, :d_in] = x_bits
    xd = dev_bf16(xj)
    if oracle.k_pad(d_in, 0) > 32768:  # past the fused kernel's activation stage (documented)
        with pytest.raises(w4.W4Error) as err:
            w4.w4a8_linear(xd, pd[0], pd[1], b, d_in, F32)
        assert err.value.status == 6  # W4_ERR_UNSUPPORTED
        return
    y32f, accf, sxf = w4.w4a8_linear(xd, pd[0], pd[1], b, d_in, F32, want_acc=True,
                                     want_scales=True)
    y16f = w4.w4a8_linear(xd, pd[0], pd[1], b, d_in, BF16)
    torch.cuda.synchronize()
    assert np.array_equal(host(sxf).view(np.uint32), s_o.astype(np.float32).view(np.uint32)), \
        f"{what}: fused token scales differ"
    assert np.array_equal(host(accf), acc_o), f"{what}: fused int32 accumulators differ"
    y32fh = host(y32f)
    assert_close(y32fh, y_ref, what + " (fused)")
    assert_bf16_is_rne_of_f32(y16f, y32fh, what + " (fused)")


def _q_with_junk_pads(q_o, d_in, ldq, seed):
    """Device int8 [M][ldq]: the codes in the first d_in columns, random bytes (any of -128..127,
    as act_quant_int8 leaves them unset) after them."""
    M = q_o.shape[0]
    rng = np.random.default_rng(seed)
    qh = rng.integers(-128, 128, size=(M, ldq), dtype=np.int64).astype(np.int8)
    qh[:, :d_in] = q_o[:, :d_in]
    return torch.from_numpy(qh).cuda()


def check_w4a8_gemm(q_o, s_o, ph, pd, bias_bits, d_in, acc_o, y_ref, what, ldq=None,
                    ldy=None):
    """w4a8_gemm against the oracle's O6: int32 accumulators bit for bit, y within the bar, bf16
    the RNE image of fp32; junk past d_in in q, optional strided q and y."""
    _announce("w4a8_gemm", what, q_o.shape, d_in)
    M = q_o.shape[0]
    d_out = pd[0].shape[0]
    ldq = ldq or (d_in + 15) // 16 * 16
    q = _q_with_junk_pads(q_o, d_in, ldq, M + d_in)
    s = torch.from_numpy(np.ascontiguousarray(s_o, dtype=np.float32)).cuda()
    b = dev_bf16(bias_bits) if bias_bits is not None else None
    if ldy is not None:
        out = torch.full((M, ldy), float("nan"), dtype=torch.float32, device="cuda")
        y32, acc = w4.w4a8_gemm(q, s, pd[0], pd[1], b, d_in, F32, want_acc=True, out=out)
        y32 = y32[:, :d_out]
    else:
        y32, acc = w4.w4a8_gemm(q, s, pd[0], pd[1], b, d_in, F32, want_acc=True)
    y16 = w4.w4a8_gemm(q, s, pd[0], pd[1], b, d_in, BF16)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), acc_o), f"{what}: w4a8_gemm int32 accumulators differ"
    y32h = host(y32)
    assert_close(y32h, y_ref, what + " (w4a8_gemm)")
    assert_bf16_is_rne_of_f32(y16, y32h, what + " (w4a8_gemm)")


def test_w4a8_gemm_ragged_token_counts():
    """Token counts across and between the 128-token tiles, ragged d_out and d_in (junk past d_in
    in q), strided q and y, bias on and off."""
    shapes = [(65, 1, 1), (127, 130, 90), (128, 128, 128), (129, 257, 1000), (300, 70, 3600),
              (257, 1000, 4100), (200, 64, 18944), (1000, 33, 161)]
    for i, (M, d_out, d_in) in enumerate(shapes):
        w = workloads.weight(51, M + d_in, d_out, d_in)
        ph, pd = check_pack_bit_exact(w, 0, SYM, f"w4a8_gemm {d_out}x{d_in}")
        x = workloads.activations(51, M, M, d_in, 0.01, 20.0)
        b = workloads.bias(51, 2, d_out) if i % 2 else None
        q_o, s_o, _ = oracle.act_quant(x, d_in)
        acc_o, y_ref, nov = oracle.w4a8(q_o, s_o, ph[0], ph[1][:, 0], b, d_in)
        assert nov == 0
        ldq = (d_in + 15) // 16 * 16 + 16 * (i % 3)
        check_w4a8_gemm(q_o, s_o, ph, pd, b, d_in, acc_o, y_ref,
                        f"M={M} {d_out}x{d_in}", ldq=ldq, ldy=d_out + 3 * (i % 2))


def test_w4a8_gemm_c4_sampled_full_size():
    """The C4 prefill shapes (M = 2048) with per-row symmetric packs: the whole output is
    computed, and every row of one token of every 128-token tile (and the tokens around the first
    tile boundary) is compared with the oracle's O6 (each token's accumulators depend on that
    token's codes only)."""
    cfg = workloads.C4
    rng = np.random.default_rng(405)
    for li, lin in enumerate(cfg.linears):
        w = workloads.linear_weight(cfg, li)
        ph, pd = check_pack_bit_exact(w, 0, SYM, f"C4/{lin.name} per-row")
        del w
        M = cfg.tokens[0]
        x = workloads.linear_x(cfg, li, M)
        q_o, s_o, _ = oracle.act_quant(x, lin.d_in)
        _announce("w4a8_gemm", f"C4/{lin.name}", M)
        q = _q_with_junk_pads(q_o, lin.d_in, (lin.d_in + 15) // 16 * 16, li)
        s = torch.from_numpy(s_o.astype(np.float32)).cuda()
        y32, acc = w4.w4a8_gemm(q, s, pd[0], pd[1], None, lin.d_in, F32, want_acc=True)
        y16 = w4.w4a8_gemm(q, s, pd[0], pd[1], None, lin.d_in, BF16)
        torch.cuda.synchronize()
        y32h, acch = host(y32), host(acc)
        assert_bf16_is_rne_of_f32(y16, y32h, f"C4/{lin.name}")
        toks = np.unique(np.concatenate([[127, 128], _stratified_tokens(rng, M)]))
        acc_o, y_ref, nov = oracle.w4a8(q_o[toks], s_o[toks], ph[0], ph[1][:, 0], None,
                                        lin.d_in)
        assert nov == 0
        assert np.array_equal(acch[toks], acc_o), f"C4/{lin.name}: accumulators differ"
        assert_close(y32h[toks], y_ref, f"C4/{lin.name} sampled tokens")


def test_w4a8_gemm_int32_extremes():
    """d_in = W4_MAX_W4A8_D_IN = 2^20 with the extreme codes and activations: level 7 or -8 times
    +-127 in every column (|acc| up to 8 * 127 * 2^20 = 1,065,353,216), checked against the
    closed forms and the oracle's O6, exactly."""
    d_in = 1 << 20
    _announce("w4a8_gemm int32 extremes", d_in)
    codes = np.empty((4, d_in), dtype=np.uint8)
    codes[0], codes[1], codes[2] = 15, 0, 8
    codes[3] = np.arange(d_in) % 16
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    q_o = np.empty((3, d_in), dtype=np.int8)
    q_o[0], q_o[1] = 127, -127
    q_o[2] = np.where(np.arange(d_in) % 2 == 0, 127, -127)
    s_o = np.array([1.0, 0.5, 0.25], dtype=np.float32)
    sw_bits = workloads.to_bf16_bits(np.array([1.0, 2.0, 1.0, 0.5], np.float32))
    acc_o, y_ref, nov = oracle.w4a8(q_o, s_o, packed, sw_bits, None, d_in)
    assert nov == 0
    L = 127 * d_in
    assert acc_o[:2, :3].tolist() == [[7 * L, -8 * L, 0], [-7 * L, 8 * L, 0]]
    assert acc_o[0, 3] == -8 * 127 * (d_in // 16) and acc_o[2, :3].tolist() == [0, 0, 0]
    ph = (packed, sw_bits[:, None], None)
    pd = (torch.from_numpy(packed).cuda(), dev_bf16(sw_bits[:, None].copy()), None)
    check_w4a8_gemm(q_o, s_o, ph, pd, None, d_in, acc_o, y_ref, "int32 extremes")


def test_w4a8_c5_full_size():
    cfg = workloads.C5
    for li, lin in enumerate(cfg.linears):
        w = workloads.linear_weight(cfg, li)
        x = workloads.linear_x(cfg, li, 1)
        b = workloads.linear_bias(cfg, li)
        check_w4a8(w, x, b, f"C5/{lin.name}")


def test_w4a8_c5_full_size_few_tokens():
    """Both C5 shapes at 16 and 33 tokens (one and three 16-token tiles, the last partial), which
    the library gives to the int8 matrix-core kernel: int32 accumulators bit for bit."""
    cfg = workloads.C5
    for li, lin in enumerate(cfg.linears):
        w = workloads.linear_weight(cfg, li)
        b = workloads.linear_bias(cfg, li)
        for M in (16, 33):
            x = workloads.linear_x(cfg, li, M)
            check_w4a8(w, x, b, f"C5/{lin.name} M={M}")


def test_w4a8_ragged_and_token_counts():
    for M, d_out, d_in in ((1, 1, 1), (3, 70, 90), (5, 257, 1000), (64, 130, 3600),
                           (16, 64, 18944)):
        w = workloads.weight(29, M + d_in, d_out, d_in)
        x = workloads.activations(29, M, M, d_in, 0.01, 20.0)
        b = workloads.bias(29, 2, d_out)
        check_w4a8(w, x, b if M % 2 else None, f"M={M} {d_out}x{d_in}")


def test_w4a8_gemv_few_tokens_junk_pads():
    """w4a8_gemv at 2-64 tokens (the int8 matrix-core kernel's 16-token tiles, full and partial)
    on ragged shapes, with random bytes in q past d_in (act_quant_int8 leaves them unset), a q
    row stride past the padded width and a strided y: the int32 accumulators equal the oracle's
    O6 bit for bit, y is within the bar and bf16 y is the RNE image of fp32 y."""
    for M, d_out, d_in, extra in ((2, 1, 1, 0), (3, 70, 90, 16), (7, 257, 1000, 32),
                                  (16, 130, 3600, 0), (17, 64, 129, 48), (40, 300, 4100, 16),
                                  (64, 33, 777, 0)):
        what = f"M={M} {d_out}x{d_in}"
        _announce("w4a8_gemv few tokens, junk pads", what)
        w = workloads.weight(37, M + d_in, d_out, d_in)
        ph, pd = check_pack_bit_exact(w, 0, SYM, what)
        x = workloads.activations(37, M, M, d_in, 0.01, 20.0)
        bias_bits = workloads.bias(37, 3, d_out) if M % 2 else None
        q_o, s_o, _ = oracle.act_quant(x, d_in)
        acc_o, y_ref, nov = oracle.w4a8(q_o, s_o, ph[0], ph[1][:, 0], bias_bits, d_in)
        assert nov == 0
        ldq = (d_in + 15) // 16 * 16 + extra
        q = _q_with_junk_pads(q_o, d_in, ldq, 7 * M + d_in)
        s = torch.from_numpy(np.ascontiguousarray(s_o, dtype=np.float32)).cuda()
        b = dev_bf16(bias_bits) if bias_bits is not None else None
        out = torch.full((M, d_out + 5), float("nan"), dtype=torch.float32, device="cuda")
        y32, acc = w4.w4a8_gemv(q, s, pd[0], pd[1], b, d_in, F32, want_acc=True, out=out)
        y16 = w4.w4a8_gemv(q, s, pd[0], pd[1], b, d_in, BF16)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), acc_o), f"{what}: int32 accumulators differ"
        y32h = host(y32)[:, :d_out]
        assert_close(y32h, y_ref, what)
        assert np.isnan(host(out)[:, d_out:]).all(), f"{what}: write past d_out"
        assert_bf16_is_rne_of_f32(y16, y32h, what)


def _near_tie_activations():
    """Tokens whose values sit on and next to the rounding ties s (k + 1/2) of their own scale
    s = max|x| / 127, for every k in [-127, 126]; one token's maximum is so small that 1/s is
    not a finite fp32 number."""
    def f32(bits):
        return (np.asarray(bits, np.uint32) << 16).view(np.float32)

    rows = []
    extra = np.exp(np.random.default_rng(31).uniform(np.log(1e-3), np.log(1e3), 30))
    for a in (1.0, 3.0, 0.0118, 100.0, 2.5e-37, *extra):
        ab = workloads.to_bf16_bits(np.array([a], np.float32))[0]
        a32 = f32([ab])[0]
        s = np.float32(a32 / np.float32(127.0))
        ties = (np.arange(-127, 127, dtype=np.float64) + 0.5) * np.float64(s)
        b = workloads.to_bf16_bits(ties.astype(np.float32)).astype(np.int64)
        cand = np.concatenate([b, b + 1, b - 1]) & 0xFFFF
        v = f32(cand)
        keep = np.isfinite(v) & (np.abs(v) <= a32)  # the token's maximum stays a
        rows.append(np.concatenate([cand[keep], [ab]]).astype(np.uint16))
    K = max(len(r) for r in rows)
    x = np.zeros((len(rows), K), dtype=np.uint16)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    return x


def test_activation_codes_at_rounding_ties():
    """act_quant_int8 and w4a8_linear (its codes read back through weights that pick one column
    per row: code 9 at (j, j), 8 elsewhere, s_w = 1) against the oracle's O5, bit for bit."""
    x = _near_tie_activations()
    M, K = x.shape
    _announce("activation codes at rounding ties", M, K)
    q_o, s_o, _ = oracle.act_quant(x, K)
    ldx = (K + 7) // 8 * 8
    xp = np.zeros((M, ldx), dtype=np.uint16)
    xp[:, :K] = x
    q, s_x, _ = w4.act_quant_int8(dev_bf16(xp), K)
    torch.cuda.synchronize()
    assert np.array_equal(host(q)[:, :K], q_o), "act_quant codes differ at rounding ties"
    assert np.array_equal(host(s_x).view(np.uint32), s_o.view(np.uint32))
    k_pad = (K + 31) // 32 * 32
    codes = np.full((K, k_pad), 8, dtype=np.uint8)
    codes[np.arange(K), np.arange(K)] = 9
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    qw = torch.from_numpy(packed).cuda()
    sw = dev_bf16(np.full(K, 0x3F80, dtype=np.uint16))
    _, acc, sxf = w4.w4a8_linear(dev_bf16(xp), qw, sw, None, K, F32, want_acc=True,
                                 want_scales=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), q_o.astype(np.int32)), "fused codes differ at rounding ties"
    assert np.array_equal(host(sxf).view(np.uint32), s_o.view(np.uint32))


@pytest.mark.parametrize("H", [3584, 18944])
def test_w4a8_worst_case_accumulator(H):
    """All weight codes 0 (level -8) and all activations -127: acc = H * 1016 (3,641,344 for
    H = 3584, the Orin page's bound), exactly, in int32."""
    _announce("w4a8 worst case", H)
    qw = torch.zeros((4, H // 2), dtype=torch.uint8, device="cuda")
    sw = dev_bf16(workloads.to_bf16_bits(np.ones(4, np.float32)))
    q = torch.full((1, H), -127, dtype=torch.int8, device="cuda")
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    y, acc = w4.w4a8_gemv(q, s, qw, sw, None, H, F32, want_acc=True)
    torch.cuda.synchronize()
    assert host(acc).tolist() == [[H * 1016] * 4]
    if H == 3584:
        assert H * 1016 == 3641344
    assert host(y).tolist() == [[float(H * 1016)] * 4]
    # the prefill GEMM over 130 tokens (two token tiles)
    q = torch.full((130, H), -127, dtype=torch.int8, device="cuda")
    s = torch.ones(130, dtype=torch.float32, device="cuda")
    y, acc = w4.w4a8_gemm(q, s, qw, sw, None, H, F32, want_acc=True)
    torch.cuda.synchronize()
    assert host(acc).tolist() == [[H * 1016] * 4] * 130
    # fused: x = -1 everywhere quantizes to -127 everywhere (s_x = 1/127)
    x = dev_bf16(np.full((1, H), 0xBF80, dtype=np.uint16))
    y, acc = w4.w4a8_linear(x, qw, sw, None, H, F32, want_acc=True)
    torch.cuda.synchronize()
    assert host(acc).tolist() == [[H * 1016] * 4]


# ------------------------------------------------------------------------------------------
# activation outlier channels through every W4A16 kernel ([Infra] section 2.4: outliers sit in a
# few fixed channels): the int8 kernel turns each 128-column group of x into integers on a grid
# set by the group's largest value, so a channel x3000 must not cost the other columns of its
# group their precision
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [20.0, 3000.0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_w4a16_activation_outlier_channels(scale, mode):
    """1% of the input channels scaled (x20, as in C5, and x3000), the same channels for every
    token, against O4: the int8 decode kernel forced onto 1-4 tokens (groups 128 and per row),
    the streaming kernel at one token (forced), the few-token matrix-core kernel (2-16 tokens;
    with 32-column groups in its transposed layout) and the GEMM."""
    d_out, d_in = 640, 3584
    w = workloads.weight(51, mode, d_out, d_in)
    workloads.add_weight_outliers(w, 51, mode, 1e-3, 0.5)
    for g in (128, 0, 32):
        ph, pd = check_pack_bit_exact(w, g, mode, f"outliers g{g}")
        runs = [("i8", (1, 2, 3, 4)), ("stream", (1,)), (None, (2, 5, 8, 16))]
        for path, tokens in runs:
            with forced_decode_path(path):
                for M in tokens:
                    x = workloads.activations(51, M, M, d_in, 0.01, scale)
                    check_linear("w4_gemv", x, ph, pd, None, d_in, g,
                                 f"x{scale:g} channels g{g} path={path} M={M}")
        for M in (8, 130):
            x = workloads.activations(51, M, M, d_in, 0.01, scale)
            check_linear("w4_gemm", x, ph, pd, None, d_in, g, f"x{scale:g} channels g{g} gemm M={M}")


def test_gemv_c2_gate_up_outlier_channels_full_size():
    """The headline GEMV (C2 gate/up, 37888 x 3584, g128 SYM with its weight outliers) on
    activations with 1% of the channels x3000, by the kernel the library picks for one token,
    and the fused SiLU(gate) * up on the same input."""
    cfg = workloads.C2
    gu = cfg.linears[0]
    w = workloads.linear_weight(cfg, 0)
    ph, pd = check_pack_bit_exact(w, gu.group_size, gu.mode, "C2 gate/up")
    x = workloads.activations(cfg.seed, 90, 1, gu.d_in, 0.01, 3000.0)
    check_linear("w4_gemv", x, ph, pd, None, gu.d_in, gu.group_size, "C2 gate/up x3000 channels")
    check_glu(w, x, None, gu.group_size, gu.mode, "C2 gate/up x3000 channels")
