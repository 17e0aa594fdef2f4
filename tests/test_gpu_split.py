"""GPU parity of w4_gemv_ws, the few-token decode with the reduction over d_in split over column
slices (partial sums through a caller workspace), against the CPU oracle (O4) on the same seeded
inputs.  Bars as in test_gpu_parity: |y - y_ref| <= 2e-3 (1 + |y_ref|) on the fp32 output, the
bf16 output the round-to-nearest-even image of the fp32 one, exact basis probes.

The library takes the split path only on matrices with few, long rows (the C3 down projection);
the small shapes here run it through the test build's hook (forced_decode_path("split"))."""
import numpy as np
import pytest
import torch

import int4_weight_only_amd as w4
import oracle
import workloads
from tests.gpu_helpers import assert_close, dev_bf16, forced_decode_path, host
from tests.test_gpu_parity import check_linear, check_pack_bit_exact

pytestmark = pytest.mark.gpu

SYM, ASYM = w4.W4_SYM, w4.W4_ASYM
F32, BF16 = w4.W4_OUT_F32, w4.W4_OUT_BF16


def _announce(*what):
    print("[case]", *what, flush=True)


def test_split_is_chosen_where_rows_are_few_and_long():
    # the library takes the split path (a workspace) for 2..64 tokens on matrices with fewer
    # than four 16-row tiles and at least 64 KiB of codes per compute unit
    assert w4.w4_gemv_work_bytes(16, 3584, 18944, 128) > 0
    assert w4.w4_gemv_work_bytes(8, 3584, 18944, 128) > 0
    assert w4.w4_gemv_work_bytes(16, 3584, 3584, 128) == 0   # short rows
    assert w4.w4_gemv_work_bytes(16, 4608, 3584, 128) == 0
    assert w4.w4_gemv_work_bytes(1, 3584, 18944, 128) == 0   # one token
    assert w4.w4_gemv_work_bytes(16, 37888, 3584, 128) == 0  # many rows
    assert w4.w4_gemv_work_bytes(16, 3584, 18944, 32) == 0   # groups inside a chunk
    with forced_decode_path("split"):
        assert w4.w4_gemv_work_bytes(16, 3584, 3584, 128) > 0
        assert w4.w4_gemv_work_bytes(2, 130, 100, 128) == 0  # one 128-column chunk: one slice


@pytest.mark.parametrize("g", [32, 64, 128, 256, 0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_gemv_ws_ragged(g, mode):
    """Ragged rows, columns and tokens (several row slices, several column slices, partial last
    tiles and chunks, a second 16-token tile), with bias, padded x rows and y rows."""
    shapes = [(2, 130, 100), (16, 257, 1000), (17, 200, 3600), (5, 1, 1), (64, 520, 2100),
              (33, 1100, 700)]
    for M, d_out, d_in in shapes:
        w = workloads.weight(61, M + d_out + d_in + g, d_out, d_in)
        ph, pd = check_pack_bit_exact(w, g, mode, "split ragged")
        x = workloads.activations(61, g + mode, M, d_in)
        b = workloads.bias(61, 1, d_out)
        ldx = (d_in + 7) // 8 * 8 + 8
        with forced_decode_path("split"):
            check_linear("w4_gemv_ws", x, ph, pd, b, d_in, g, f"split M={M} {d_out}x{d_in}",
                         ldx=ldx, ldy=d_out + 3)


def test_gemv_ws_c3_layers():
    """The C3 shapes (asymmetric g128) at 8 and 16 tokens, first and last layer, with the
    library's choice (down takes the split path, the others w4_gemv's kernels) and with the split
    forced wherever it applies (q/k/v, o, down)."""
    cfg = workloads.C3
    for layer in (0, cfg.repeat_layers - 1):
        for li, lin in enumerate(cfg.linears):
            w = workloads.linear_weight(cfg, li, layer=layer)
            ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, f"C3/L{layer}/{lin.name}")
            for M in cfg.tokens:
                if M < 2:
                    continue
                x = workloads.linear_x(cfg, li, M, layer=layer)
                for path in (None, "split"):
                    with forced_decode_path(path):
                        check_linear("w4_gemv_ws", x, ph, pd, None, lin.d_in, lin.group_size,
                                     f"split C3/L{layer}/{lin.name} M={M} path={path}")


def test_gemv_ws_basis_probes_exact():
    """x = e_k gives y[j] = w_hat[j][k] exactly: pins the nibble order, the group index, the
    scale and the zero point of every probed column on the split path (15 tokens)."""
    d_out, d_in = 96, 300
    w = workloads.weight(62, 0, d_out, d_in)
    cols = [0, 1, 2, 7, 8, 31, 32, 33, 63, 64, 127, 128, 255, 256, 299]
    for g, mode in ((32, SYM), (64, ASYM), (128, ASYM), (256, SYM), (0, SYM)):
        ph, pd = check_pack_bit_exact(w, g, mode, "split probe")
        wh = oracle.dequant(ph[0], ph[1], ph[2], d_in, g)
        x = np.zeros((len(cols), (d_in + 7) // 8 * 8), dtype=np.uint16)
        for i, k in enumerate(cols):
            x[i, k] = 0x3F80
        with forced_decode_path("split"):
            # groups of 32 and 64 columns take the w4_gemv path (no workspace)
            assert (w4.w4_gemv_work_bytes(len(cols), d_out, d_in, g) > 0) == (g not in (32, 64))
            y = w4.w4_gemv_ws(dev_bf16(x), *pd, None, d_in, g, F32)
        assert np.array_equal(host(y).astype(np.float64), wh[:, cols].T), \
            f"split basis probe g={g} mode={mode}"


def test_gemv_ws_zero_points_beyond_pack():
    """Zero points w4_pack never writes (non-integers, beyond the code range): the residual path."""
    d_out, d_in = 300, 1000
    w = workloads.weight(63, 0, d_out, d_in)
    rng = np.random.default_rng(63)
    for gg in (128, 32):
        ph, pd = check_pack_bit_exact(w, gg, ASYM, f"split zero points g{gg}")
        zf = rng.choice(np.array([0.5, 7.25, -3.0, 20.0, 300.0, -1000.0, 7.0, 15.0], np.float32),
                        size=ph[2].shape)
        zb = workloads.to_bf16_bits(zf)
        ph2 = (ph[0], ph[1], zb)
        pd2 = (pd[0], pd[1], dev_bf16(zb))
        b = workloads.bias(63, 1, d_out)
        for M in (2, 5, 16, 20):
            x = workloads.activations(63, M, M, d_in)
            with forced_decode_path("split"):
                check_linear("w4_gemv_ws", x, ph2, pd2, b, d_in, gg,
                             f"split z beyond pack g{gg} M={M}")


@pytest.mark.parametrize("scale", [20.0, 3000.0])
@pytest.mark.parametrize("mode", [SYM, ASYM])
def test_gemv_ws_activation_outlier_channels(scale, mode):
    """1% of the input channels scaled x20 (as in C5) and x3000, the same channels for every token."""
    d_out, d_in = 640, 3584
    w = workloads.weight(64, mode, d_out, d_in)
    workloads.add_weight_outliers(w, 64, mode, 1e-3, 0.5)
    for g in (128, 0, 32):
        ph, pd = check_pack_bit_exact(w, g, mode, f"split outliers g{g}")
        for M in (2, 8, 16):
            x = workloads.activations(64, M, M, d_in, 0.01, scale)
            with forced_decode_path("split"):
                check_linear("w4_gemv_ws", x, ph, pd, None, d_in, g,
                             f"split x{scale:g} channels g{g} M={M}")


def test_gemv_ws_junk_pads():
    """d_in := k_pad on activations whose pad columns hold 1e3: the pad columns must be multiplied
    by exact zeros (the d_in = 3600 layer of C3, 8 and 16 tokens)."""
    cfg = workloads.C3
    lin = cfg.extra[0]
    w = workloads.linear_weight(cfg, 4, lin=lin)
    ph, pd = check_pack_bit_exact(w, lin.group_size, lin.mode, "split pad3600")
    k_pad = oracle.k_pad(lin.d_in, lin.group_size)
    for M in (8, 16):
        x = workloads.linear_x(cfg, 4, M, lin=lin)
        xj = np.zeros((M, k_pad), dtype=np.uint16)
        xj[:, :lin.d_in] = x
        xj[:, lin.d_in:] = workloads.to_bf16_bits(np.array([1000.0], np.float32))[0]
        _announce("w4_gemv_ws", "junk pads", M)
        with forced_decode_path("split"):
            y = w4.w4_gemv_ws(dev_bf16(xj), *pd, None, k_pad, lin.group_size, F32)
        y_ref = oracle.w4a16(x, ph[0], ph[1], ph[2], None, lin.d_in, lin.group_size)
        assert_close(host(y), y_ref, f"split junk pads M={M}")


def test_gemv_ws_longest_rows():
    """d_in = 65536, the decode limit (the most column slices and chunks per slice)."""
    d_out, d_in, g = 200, 65536, 128
    w = workloads.weight(65, 0, d_out, d_in)
    ph, pd = check_pack_bit_exact(w, g, ASYM, "split d_in 65536")
    for M in (3, 16):
        x = workloads.activations(65, M, M, d_in)
        with forced_decode_path("split"):
            check_linear("w4_gemv_ws", x, ph, pd, None, d_in, g, f"split d_in=65536 M={M}")


def test_gemv_ws_workspace_reuse_and_determinism():
    """One workspace, filled with NaN first, shared by calls of different shapes and token counts
    in turn: the results are bitwise those of a fresh workspace, and repeated calls are bitwise
    identical (the slices are added in a fixed order). Every call writes into an output filled
    with NaN first."""
    d_out, d_in, g = 1000, 3584, 128
    w = workloads.weight(66, 0, d_out, d_in)
    _, pd = check_pack_bit_exact(w, g, ASYM, "split workspace")
    x = dev_bf16(workloads.activations(66, 0, 16, d_in))
    w2 = workloads.weight(66, 1, 3584, 18944)
    _, pd2 = check_pack_bit_exact(w2, 128, SYM, "split workspace 2")
    x2 = dev_bf16(workloads.activations(66, 1, 5, 18944))

    def run(xx, p, din, gg, rows, wk):
        out = torch.full((xx.shape[0], rows), float("nan"), dtype=torch.float32, device="cuda")
        return host(w4.w4_gemv_ws(xx, *p, None, din, gg, F32, out=out, work=wk))

    with forced_decode_path("split"):
        n1 = w4.w4_gemv_work_bytes(16, d_out, d_in, g)
        n2 = w4.w4_gemv_work_bytes(5, 3584, 18944, 128)
        assert n1 > 0 and n2 > 0
        work = torch.full((max(n1, n2) // 4,), float("nan"), dtype=torch.float32,
                          device="cuda").view(torch.uint8)
        first = run(x, pd, d_in, g, d_out, work)
        first2 = run(x2, pd2, 18944, 128, 3584, work)
        assert np.all(np.isfinite(first)) and np.all(np.isfinite(first2))
        for _ in range(3):
            again = run(x, pd, d_in, g, d_out, work)
            again2 = run(x2, pd2, 18944, 128, 3584, work)
            assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
            assert np.array_equal(first2.view(np.uint32), again2.view(np.uint32))
        fresh = run(x, pd, d_in, g, d_out, None)
        assert np.array_equal(first.view(np.uint32), fresh.view(np.uint32))


def test_gemv_ws_agrees_with_gemv():
    """Both decode entry points on the same C3-like inputs, within the bar of each other's oracle
    distance (each is also checked against the oracle above)."""
    d_out, d_in, g = 3584, 18944, 128
    w = workloads.weight(67, 0, d_out, d_in)
    ph, pd = check_pack_bit_exact(w, g, ASYM, "split vs gemv")
    x_bits = workloads.activations(67, 0, 16, d_in)
    x = dev_bf16(x_bits)
    a = host(w4.w4_gemv_ws(x, *pd, None, d_in, g, F32))
    b = host(w4.w4_gemv(x, *pd, None, d_in, g, F32))
    y_ref = oracle.w4a16(x_bits, ph[0], ph[1], ph[2], None, d_in, g)
    assert_close(a, y_ref, "split down M=16")
    assert_close(b, y_ref, "gemv down M=16")
