"""Host-side checks of the Python binding (no GPU): a caller-supplied output must hold the
(M, d_out) result at its own row stride, or the call is refused before anything reaches the
library (a short or overlapping `out` would let the kernels write past the tensor)."""
import pytest
import torch

import int4_weight_only_amd as w4


def test_out_must_cover_every_row_and_column():
    ok = torch.empty((4, 128))
    w4._check_out_shape(ok, 4, 128)
    w4._check_out_shape(torch.empty((8, 200))[:, :128], 4, 128)  # strided view, stride 200
    with pytest.raises(ValueError):
        w4._check_out_shape(torch.empty((1, 128)), 4, 128)  # too few rows
    with pytest.raises(ValueError):
        w4._check_out_shape(torch.empty((4, 127)), 4, 128)  # too few columns
    with pytest.raises(ValueError):
        w4._check_out_shape(torch.empty((4, 200))[:, :100], 4, 128)  # a view narrower than d_out
    overlapping = torch.empty(4 * 64 + 64).as_strided((4, 128), (64, 1))
    with pytest.raises(ValueError):
        w4._check_out_shape(overlapping, 4, 128)  # rows that overlap


def test_single_row_out_may_have_any_stride():
    w4._check_out_shape(torch.empty(128).as_strided((1, 128), (1, 1)), 1, 128)


def test_binding_never_computes_on_the_cpu():
    """No CPU fallback: host tensors are refused."""
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    qw = torch.zeros((128, 128), dtype=torch.uint8)
    sc = torch.zeros((128, 2), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        w4.w4_gemv(x, qw, sc, None, None, 256, 128)
