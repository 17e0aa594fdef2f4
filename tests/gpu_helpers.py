"""Helpers shared by the GPU parity tests: host <-> device conversion of bf16 bit patterns and
the parity bar.  No quantization arithmetic lives here."""
import contextlib
import os

import numpy as np
import torch

import int4_weight_only_amd as w4
import oracle

HOOKS_LIB = os.path.join(os.path.dirname(w4.__file__), "libw4_hooks.so")

REL_TOL = 2e-3  # |y - y_ref| <= REL_TOL * (1 + |y_ref|) on fp32 outputs


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on cuda:0."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    """torch.bfloat16 (any device) -> uint16 numpy bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().contiguous().cpu().numpy()


def assert_close(y, y_ref, what=""):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = np.abs(y - y_ref)
    bound = REL_TOL * (1.0 + np.abs(y_ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside "
                             f"2e-3*(1+|y|); worst at {i}: got {y[i]!r} want {y_ref[i]!r}")
    return float((err / bound).max())


def assert_bf16_is_rne_of_f32(y_bf16, y_f32, what=""):
    """The bf16 output of a call must be the round-to-nearest-even image of the fp32 output of
    the same call (same deterministic accumulation)."""
    want = oracle.f32_to_bf16(np.asarray(y_f32, dtype=np.float32))
    got = host_bits(y_bf16)
    assert np.array_equal(got, want), f"{what}: bf16 output is not RNE(fp32 output)"


@contextlib.contextmanager
def forced_decode_path(path):
    """Run the library's test build (libw4_hooks.so: the same kernels, plus a hook on the decode
    kernel choice) with the choice forced: "i8" = the int8 matrix-core kernel wherever it applies,
    "stream" = never it, "split" = the column-split kernel of w4_gemv_ws wherever it applies,
    None = the library's own choice."""
    code = {None: 0, "i8": 1, "stream": 2, "split": 3}[path]
    prev = w4._select_library(HOOKS_LIB)
    try:
        assert w4._lib.w4_test_force_decode_path(code) == 0
        yield
    finally:
        w4._lib.w4_test_force_decode_path(0)
        w4._select_library(prev)
