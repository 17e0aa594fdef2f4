"""CPU oracle for the group-wise INT4 weight-only linear layer (numpy front end).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline leg of the
benchmark import this package; the product library never does, and this package imports nothing
from it.  The arithmetic lives in oracle.c (plain C); this module only marshals numpy arrays.
The GPTQ reference (O9) is numpy fp64 in oracle/gptq.py.

Every function follows the pages cited in oracle.c:
  [Lab5]  "Lab 5: Gemma4 端到端推理优化"
  [Orin]  "Jetson Orin AGX INT4 推理优化实践：super 分支从 9 tok/s 到 24 tok/s"
  [Infra] "【infra之路】12-投机解码、量化与推理引擎对比"
  [QAT]   "Yeniden paketlenmiş QAT Gemma 4 26B-A4B, tek bir TPU v6e'de FP8 işlemenin 1.9 katı
          verimle sunuluyor"

Arrays: weights fp32 [d_out][d_in]; bf16 values travel as uint16 bit patterns; packed weights
uint8 [d_out][k_pad/2] (earlier column in the low nibble); scales/zeros uint16 (bf16)
[d_out][n_groups].
"""
import ctypes
import os

import numpy as np

SYM = 0
ASYM = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


class use_library:
    """Context manager: run the oracle API against another build of oracle.c (the mutation
    tests use it to show that the pins catch planted mistakes)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _lib
        _lib = _declare(ctypes.CDLL(self.path))
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _declare(lib):
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_bf16_to_f32_array.argtypes = [_p, _i64, _p]
    lib.oracle_bf16_to_f32_array.restype = None
    lib.oracle_f32_to_bf16_array.argtypes = [_p, _i64, _p]
    lib.oracle_f32_to_bf16_array.restype = None
    lib.oracle_k_pad.argtypes = [_i64, ctypes.c_int]
    lib.oracle_k_pad.restype = _i64
    lib.oracle_n_groups.argtypes = [_i64, ctypes.c_int]
    lib.oracle_n_groups.restype = _i64
    lib.oracle_pack.argtypes = [_p, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _p, _p, _p]
    lib.oracle_pack.restype = None
    lib.oracle_unpack.argtypes = [_p, _i64, _i64, _p]
    lib.oracle_unpack.restype = None
    lib.oracle_dequant.argtypes = [_p, _p, _p, _i64, _i64, ctypes.c_int, _p]
    lib.oracle_dequant.restype = None
    lib.oracle_w4a16.argtypes = [_p, _i64, _i64, _p, _p, _p, _p, _i64, _i64, ctypes.c_int, _p]
    lib.oracle_w4a16.restype = None
    lib.oracle_w4a16_points.argtypes = [_p, _i64, _p, _p, _p, _p, _i64, ctypes.c_int, _p, _p,
                                        _i64, _p]
    lib.oracle_w4a16_points.restype = None
    lib.oracle_act_quant.argtypes = [_p, _i64, _i64, _i64, _p, _i64, _p, _p]
    lib.oracle_act_quant.restype = None
    lib.oracle_w4a8.argtypes = [_p, _p, _i64, _i64, _p, _p, _p, _i64, _i64, _p, _p]
    lib.oracle_w4a8.restype = _i64
    lib.oracle_silu_mul.argtypes = [_p, _p, _i64, _p]
    lib.oracle_silu_mul.restype = None
    lib.oracle_qat_repack.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p]
    lib.oracle_qat_repack.restype = None
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def bf16_to_f32(bits):
    """bf16 bit patterns -> fp32 values (exact)."""
    lib = _load()
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(b.shape, dtype=np.float32)
    lib.oracle_bf16_to_f32_array(_ptr(b), b.size, _ptr(out))
    return out


def f32_to_bf16(vals):
    """fp32 values -> bf16 bit patterns, round to nearest even."""
    lib = _load()
    v = np.ascontiguousarray(vals, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    lib.oracle_f32_to_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def k_pad(d_in, group_size):
    return int(_load().oracle_k_pad(d_in, group_size))


def n_groups(d_in, group_size):
    return int(_load().oracle_n_groups(d_in, group_size))


def pack(w, group_size, mode):
    """O1 RTN pack.  Returns (qweight u8 [d_out][k_pad/2], scales u16 [d_out][G],
    zeros u16 [d_out][G] or None for symmetric)."""
    lib = _load()
    w = _c(w, np.float32)
    d_out, d_in = w.shape
    kp, ng = k_pad(d_in, group_size), n_groups(d_in, group_size)
    qw = np.zeros((d_out, kp // 2), dtype=np.uint8)
    sc = np.zeros((d_out, ng), dtype=np.uint16)
    zr = np.zeros((d_out, ng), dtype=np.uint16) if mode == ASYM else None
    lib.oracle_pack(_ptr(w), d_out, d_in, d_in, group_size, mode, _ptr(qw), _ptr(sc), _ptr(zr))
    return qw, sc, zr


def unpack(qweight):
    """O2: codes u8 [d_out][k_pad] from packed bytes."""
    lib = _load()
    qw = _c(qweight, np.uint8)
    d_out, nb = qw.shape
    codes = np.zeros((d_out, 2 * nb), dtype=np.uint8)
    lib.oracle_unpack(_ptr(qw), d_out, 2 * nb, _ptr(codes))
    return codes


def dequant(qweight, scales, zeros, d_in, group_size):
    """O3: fp64 w_hat [d_out][k_pad] (pads included)."""
    lib = _load()
    qw, sc, zr = _c(qweight, np.uint8), _c(scales, np.uint16), _c(zeros, np.uint16)
    d_out = qw.shape[0]
    out = np.zeros((d_out, k_pad(d_in, group_size)), dtype=np.float64)
    lib.oracle_dequant(_ptr(qw), _ptr(sc), _ptr(zr), d_out, d_in, group_size, _ptr(out))
    return out


def w4a16(x_bits, qweight, scales, zeros, bias_bits, d_in, group_size):
    """O4: fp64 y [M][d_out] = x . w_hat^T (+ b).  x_bits: u16 (bf16) [M][ldx >= d_in]."""
    lib = _load()
    x = _c(x_bits, np.uint16)
    qw, sc, zr, b = (_c(qweight, np.uint8), _c(scales, np.uint16), _c(zeros, np.uint16),
                     _c(bias_bits, np.uint16))
    M, ldx = x.shape
    d_out = qw.shape[0]
    y = np.zeros((M, d_out), dtype=np.float64)
    lib.oracle_w4a16(_ptr(x), M, ldx, _ptr(qw), _ptr(sc), _ptr(zr), _ptr(b), d_out, d_in,
                     group_size, _ptr(y))
    return y


def w4a16_points(x_bits, qweight, scales, zeros, bias_bits, d_in, group_size, tok, row):
    """O4 at the listed (token, row) pairs: fp64 [n]."""
    lib = _load()
    x = _c(x_bits, np.uint16)
    qw, sc, zr, b = (_c(qweight, np.uint8), _c(scales, np.uint16), _c(zeros, np.uint16),
                     _c(bias_bits, np.uint16))
    tok, row = _c(tok, np.int64), _c(row, np.int64)
    out = np.zeros(tok.shape[0], dtype=np.float64)
    lib.oracle_w4a16_points(_ptr(x), x.shape[1], _ptr(qw), _ptr(sc), _ptr(zr), _ptr(b), d_in,
                            group_size, _ptr(tok), _ptr(row), tok.shape[0], _ptr(out))
    return out


def act_quant(x_bits, K=None):
    """O5: (q int8 [M][K], s_x fp32 [M], q_sum int32 [M])."""
    lib = _load()
    x = _c(x_bits, np.uint16)
    M, ldx = x.shape
    K = ldx if K is None else K
    q = np.zeros((M, K), dtype=np.int8)
    s = np.zeros(M, dtype=np.float32)
    qs = np.zeros(M, dtype=np.int32)
    lib.oracle_act_quant(_ptr(x), M, K, ldx, _ptr(q), K, _ptr(s), _ptr(qs))
    return q, s, qs


def w4a8(q, s_x, qweight, s_w, bias_bits, d_in):
    """O6: (acc int32 [M][d_out], y fp64 [M][d_out], n_overflow)."""
    lib = _load()
    q = _c(q, np.int8)
    s_x = _c(s_x, np.float32)
    qw, sw, b = _c(qweight, np.uint8), _c(np.asarray(s_w).reshape(-1), np.uint16), _c(
        bias_bits, np.uint16)
    M, ldq = q.shape
    d_out = qw.shape[0]
    acc = np.zeros((M, d_out), dtype=np.int32)
    y = np.zeros((M, d_out), dtype=np.float64)
    n = lib.oracle_w4a8(_ptr(q), _ptr(s_x), M, ldq, _ptr(qw), _ptr(sw), _ptr(b), d_out, d_in,
                        _ptr(acc), _ptr(y))
    return acc, y, int(n)


def silu_mul(g, u):
    """O7: h = SiLU(g) * u elementwise (fp64), SiLU(v) = v / (1 + exp(-v))."""
    lib = _load()
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    if g.shape != u.shape:
        raise ValueError("g and u must have the same shape")
    h = np.zeros(g.shape, dtype=np.float64)
    lib.oracle_silu_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def w4a16_silu_mul(x_bits, qweight, scales, zeros, bias_bits, d_in, group_size):
    """O4 then O7 on a fused gate/up weight of 2H rows (gate rows [0, H), up rows [H, 2H)):
    h [M][H] fp64."""
    y = w4a16(x_bits, qweight, scales, zeros, bias_bits, d_in, group_size)
    H = y.shape[1] // 2
    return silu_mul(y[:, :H], y[:, H:])


def qat_repack(w_bits, d_in=None):
    """O8: repack of bf16 weights that sit on a 16-level grid per group of 32 columns.
    w_bits: u16 (bf16) [d_out][ldw >= d_in].  Returns (qweight u8 [d_out][k_pad/2],
    scales u16 [d_out][n_groups], m u8 [d_out][n_groups]; m = 0 marks a group off the grid)."""
    lib = _load()
    w = _c(w_bits, np.uint16)
    d_out, ldw = w.shape
    d_in = ldw if d_in is None else d_in
    kp = k_pad(d_in, 32)
    qw = np.zeros((d_out, kp // 2), dtype=np.uint8)
    sc = np.zeros((d_out, kp // 32), dtype=np.uint16)
    m = np.zeros((d_out, kp // 32), dtype=np.uint8)
    lib.oracle_qat_repack(_ptr(w), d_out, d_in, ldw, _ptr(qw), _ptr(sc), _ptr(m))
    return qw, sc, m


def set_num_threads(n):
    """Threads of the oracle's OpenMP loops from now on (the benchmark's timing leg sets 1 for its
    single-thread figures).  No effect on results: every parallel loop is over independent
    outputs."""
    _load()
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))


def max_threads():
    """Threads the next OpenMP loop of the oracle uses."""
    _load()
    return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())


def tolerance_ok(y, y_ref, rel=2e-3):
    """The floating-point parity bar: |y - y_ref| <= rel * (1 + |y_ref|), elementwise."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return np.abs(y - y_ref) <= rel * (1.0 + np.abs(y_ref))
