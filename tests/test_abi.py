"""Host-side checks of the C ABI (no GPU): the library loads, exports every function declared in
include/w4.h, reports the packed layout, and rejects invalid arguments before touching the GPU.
Pointer arguments here are fake addresses that the library must never dereference: every call
below fails validation first."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")
LIB = os.path.join(ROOT, "int4_weight_only_amd", "libw4.so")

W4_OK, W4_ERR_NULL, W4_ERR_SHAPE, W4_ERR_GROUP, W4_ERR_ALIGN, W4_ERR_RANGE = 0, 1, 2, 3, 4, 5
W4_ERR_UNSUPPORTED, W4_ERR_HIP = 6, 7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:int|size_t|const char \*)\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libw4.so is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.w4_packed_layout.argtypes = [i64, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                   ctypes.POINTER(ctypes.c_size_t)]
    L.w4_pack.argtypes = [p, i64, i64, i64, i32, i32, p, p, p, p]
    L.w4_qat_repack.argtypes = [p, i64, i64, i64, p, p, p, p]
    L.w4_gptq_hessian.argtypes = [p, i64, i64, i64, p, p]
    L.w4_gptq_factor.argtypes = [p, i64, ctypes.c_float, p, p, p, p]
    L.w4_gptq_quantize.argtypes = [p, i64, i64, i64, p, p, i32, i32, p, p, p, p, p, p]
    lin = [p, i64, i64, p, p, p, p, i64, i64, i32, p, i64, i32]
    L.w4_gemv.argtypes = lin + [p]
    L.w4_gemv_ws.argtypes = lin + [p, ctypes.c_size_t, p]
    L.w4_gemv_work_bytes.argtypes = [i64, i64, i64, i32]
    L.w4_gemv_work_bytes.restype = ctypes.c_size_t
    L.w4_gemv_glu.argtypes = lin + [p]
    L.w4_gemm.argtypes = lin + [p]
    L.act_quant_int8.argtypes = [p, i64, i64, i64, p, i64, p, p, p]
    L.w4a8_gemv.argtypes = [p, p, i64, i64, p, p, p, i64, i64, p, i64, i32, p, p]
    L.w4a8_gemm.argtypes = L.w4a8_gemv.argtypes
    L.w4a8_linear.argtypes = [p, i64, i64, p, p, p, i64, i64, p, i64, i32, p, p, p]
    L.w4_status_string.restype = ctypes.c_char_p
    L.w4_last_hip_error.restype = ctypes.c_char_p
    return L


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("w4_pack", "w4_gemv", "w4_gemv_ws", "w4_gemv_work_bytes", "w4_gemv_glu", "w4_gemm", "act_quant_int8", "w4a8_gemv",
              "w4a8_gemm", "w4a8_linear", "w4_qat_repack", "w4_gptq_hessian", "w4_gptq_factor",
              "w4_gptq_quantize",
              "w4_packed_layout", "w4_status_string",
              "w4_last_hip_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_test_hook_only_in_the_test_build(lib):
    """The kernel-choice hook exists only in libw4_hooks.so (the tests' build); the product
    library has no runtime switch of any kind."""
    assert not hasattr(lib, "w4_test_force_decode_path")
    hooks = os.path.join(ROOT, "int4_weight_only_amd", "libw4_hooks.so")
    h = ctypes.CDLL(hooks)
    assert hasattr(h, "w4_test_force_decode_path")
    for name in declared_functions():
        assert hasattr(h, name), name
    h.w4_test_force_decode_path.argtypes = [ctypes.c_int]
    assert h.w4_test_force_decode_path(4) == W4_ERR_RANGE
    assert h.w4_test_force_decode_path(-1) == W4_ERR_RANGE
    assert h.w4_test_force_decode_path(0) == W4_OK


def test_library_sources_read_no_environment():
    csrc = os.path.join(ROOT, "int4_weight_only_amd", "csrc")
    for f in os.listdir(csrc):
        assert "getenv" not in open(os.path.join(csrc, f)).read(), f


def test_status_strings(lib):
    for s in range(8):
        assert lib.w4_status_string(s)
    assert lib.w4_last_hip_error() == b""


def test_packed_layout(lib):
    kp, ng, nb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    cases = [
        # (d_out, d_in, g) -> (k_pad, n_groups)
        ((3584, 3600, 128), (3712, 29)),
        ((37888, 3584, 128), (3584, 28)),
        ((3584, 18944, 32), (18944, 592)),
        ((18944, 3584, 0), (3584, 1)),
        ((7, 70, 0), (96, 1)),
        ((1, 1, 256), (256, 1)),
    ]
    for (d_out, d_in, g), (k_pad, n_groups) in cases:
        assert lib.w4_packed_layout(d_out, d_in, g, ctypes.byref(kp), ctypes.byref(ng),
                                    ctypes.byref(nb)) == W4_OK
        assert (kp.value, ng.value, nb.value) == (k_pad, n_groups, d_out * k_pad // 2)
    # one packed row of hidden size 3584 is 1792 bytes (the Orin page's per-row table)
    lib.w4_packed_layout(1, 3584, 128, ctypes.byref(kp), ctypes.byref(ng), ctypes.byref(nb))
    assert nb.value == 1792
    assert lib.w4_packed_layout(1, 64, 48, None, None, None) == W4_ERR_GROUP
    assert lib.w4_packed_layout(0, 64, 32, None, None, None) == W4_ERR_SHAPE
    assert lib.w4_packed_layout(1, (1 << 24) + 1, 32, None, None, None) == W4_ERR_RANGE


A = 0x10000  # fake, 16-byte aligned "device" addresses (never dereferenced)
B, C, D, E = 0x20000, 0x30000, 0x40000, 0x50000


def _lin(fn, **kw):
    a = dict(x=A, M=1, ldx=256, qw=B, sc=C, zr=None, bias=None, d_out=128, d_in=256, g=32, y=D,
             ldy=128, out=0)
    a.update(kw)
    args = [a["x"], a["M"], a["ldx"], a["qw"], a["sc"], a["zr"], a["bias"], a["d_out"],
            a["d_in"], a["g"], a["y"], a["ldy"], a["out"]]
    return fn(*args, None)


@pytest.mark.parametrize("entry", ["w4_gemv", "w4_gemm"])
def test_linear_rejects_bad_arguments(lib, entry):
    fn = getattr(lib, entry)
    assert _lin(fn, x=None) == W4_ERR_NULL
    assert _lin(fn, qw=None) == W4_ERR_NULL
    assert _lin(fn, sc=None) == W4_ERR_NULL
    assert _lin(fn, y=None) == W4_ERR_NULL
    assert _lin(fn, M=0) == W4_ERR_SHAPE
    assert _lin(fn, d_out=0) == W4_ERR_SHAPE
    assert _lin(fn, d_in=0) == W4_ERR_SHAPE
    assert _lin(fn, ldx=128) == W4_ERR_SHAPE
    assert _lin(fn, ldy=64) == W4_ERR_SHAPE
    assert _lin(fn, g=16) == W4_ERR_GROUP
    assert _lin(fn, g=96) == W4_ERR_GROUP
    assert _lin(fn, out=2) == W4_ERR_UNSUPPORTED
    assert _lin(fn, x=A + 8) == W4_ERR_ALIGN
    assert _lin(fn, ldx=260) == W4_ERR_ALIGN
    assert _lin(fn, qw=B + 4) == W4_ERR_ALIGN
    assert _lin(fn, y=D + 1) == W4_ERR_ALIGN
    assert _lin(fn, y=D + 2, out=1) == W4_ERR_ALIGN
    assert _lin(fn, zr=E + 1) == W4_ERR_ALIGN
    assert _lin(fn, d_in=(1 << 24) + 8, ldx=(1 << 24) + 8) == W4_ERR_RANGE


def _lin_ws(lib, work, work_bytes, **kw):
    a = dict(x=A, M=16, ldx=18944, qw=B, sc=C, zr=None, bias=None, d_out=3584, d_in=18944, g=128,
             y=D, ldy=3584, out=0)
    a.update(kw)
    args = [a["x"], a["M"], a["ldx"], a["qw"], a["sc"], a["zr"], a["bias"], a["d_out"],
            a["d_in"], a["g"], a["y"], a["ldy"], a["out"]]
    return lib.w4_gemv_ws(*args, work, work_bytes, None)


def test_gemv_work_bytes(lib):
    # few rows per compute unit and 2..64 tokens: S column slices of fp32 partial sums
    # S column slices of fp32 partial sums
    need = lib.w4_gemv_work_bytes(16, 3584, 18944, 128)
    assert need > 0 and need % (16 * 3584 * 4) == 0
    assert 2 <= need // (16 * 3584 * 4) <= 18944 // 128 + 1
    # short rows (q/k/v, o: under 64 KiB of codes per compute unit) take the w4_gemv path
    assert lib.w4_gemv_work_bytes(16, 4608, 3584, 128) == 0
    # one token, more than 64 tokens, many rows, invalid arguments: no workspace
    assert lib.w4_gemv_work_bytes(1, 3584, 18944, 128) == 0
    assert lib.w4_gemv_work_bytes(65, 3584, 18944, 128) == 0
    assert lib.w4_gemv_work_bytes(16, 37888, 3584, 128) == 0
    assert lib.w4_gemv_work_bytes(16, 3584, 18944, 48) == 0
    assert lib.w4_gemv_work_bytes(16, 0, 18944, 128) == 0


def test_gemv_ws_rejects_bad_workspaces(lib):
    need = lib.w4_gemv_work_bytes(16, 3584, 18944, 128)
    assert _lin_ws(lib, None, need) == W4_ERR_NULL
    assert _lin_ws(lib, E, need - 4) == W4_ERR_RANGE
    assert _lin_ws(lib, E + 4, need) == W4_ERR_ALIGN
    # the checks of w4_gemv come first
    assert _lin_ws(lib, E, need, x=None) == W4_ERR_NULL
    assert _lin_ws(lib, E, need, M=65) == W4_ERR_UNSUPPORTED
    assert _lin_ws(lib, E, need, g=96) == W4_ERR_GROUP


def test_gemv_token_limit(lib):
    # M > 64 belongs to the prefill path
    assert _lin(lib.w4_gemv, M=65) == W4_ERR_UNSUPPORTED
    assert _lin(lib.w4_gemv, d_in=65544, ldx=65544) == W4_ERR_RANGE


def test_pack_rejects_bad_arguments(lib):
    f = lib.w4_pack
    ok = dict(w=A, d_out=128, d_in=256, ldw=256, g=32, mode=0, qw=B, sc=C, zr=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["w"], a["d_out"], a["d_in"], a["ldw"], a["g"], a["mode"], a["qw"], a["sc"],
                 a["zr"], None)

    assert call(w=None) == W4_ERR_NULL
    assert call(zr=E) == W4_ERR_NULL  # symmetric packs have no zeros
    assert call(mode=1) == W4_ERR_NULL  # asymmetric packs need zeros
    assert call(mode=2) == W4_ERR_UNSUPPORTED
    assert call(ldw=255) == W4_ERR_SHAPE
    assert call(g=8) == W4_ERR_GROUP
    assert call(qw=B + 8) == W4_ERR_ALIGN
    assert call(w=A + 2) == W4_ERR_ALIGN


def test_act_quant_rejects_bad_arguments(lib):
    f = lib.act_quant_int8
    assert f(None, 1, 256, 256, B, 256, C, None, None) == W4_ERR_NULL
    assert f(A, 0, 256, 256, B, 256, C, None, None) == W4_ERR_SHAPE
    assert f(A, 1, 256, 128, B, 256, C, None, None) == W4_ERR_SHAPE
    assert f(A, 1, 256, 256, B, 248, C, None, None) == W4_ERR_SHAPE
    assert f(A, 1, 256, 256, B, 264, C, None, None) == W4_ERR_ALIGN
    assert f(A, 1, 256, 256, B + 8, 256, C, None, None) == W4_ERR_ALIGN
    assert f(A + 2, 1, 256, 256, B, 256, C, None, None) == W4_ERR_ALIGN


def test_w4a8_rejects_bad_arguments(lib):
    f = lib.w4a8_gemv

    def call(**kw):
        a = dict(q=A, sx=B, M=1, ldq=256, qw=C, sw=D, bias=None, d_out=128, d_in=256, y=E,
                 ldy=128, out=0, acc=None)
        a.update(kw)
        return f(a["q"], a["sx"], a["M"], a["ldq"], a["qw"], a["sw"], a["bias"], a["d_out"],
                 a["d_in"], a["y"], a["ldy"], a["out"], a["acc"], None)

    assert call(q=None) == W4_ERR_NULL
    assert call(sw=None) == W4_ERR_NULL
    assert call(M=0) == W4_ERR_SHAPE
    assert call(M=65) == W4_ERR_UNSUPPORTED
    assert call(ldq=255) == W4_ERR_SHAPE
    assert call(ldq=264) == W4_ERR_ALIGN
    assert call(acc=E + 2) == W4_ERR_ALIGN
    big = (1 << 20) + 16
    assert call(d_in=big, ldq=big) == W4_ERR_RANGE
    # the decode kernels' limit: d_in <= W4_DECODE_MAX_D_IN = 65536 (w4a8_gemm serves up to 2^20)
    assert call(d_in=65552, ldq=65552) == W4_ERR_RANGE
    assert call(d_in=65536, ldq=65536, q=None) == W4_ERR_NULL  # in range: fails only on the NULL


def test_header_states_the_decode_limit():
    text = open(HEADER).read()
    assert re.search(r"#define W4_DECODE_MAX_D_IN \(\(int64_t\)1 << 16\)", text)
    for fn in ("w4_gemv", "w4a8_gemv", "w4a8_linear", "w4_gemv_glu"):
        block = text[text.index(f" * {fn} --"):]
        block = block[:block.index("void *stream);")]
        assert "W4_DECODE_MAX_D_IN" in block, fn


def test_gptq_rejects_bad_arguments(lib):
    h = lib.w4_gptq_hessian
    assert h(None, 8, 64, 64, B, None) == W4_ERR_NULL
    assert h(A, 8, 64, 64, None, None) == W4_ERR_NULL
    assert h(A, 0, 64, 64, B, None) == W4_ERR_SHAPE
    assert h(A, 8, 64, 32, B, None) == W4_ERR_SHAPE
    assert h(A + 1, 8, 64, 64, B, None) == W4_ERR_ALIGN
    assert h(A, 8, 8193, 8200, B, None) == W4_ERR_RANGE
    f = lib.w4_gptq_factor
    assert f(None, 64, 0.01, B, C, D, None) == W4_ERR_NULL
    assert f(A, 64, 0.01, B, C, None, None) == W4_ERR_NULL
    assert f(A, 0, 0.01, B, C, D, None) == W4_ERR_SHAPE
    assert f(A, 8193, 0.01, B, C, D, None) == W4_ERR_RANGE
    assert f(A, 64, -1.0, B, C, D, None) == W4_ERR_RANGE
    assert f(A, 64, float("nan"), B, C, D, None) == W4_ERR_RANGE
    assert f(A + 2, 64, 0.01, B, C, D, None) == W4_ERR_ALIGN
    q = lib.w4_gptq_quantize

    def call(**kw):
        a = dict(w=A, d_out=16, d_in=64, ldw=64, u=B, dead=None, g=32, mode=0, qw=C, sc=D, zr=None,
                 work=E, loss=None)
        a.update(kw)
        return q(a["w"], a["d_out"], a["d_in"], a["ldw"], a["u"], a["dead"], a["g"], a["mode"],
                 a["qw"], a["sc"], a["zr"], a["work"], a["loss"], None)

    assert call(w=None) == W4_ERR_NULL
    assert call(work=None) == W4_ERR_NULL
    assert call(mode=1) == W4_ERR_NULL  # asymmetric without zeros
    assert call(zr=E) == W4_ERR_NULL    # symmetric with zeros
    assert call(mode=2) == W4_ERR_UNSUPPORTED
    assert call(d_out=0) == W4_ERR_SHAPE
    assert call(ldw=32) == W4_ERR_SHAPE
    assert call(g=48) == W4_ERR_GROUP
    assert call(d_in=8193, ldw=8193) == W4_ERR_RANGE
    assert call(w=A + 2) == W4_ERR_ALIGN
    assert call(loss=E + 2) == W4_ERR_ALIGN


def test_qat_repack_rejects_bad_arguments(lib):
    f = lib.w4_qat_repack

    def call(**kw):
        a = dict(w=A, d_out=16, d_in=100, ldw=104, qw=C, sc=D, m=None)
        a.update(kw)
        return f(a["w"], a["d_out"], a["d_in"], a["ldw"], a["qw"], a["sc"], a["m"], None)

    assert call(w=None) == W4_ERR_NULL
    assert call(qw=None) == W4_ERR_NULL
    assert call(sc=None) == W4_ERR_NULL
    assert call(d_out=0) == W4_ERR_SHAPE
    assert call(d_in=0) == W4_ERR_SHAPE
    assert call(ldw=96) == W4_ERR_SHAPE
    assert call(ldw=108) == W4_ERR_ALIGN
    assert call(w=A + 8) == W4_ERR_ALIGN
    assert call(qw=C + 8) == W4_ERR_ALIGN
    assert call(sc=D + 1) == W4_ERR_ALIGN
    assert call(d_in=(1 << 24) + 8, ldw=(1 << 24) + 8) == W4_ERR_RANGE
    # the grid: d_out * ceil(d_in / 32) / 256 < 2^31
    assert call(d_out=1 << 24, d_in=1 << 24, ldw=1 << 24) == W4_ERR_RANGE


def test_w4a8_gemm_rejects_bad_arguments(lib):
    f = lib.w4a8_gemm

    def call(**kw):
        a = dict(q=A, sx=B, M=1000, ldq=256, qw=C, sw=D, bias=None, d_out=128, d_in=256, y=E,
                 ldy=128, out=0, acc=None)
        a.update(kw)
        return f(a["q"], a["sx"], a["M"], a["ldq"], a["qw"], a["sw"], a["bias"], a["d_out"],
                 a["d_in"], a["y"], a["ldy"], a["out"], a["acc"], None)

    assert call(q=None) == W4_ERR_NULL
    assert call(sx=None) == W4_ERR_NULL
    assert call(qw=None) == W4_ERR_NULL
    assert call(sw=None) == W4_ERR_NULL
    assert call(y=None) == W4_ERR_NULL
    assert call(M=0) == W4_ERR_SHAPE
    assert call(d_out=0) == W4_ERR_SHAPE
    assert call(ldq=255) == W4_ERR_SHAPE
    assert call(ldy=127) == W4_ERR_SHAPE
    assert call(ldq=264) == W4_ERR_ALIGN
    assert call(q=A + 8) == W4_ERR_ALIGN
    assert call(qw=C + 8) == W4_ERR_ALIGN
    assert call(sx=B + 2) == W4_ERR_ALIGN
    assert call(acc=E + 2) == W4_ERR_ALIGN
    assert call(y=E + 2, out=1) == W4_ERR_ALIGN
    assert call(out=2) == W4_ERR_UNSUPPORTED
    big = (1 << 20) + 16
    assert call(d_in=big, ldq=big) == W4_ERR_RANGE
    assert call(M=(1 << 24) + 1) == W4_ERR_RANGE
    # 32-bit buffer offsets: M * ldq and d_out * k_pad / 2 must stay below 2^31
    assert call(M=1 << 22, ldq=1024, d_in=1024) == W4_ERR_RANGE
    assert call(d_out=1 << 22, ldy=1 << 22, d_in=2048, ldq=2048) == W4_ERR_RANGE
    # the grid's thread count: (M / 128) (d_out / 256) 256 < 2^31
    assert call(M=1 << 22, ldq=16, d_in=16, d_out=1 << 20, ldy=1 << 20) == W4_ERR_RANGE
    # any token count: the decode limit of 64 does not apply
    assert call(M=65, q=None) == W4_ERR_NULL


def test_w4a8_linear_rejects_bad_arguments(lib):
    f = lib.w4a8_linear

    def call(**kw):
        a = dict(x=A, M=1, ldx=256, qw=C, sw=D, bias=None, d_out=128, d_in=256, y=E, ldy=128,
                 out=0, sx=None, acc=None)
        a.update(kw)
        return f(a["x"], a["M"], a["ldx"], a["qw"], a["sw"], a["bias"], a["d_out"], a["d_in"],
                 a["y"], a["ldy"], a["out"], a["sx"], a["acc"], None)

    assert call(x=None) == W4_ERR_NULL
    assert call(qw=None) == W4_ERR_NULL
    assert call(sw=None) == W4_ERR_NULL
    assert call(y=None) == W4_ERR_NULL
    assert call(M=0) == W4_ERR_SHAPE
    assert call(M=65) == W4_ERR_UNSUPPORTED
    assert call(d_out=0) == W4_ERR_SHAPE
    assert call(ldx=255) == W4_ERR_SHAPE
    assert call(ldy=127) == W4_ERR_SHAPE
    assert call(ldx=260) == W4_ERR_ALIGN
    assert call(x=A + 8) == W4_ERR_ALIGN
    assert call(sx=B + 2) == W4_ERR_ALIGN
    assert call(acc=B + 2) == W4_ERR_ALIGN
    assert call(out=2) == W4_ERR_UNSUPPORTED
    big = (1 << 20) + 16
    assert call(d_in=big, ldx=big) == W4_ERR_RANGE
    assert call(d_in=65552, ldx=65552) == W4_ERR_RANGE  # W4_DECODE_MAX_D_IN
    # rows longer than the fused kernel's activation stage: the two-call path serves them
    assert call(d_in=60000, ldx=60000) == W4_ERR_UNSUPPORTED


def test_gemv_glu_rejects_bad_arguments(lib):
    f = lib.w4_gemv_glu
    assert _lin(f, x=None) == W4_ERR_NULL
    assert _lin(f, M=0) == W4_ERR_SHAPE
    assert _lin(f, d_out=0) == W4_ERR_SHAPE
    assert _lin(f, ldy=64) == W4_ERR_SHAPE
    assert _lin(f, g=96) == W4_ERR_GROUP
    assert _lin(f, x=A + 8) == W4_ERR_ALIGN
    assert _lin(f, zr=E + 1) == W4_ERR_ALIGN
    # shapes the fused kernel does not serve: more than 4 tokens, 32- and 64-column groups
    assert _lin(f, M=5, g=128) == W4_ERR_UNSUPPORTED
    assert _lin(f, g=32) == W4_ERR_UNSUPPORTED
    assert _lin(f, g=64) == W4_ERR_UNSUPPORTED
