"""int4_weight_only_amd -- Python binding of libw4.so, the MI355X (gfx950) group-wise INT4
weight-only linear layer.

The binding only marshals arguments: it checks tensor dtypes/devices/shapes, allocates outputs
with torch (device memory is torch's), passes raw pointers and the current HIP stream to the C
ABI declared in include/w4.h, and turns a nonzero status into an exception.  Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch fallback: if libw4.so is
missing or cannot be loaded, importing this package raises.

bf16 tensors are passed as torch.bfloat16 (their bits are the uint16 patterns of the ABI).
"""
import ctypes
import os

import torch

__all__ = [
    "W4_SYM", "W4_ASYM", "W4_OUT_BF16", "W4_OUT_F32", "W4Error", "packed_layout", "w4_pack",
    "w4_gemv", "w4_gemv_ws", "w4_gemv_work_bytes", "w4_gemv_glu", "w4_gemm", "act_quant_int8", "w4a8_gemv", "w4a8_gemm", "w4a8_linear",
    "w4_qat_repack", "gptq_hessian", "gptq_factor", "gptq_quantize", "gptq_quantize_noalloc",
    "gptq",
    "w4_linear",
    "library_path",
]

W4_SYM, W4_ASYM = 0, 1
W4_OUT_BF16, W4_OUT_F32 = 0, 1
GEMV_MAX_M = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libw4.so")


class W4Error(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def _load(path):
    if not os.path.exists(path):
        raise ImportError(f"{os.path.basename(path)} not found at {path}; build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'` or "
                          "`python int4_weight_only_amd/build.py`")
    lib = ctypes.CDLL(path)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.w4_packed_layout.argtypes = [i64, i64, i32, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                     ctypes.POINTER(ctypes.c_size_t)]
    lib.w4_pack.argtypes = [p, i64, i64, i64, i32, i32, p, p, p, p]
    lib.w4_qat_repack.argtypes = [p, i64, i64, i64, p, p, p, p]
    lib.w4_gptq_hessian.argtypes = [p, i64, i64, i64, p, p]
    lib.w4_gptq_factor.argtypes = [p, i64, ctypes.c_float, p, p, p, p]
    lib.w4_gptq_quantize.argtypes = [p, i64, i64, i64, p, p, i32, i32, p, p, p, p, p, p]
    lib.w4_gptq_quantize_noalloc.argtypes = [p, i64, i64, i64, p, p, i32, i32, p, p, p, p, p]
    lin = [p, i64, i64, p, p, p, p, i64, i64, i32, p, i64, i32]
    lib.w4_gemv.argtypes = lin + [p]
    lib.w4_gemv_ws.argtypes = lin + [p, ctypes.c_size_t, p]
    lib.w4_gemv_work_bytes.argtypes = [i64, i64, i64, i32]
    lib.w4_gemv_work_bytes.restype = ctypes.c_size_t
    lib.w4_gemv_glu.argtypes = lin + [p]
    lib.w4_gemm.argtypes = lin + [p]
    lib.act_quant_int8.argtypes = [p, i64, i64, i64, p, i64, p, p, p]
    lib.w4a8_gemv.argtypes = [p, p, i64, i64, p, p, p, i64, i64, p, i64, i32, p, p]
    lib.w4a8_gemm.argtypes = lib.w4a8_gemv.argtypes
    lib.w4a8_linear.argtypes = [p, i64, i64, p, p, p, i64, i64, p, i64, i32, p, p, p]
    for f in ("w4_packed_layout", "w4_pack", "w4_qat_repack", "w4_gptq_hessian", "w4_gptq_factor",
              "w4_gptq_quantize", "w4_gptq_quantize_noalloc", "w4_gemv", "w4_gemv_ws",
              "w4_gemv_glu", "w4_gemm",
              "act_quant_int8", "w4a8_gemv", "w4a8_gemm", "w4a8_linear"):
        getattr(lib, f).restype = i32
    lib.w4_status_string.argtypes = [i32]
    lib.w4_status_string.restype = ctypes.c_char_p
    lib.w4_last_hip_error.argtypes = []
    lib.w4_last_hip_error.restype = ctypes.c_char_p
    return lib


_lib = _load(_LIB_PATH)


def library_path():
    return _LIB_PATH


def _select_library(path):
    """Bind every entry point of this module to another build of the library (the tests use the
    build with the kernel-choice hook, libw4_hooks.so); returns the path bound before."""
    global _lib, _LIB_PATH
    prev = _LIB_PATH
    _lib = _load(path)
    _LIB_PATH = path
    return prev


def _check(fn, status):
    if status != 0:
        text = _lib.w4_status_string(status).decode()
        if status == 7:  # W4_ERR_HIP
            text += ": " + _lib.w4_last_hip_error().decode()
        raise W4Error(fn, status, text)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, device=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dims, got {t.dim()}")
    if t.dim() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous along its last dim")


def _check_out_shape(out, rows, cols, name="out"):
    """A caller-supplied output must hold `rows` x `cols` elements at its own row stride: the
    kernels write rows 0 .. rows-1, columns 0 .. cols-1, with ldy = out.stride(0)."""
    if out.shape[0] < rows or out.shape[1] < cols:
        raise ValueError(f"{name} has shape {tuple(out.shape)}, needs at least ({rows}, {cols})")
    if rows > 1 and out.stride(0) < cols:
        raise ValueError(f"{name} rows overlap: stride {out.stride(0)} < {cols} columns")


def _out(out, rows, cols, tdtype, dev):
    if out is None:
        return torch.empty((rows, cols), dtype=tdtype, device=dev)
    _need(out, "out", tdtype, dev, 2)
    _check_out_shape(out, rows, cols)
    return out


def packed_layout(d_out, d_in, group_size):
    """(k_pad, n_groups, qweight_bytes) of the packed format (host-only query)."""
    kp, ng, nb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_size_t()
    _check("w4_packed_layout", _lib.w4_packed_layout(d_out, d_in, group_size, ctypes.byref(kp),
                                                     ctypes.byref(ng), ctypes.byref(nb)))
    return kp.value, ng.value, nb.value


def w4_pack(w, group_size, mode, d_in=None):
    """RTN-pack an fp32 weight [d_out][ldw] (first d_in columns) on the GPU.
    Returns (qweight uint8 [d_out][k_pad/2], scales bf16 [d_out][G], zeros bf16 or None)."""
    _need(w, "w", torch.float32, dim=2)
    d_out, ldw = w.shape
    d_in = ldw if d_in is None else d_in
    k_pad, n_groups, _ = packed_layout(d_out, d_in, group_size)
    dev = w.device
    qweight = torch.empty((d_out, k_pad // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, n_groups), dtype=torch.bfloat16, device=dev)
    zeros = torch.empty_like(scales) if mode == W4_ASYM else None
    _check("w4_pack", _lib.w4_pack(_ptr(w), d_out, d_in, w.stride(0), group_size, mode,
                                   _ptr(qweight), _ptr(scales), _ptr(zeros), _stream(dev)))
    return qweight, scales, zeros


def w4_qat_repack(w, d_in=None, want_m=False):
    """Pack a bf16 weight [d_out][ldw] (first d_in columns) that lies on the 4-bit grid per group
    of 32 columns, keeping its levels (the g32 symmetric format).  Returns (qweight, scales), plus
    m uint8 [d_out][G] (the divisor kept per group, 0 off the grid) when want_m."""
    _need(w, "w", torch.bfloat16, dim=2)
    d_out, ldw = w.shape
    d_in = ldw if d_in is None else d_in
    k_pad, n_groups, _ = packed_layout(d_out, d_in, 32)
    dev = w.device
    qweight = torch.empty((d_out, k_pad // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, n_groups), dtype=torch.bfloat16, device=dev)
    m = torch.empty((d_out, n_groups), dtype=torch.uint8, device=dev) if want_m else None
    _check("w4_qat_repack", _lib.w4_qat_repack(_ptr(w), d_out, d_in, w.stride(0), _ptr(qweight),
                                               _ptr(scales), _ptr(m), _stream(dev)))
    return (qweight, scales, m) if want_m else (qweight, scales)


def gptq_hessian(x, d_in=None):
    """H = (2/N) X^T X, fp32 [d_in][d_in], from bf16 calibration activations x [N][ldx]."""
    _need(x, "x", torch.bfloat16, dim=2)
    N = x.shape[0]
    d_in = x.shape[1] if d_in is None else d_in
    h = torch.empty((d_in, d_in), dtype=torch.float32, device=x.device)
    _check("w4_gptq_hessian", _lib.w4_gptq_hessian(_ptr(x), N, d_in, x.stride(0), _ptr(h),
                                                   _stream(x.device)))
    return h


def gptq_factor(h, alpha=0.01):
    """Dead columns, damping and U with (H + lambda I)^-1 = U^T U.  h fp32 [d_in][d_in] is used as
    the working matrix and destroyed.  Returns (u fp32 [d_in][d_in], dead uint8 [d_in])."""
    _need(h, "h", torch.float32, dim=2)
    d_in = h.shape[0]
    if h.shape[1] != d_in or not h.is_contiguous():
        raise ValueError("h must be a contiguous square matrix")
    u = torch.empty_like(h)
    work = torch.empty_like(h)
    dead = torch.empty((d_in,), dtype=torch.uint8, device=h.device)
    _check("w4_gptq_factor", _lib.w4_gptq_factor(_ptr(h), d_in, float(alpha), _ptr(u), _ptr(work),
                                                 _ptr(dead), _stream(h.device)))
    return u, dead


def gptq_quantize(w, u, dead, group_size, mode, d_in=None):
    """The GPTQ column loop on fp32 weights w [d_out][ldw] (used as the working copy and
    destroyed).  Returns (qweight, scales, zeros or None, row_loss fp32 [d_out])."""
    _need(w, "w", torch.float32, dim=2)
    dev = w.device
    _need(u, "u", torch.float32, dev, 2)
    if dead is not None:
        _need(dead, "dead", torch.uint8, dev, 1)
    d_out, ldw = w.shape
    d_in = ldw if d_in is None else d_in
    if tuple(u.shape) != (d_in, d_in) or not u.is_contiguous():
        raise ValueError(f"u must be contiguous [{d_in}][{d_in}]")
    k_pad, n_groups, _ = packed_layout(d_out, d_in, group_size)
    qweight = torch.empty((d_out, k_pad // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, n_groups), dtype=torch.bfloat16, device=dev)
    zeros = torch.empty_like(scales) if mode == W4_ASYM else None
    work = torch.empty((d_out, 32), dtype=torch.float32, device=dev)
    row_loss = torch.empty((d_out,), dtype=torch.float32, device=dev)
    _check("w4_gptq_quantize", _lib.w4_gptq_quantize(
        _ptr(w), d_out, d_in, w.stride(0), _ptr(u), _ptr(dead), group_size, mode, _ptr(qweight),
        _ptr(scales), _ptr(zeros), _ptr(work), _ptr(row_loss), _stream(dev)))
    return qweight, scales, zeros, row_loss


def gptq_quantize_noalloc(w, u, dead, group_size, mode, d_in=None, row_loss=None, out=None):
    """gptq_quantize for callers that cannot allocate: the block errors live in the library's own
    device array (calls that overlap on one GPU race), and the outputs are the caller's
    out=(qweight, scales, zeros or None) and row_loss (nothing is allocated here either when
    they are given).  Returns (qweight, scales, zeros or None, row_loss or None)."""
    _need(w, "w", torch.float32, dim=2)
    dev = w.device
    _need(u, "u", torch.float32, dev, 2)
    if dead is not None:
        _need(dead, "dead", torch.uint8, dev, 1)
    d_out, ldw = w.shape
    d_in = ldw if d_in is None else d_in
    if tuple(u.shape) != (d_in, d_in) or not u.is_contiguous():
        raise ValueError(f"u must be contiguous [{d_in}][{d_in}]")
    k_pad, n_groups, _ = packed_layout(d_out, d_in, group_size)
    if out is None:
        qweight = torch.empty((d_out, k_pad // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((d_out, n_groups), dtype=torch.bfloat16, device=dev)
        zeros = torch.empty_like(scales) if mode == W4_ASYM else None
    else:
        qweight, scales, zeros = out
        _need(qweight, "qweight", torch.uint8, dev, 2)
        _need(scales, "scales", torch.bfloat16, dev, 2)
        if tuple(qweight.shape) != (d_out, k_pad // 2) or not qweight.is_contiguous():
            raise ValueError(f"qweight must be contiguous [{d_out}][{k_pad // 2}]")
        for name, t in (("scales", scales), ("zeros", zeros)):
            if t is not None and (tuple(t.shape) != (d_out, n_groups) or not t.is_contiguous()):
                raise ValueError(f"{name} must be contiguous [{d_out}][{n_groups}]")
    if row_loss is not None:
        _need(row_loss, "row_loss", torch.float32, dev, 1)
        if row_loss.shape[0] < d_out:
            raise ValueError(f"row_loss must hold {d_out} values")
    _check("w4_gptq_quantize_noalloc", _lib.w4_gptq_quantize_noalloc(
        _ptr(w), d_out, d_in, w.stride(0), _ptr(u), _ptr(dead), group_size, mode, _ptr(qweight),
        _ptr(scales), _ptr(zeros), _ptr(row_loss), _stream(dev)))
    return qweight, scales, zeros, row_loss


def gptq(w, x, group_size, mode, alpha=0.01, d_in=None):
    """GPTQ of fp32 weights w [d_out][>= d_in] with bf16 calibration activations x [N][>= d_in]
    (w is not modified).  Returns (qweight, scales, zeros or None, row_loss)."""
    d_in = w.shape[1] if d_in is None else d_in
    h = gptq_hessian(x, d_in)
    u, dead = gptq_factor(h, alpha)
    return gptq_quantize(w.clone(), u, dead, group_size, mode, d_in)


def _linear(fn_name, x, qweight, scales, zeros, bias, d_in, group_size, out_dtype, out,
            extra=()):
    _need(x, "x", torch.bfloat16, dim=2)
    dev = x.device
    _need(qweight, "qweight", torch.uint8, dev, 2)
    _need(scales, "scales", torch.bfloat16, dev, 2)
    if zeros is not None:
        _need(zeros, "zeros", torch.bfloat16, dev, 2)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, dev, 1)
    M = x.shape[0]
    d_out = qweight.shape[0]
    k_pad, n_groups, _ = packed_layout(d_out, d_in, group_size)
    if tuple(qweight.shape) != (d_out, k_pad // 2) or not qweight.is_contiguous():
        raise ValueError(f"qweight must be contiguous [{d_out}][{k_pad // 2}]")
    for name, t in (("scales", scales), ("zeros", zeros)):
        if t is not None and (tuple(t.shape) != (d_out, n_groups) or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous [{d_out}][{n_groups}]")
    if bias is not None and bias.shape[0] != d_out:
        raise ValueError(f"bias must have {d_out} elements")
    if x.shape[1] < d_in:
        raise ValueError(f"x has {x.shape[1]} columns, fewer than d_in={d_in}")
    tdtype = torch.float32 if out_dtype == W4_OUT_F32 else torch.bfloat16
    out = _out(out, M, d_out, tdtype, dev)
    fn = getattr(_lib, fn_name)
    args = [_ptr(x), M, x.stride(0), _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(bias),
            d_out, d_in, group_size, _ptr(out), out.stride(0), out_dtype]
    _check(fn_name, fn(*args, *extra, _stream(dev)))
    return out


def w4_gemv_work_bytes(M, d_out, d_in, group_size):
    """Bytes of workspace w4_gemv_ws needs for these sizes (0: none)."""
    return int(_lib.w4_gemv_work_bytes(M, d_out, d_in, group_size))


def w4_gemv_ws(x, qweight, scales, zeros, bias, d_in, group_size, out_dtype=W4_OUT_BF16,
               out=None, work=None):
    """w4_gemv with a workspace (a device uint8 tensor of at least w4_gemv_work_bytes bytes; one
    is allocated with torch when work is None): the reduction over d_in split over column slices
    on matrices with few, long rows per compute unit."""
    need = w4_gemv_work_bytes(x.shape[0], qweight.shape[0], d_in, group_size)
    if work is None:
        work = torch.zeros(max(need, 16), dtype=torch.uint8, device=x.device)
    _need(work, "work", torch.uint8, x.device, 1)
    return _linear("w4_gemv_ws", x, qweight, scales, zeros, bias, d_in, group_size, out_dtype,
                   out, extra=(_ptr(work), work.numel()))


def w4_gemv(x, qweight, scales, zeros, bias, d_in, group_size, out_dtype=W4_OUT_BF16, out=None):
    """Decode W4A16 linear, 1 <= M <= 64: y[M][d_out] = x . W_hat^T (+ b)."""
    return _linear("w4_gemv", x, qweight, scales, zeros, bias, d_in, group_size, out_dtype, out)


def w4_gemv_glu(x, qweight, scales, zeros, bias, d_in, group_size, out_dtype=W4_OUT_BF16,
                out=None):
    """Gate/up GEMV with the SiLU(gate) * up epilogue: qweight holds 2 d_ff rows (gate rows, then
    up rows), bias 2 d_ff values or None; returns h [M][d_ff]."""
    _need(x, "x", torch.bfloat16, dim=2)
    dev = x.device
    _need(qweight, "qweight", torch.uint8, dev, 2)
    _need(scales, "scales", torch.bfloat16, dev, 2)
    if zeros is not None:
        _need(zeros, "zeros", torch.bfloat16, dev, 2)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, dev, 1)
    M = x.shape[0]
    rows = qweight.shape[0]
    if rows % 2:
        raise ValueError("a fused gate/up weight has an even number of rows")
    d_ff = rows // 2
    k_pad, n_groups, _ = packed_layout(rows, d_in, group_size)
    if tuple(qweight.shape) != (rows, k_pad // 2) or not qweight.is_contiguous():
        raise ValueError(f"qweight must be contiguous [{rows}][{k_pad // 2}]")
    for name, t in (("scales", scales), ("zeros", zeros)):
        if t is not None and (tuple(t.shape) != (rows, n_groups) or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous [{rows}][{n_groups}]")
    if bias is not None and bias.shape[0] != rows:
        raise ValueError(f"bias must have {rows} elements")
    if x.shape[1] < d_in:
        raise ValueError(f"x has {x.shape[1]} columns, fewer than d_in={d_in}")
    tdtype = torch.float32 if out_dtype == W4_OUT_F32 else torch.bfloat16
    out = _out(out, M, d_ff, tdtype, dev)
    _check("w4_gemv_glu", _lib.w4_gemv_glu(_ptr(x), M, x.stride(0), _ptr(qweight), _ptr(scales),
                                           _ptr(zeros), _ptr(bias), d_ff, d_in, group_size,
                                           _ptr(out), out.stride(0), out_dtype, _stream(dev)))
    return out


def w4_gemm(x, qweight, scales, zeros, bias, d_in, group_size, out_dtype=W4_OUT_BF16, out=None):
    """Prefill W4A16 linear, any M >= 1 (bf16 matrix cores)."""
    return _linear("w4_gemm", x, qweight, scales, zeros, bias, d_in, group_size, out_dtype, out)


def w4_linear(x, qweight, scales, zeros, bias, d_in, group_size, out_dtype=W4_OUT_BF16,
              out=None):
    """Dispatch by token count: the decode kernel for M <= 64, the matrix-core GEMM above."""
    fn = w4_gemv if x.shape[0] <= GEMV_MAX_M else w4_gemm
    return fn(x, qweight, scales, zeros, bias, d_in, group_size, out_dtype, out)


def act_quant_int8(x, K=None, with_sum=True, out=None):
    """Per-token int8 quantization.  Returns (q int8 [M][ldq], s_x fp32 [M], q_sum int32 [M] or
    None); ldq is K rounded up to 16 (columns >= K are left unset).  out=(q, s_x) reuses
    caller tensors of those shapes."""
    _need(x, "x", torch.bfloat16, dim=2)
    M = x.shape[0]
    K = x.shape[1] if K is None else K
    dev = x.device
    ldq = (K + 15) // 16 * 16
    if out is None:
        q = torch.empty((M, ldq), dtype=torch.int8, device=dev)
        s_x = torch.empty((M,), dtype=torch.float32, device=dev)
    else:
        q, s_x = out
        _need(q, "q", torch.int8, dev, 2)
        _need(s_x, "s_x", torch.float32, dev, 1)
        if q.shape[0] != M or q.shape[1] < K or q.stride(1) != 1 or s_x.shape[0] != M:
            raise ValueError("out must be (q [M][>= K] row-major, s_x [M])")
        ldq = q.stride(0)
    q_sum = torch.empty((M,), dtype=torch.int32, device=dev) if with_sum else None
    _check("act_quant_int8", _lib.act_quant_int8(_ptr(x), M, K, x.stride(0), _ptr(q), ldq,
                                                 _ptr(s_x), _ptr(q_sum), _stream(dev)))
    return q, s_x, q_sum


def w4a8_gemv(q, s_x, qweight, s_w, bias, d_in, out_dtype=W4_OUT_BF16, want_acc=False,
              out=None):
    """W4A8 decode linear (M <= 64).  Returns y, or (y, acc int32 [M][d_out]) when want_acc."""
    return _w4a8("w4a8_gemv", q, s_x, qweight, s_w, bias, d_in, out_dtype, want_acc, out)


def w4a8_gemm(q, s_x, qweight, s_w, bias, d_in, out_dtype=W4_OUT_BF16, want_acc=False,
              out=None):
    """W4A8 prefill linear on the int8 matrix cores (any M), the arguments and result of
    w4a8_gemv.  Returns y, or (y, acc int32 [M][d_out]) when want_acc."""
    return _w4a8("w4a8_gemm", q, s_x, qweight, s_w, bias, d_in, out_dtype, want_acc, out)


def _w4a8(name, q, s_x, qweight, s_w, bias, d_in, out_dtype, want_acc, out):
    _need(q, "q", torch.int8, dim=2)
    dev = q.device
    _need(s_x, "s_x", torch.float32, dev, 1)
    _need(qweight, "qweight", torch.uint8, dev, 2)
    s_w = s_w.reshape(-1)
    _need(s_w, "s_w", torch.bfloat16, dev, 1)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, dev, 1)
    M = q.shape[0]
    d_out = qweight.shape[0]
    k_pad, _, _ = packed_layout(d_out, d_in, 0)
    if tuple(qweight.shape) != (d_out, k_pad // 2) or not qweight.is_contiguous():
        raise ValueError(f"qweight must be contiguous [{d_out}][{k_pad // 2}]")
    if s_w.shape[0] != d_out or (bias is not None and bias.shape[0] != d_out):
        raise ValueError(f"s_w and bias must have {d_out} elements")
    if s_x.shape[0] != M or q.shape[1] < d_in:
        raise ValueError("q must be [M][>= d_in] and s_x [M]")
    tdtype = torch.float32 if out_dtype == W4_OUT_F32 else torch.bfloat16
    out = _out(out, M, d_out, tdtype, dev)
    acc = torch.empty((M, d_out), dtype=torch.int32, device=dev) if want_acc else None
    _check(name, getattr(_lib, name)(_ptr(q), _ptr(s_x), M, q.stride(0), _ptr(qweight),
                                     _ptr(s_w), _ptr(bias), d_out, d_in, _ptr(out),
                                     out.stride(0), out_dtype, _ptr(acc), _stream(dev)))
    return (out, acc) if want_acc else out


def w4a8_linear(x, qweight, s_w, bias, d_in, out_dtype=W4_OUT_BF16, want_acc=False,
                want_scales=False, out=None):
    """W4A8 decode linear on bf16 activations, quantized per token inside the kernel (the result
    of act_quant_int8 + w4a8_gemv in one launch).  Returns y, then acc int32 [M][d_out] if
    want_acc, then s_x fp32 [M] if want_scales."""
    _need(x, "x", torch.bfloat16, dim=2)
    dev = x.device
    _need(qweight, "qweight", torch.uint8, dev, 2)
    s_w = s_w.reshape(-1)
    _need(s_w, "s_w", torch.bfloat16, dev, 1)
    if bias is not None:
        _need(bias, "bias", torch.bfloat16, dev, 1)
    M = x.shape[0]
    d_out = qweight.shape[0]
    k_pad, _, _ = packed_layout(d_out, d_in, 0)
    if tuple(qweight.shape) != (d_out, k_pad // 2) or not qweight.is_contiguous():
        raise ValueError(f"qweight must be contiguous [{d_out}][{k_pad // 2}]")
    if s_w.shape[0] != d_out or (bias is not None and bias.shape[0] != d_out):
        raise ValueError(f"s_w and bias must have {d_out} elements")
    if x.shape[1] < d_in:
        raise ValueError(f"x has {x.shape[1]} columns, fewer than d_in={d_in}")
    tdtype = torch.float32 if out_dtype == W4_OUT_F32 else torch.bfloat16
    out = _out(out, M, d_out, tdtype, dev)
    acc = torch.empty((M, d_out), dtype=torch.int32, device=dev) if want_acc else None
    s_x = torch.empty(M, dtype=torch.float32, device=dev) if want_scales else None
    _check("w4a8_linear", _lib.w4a8_linear(_ptr(x), M, x.stride(0), _ptr(qweight), _ptr(s_w),
                                           _ptr(bias), d_out, d_in, _ptr(out), out.stride(0),
                                           out_dtype, _ptr(s_x), _ptr(acc), _stream(dev)))
    res = (out,) + ((acc,) if want_acc else ()) + ((s_x,) if want_scales else ())
    return res if len(res) > 1 else out
