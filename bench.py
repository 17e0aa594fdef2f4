"""Benchmark of the INT4 weight-only linear hot path on one MI355X.

Headline workload (one "step"): the 7B-class MLP decode at M = 1 -- the fused gate/up GEMV
(37888 x 3584) followed by the down GEMV (3584 x 18944), symmetric INT4 with group 128 and 0.1%
weight outliers, bf16 activations and outputs.  `value` is the step's algorithmic bytes (packed
weights + scales + activations + outputs) divided by its time, in GB/s.  Weights are rotated over
distinct copies totalling more than twice the 256 MB Infinity Cache, so they stream from HBM.

Also reported (in "secondary"): the prefill GEMM at M = 2048 (TFLOP/s and MFMA-peak fraction),
the W4A8 decode path, and the 28-layer asymmetric decoder-step linear set at M = 1, 8, 16.

Prints ONE JSON line.  Only --gpus 1 is supported (the library runs on one GPU).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
INT8_MFMA_PEAK_TOPS = 5000.0    # MI355X dense int8 matrix peak, TOP/s
INFINITY_CACHE_BYTES = 256 << 20

METRIC = "W4A16 decode GEMV GB/s & % HBM peak (M=1); prefill GEMM TFLOP/s"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def linear_bytes(M, d_out, d_in, g, asym, out_bytes=2, bias=False, x_bytes=2):
    """Algorithmic bytes of one call: what the method must move."""
    q = 32 if g == 0 else g
    k_pad = (d_in + q - 1) // q * q
    n_groups = 1 if g == 0 else k_pad // g
    b = d_out * k_pad // 2 + d_out * n_groups * 2 * (2 if asym else 1)
    b += M * d_in * x_bytes + M * d_out * out_bytes
    if bias:
        b += d_out * 2
    return b


def source_hash(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the sources of the C2 gate/up GEMV's kernel, of the routing that picks it and of the build
# flags: the committed traffic figure is reported only while their hash matches the one it was
# measured on
TRAFFIC_SOURCES = ("int4_weight_only_amd/csrc/decode_i8.hip",
                   "int4_weight_only_amd/csrc/w4_device.h",
                   "int4_weight_only_amd/csrc/decode.hip",
                   "int4_weight_only_amd/build.py")


# the sources of the C2 down GEMV's kernel (the streaming kernel) and of its routing
DOWN_SOURCES = ("int4_weight_only_amd/csrc/decode_stream.hip",
                "int4_weight_only_amd/csrc/w4_device.h",
                "int4_weight_only_amd/csrc/w4_quant.h",
                "int4_weight_only_amd/csrc/decode.hip",
                "int4_weight_only_amd/build.py")


def load_trace(kernel_key, src_hash):
    """Kernel-trace average duration (us) of a C2 GEMV from the committed rocprofv3 summary, if it
    was measured on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "kernel_trace.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entry = json.load(f).get(kernel_key)
    if not entry or entry.get("source_hash") != src_hash:
        return None
    return entry.get("avg_us")


def load_traffic(kernel_key, src_hash):
    """HBM traffic per launch from the committed PMC summary, if it was measured on the current
    kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(kernel_key)
    if not entry or entry.get("source_hash") != src_hash:
        return None
    return entry.get("bytes_per_launch")


class Timer:
    """HIP events on torch's current stream, which is the stream the library launches on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def start(self, key):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.pairs.setdefault(key, []).append([ev, None])

    def stop(self, key):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.pairs[key][-1][1] = ev

    def mean_ms(self, key):
        v = [a.elapsed_time(b) for a, b in self.pairs.get(key, [])]
        return float(np.mean(v)) if v else float("nan")


def graph_ms(torch, body, launches, replays):
    """Capture `body` (which enqueues `launches` kernel calls through the library) in a HIP graph
    and time `replays` replays with HIP events on the replaying stream; returns ms per launch.
    Graph replay keeps the GPU fed: the Python binding's per-call cost does not enter the
    measured region."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / (replays * launches)
    del g
    return ms


def bench_c2(torch, w4, workloads, steps, warmup, rotate_bytes):
    cfg = workloads.C2
    gu, dn = cfg.linears
    dev = torch.device("cuda", 0)

    def packed(lin, li):
        w = torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev)
        return w4.w4_pack(w, lin.group_size, lin.mode)

    base = [packed(gu, 0), packed(dn, 1)]
    per_copy = sum(t.numel() * t.element_size() for p in base for t in p if t is not None)
    n_copies = max(2, int(np.ceil(rotate_bytes / per_copy)))
    copies = [base]
    for _ in range(n_copies - 1):
        copies.append([tuple(None if t is None else t.clone() for t in p) for p in base])
    x_gu = torch.from_numpy(workloads.linear_x(cfg, 0, 1).view(np.int16)).view(
        torch.bfloat16).to(dev)
    x_dn = torch.from_numpy(workloads.linear_x(cfg, 1, 1).view(np.int16)).view(
        torch.bfloat16).to(dev)
    y_gu = torch.empty((1, gu.d_out), dtype=torch.bfloat16, device=dev)
    y_dn = torch.empty((1, dn.d_out), dtype=torch.bfloat16, device=dev)

    def gate_up(c):
        w4.w4_gemv(x_gu, *c[0], None, gu.d_in, gu.group_size, out=y_gu)

    def down(c):
        w4.w4_gemv(x_dn, *c[1], None, dn.d_in, dn.group_size, out=y_dn)

    def steps_body():
        for c in copies:
            gate_up(c)
            down(c)

    for i in range(warmup):
        c = copies[i % n_copies]
        gate_up(c)
        down(c)
    torch.cuda.synchronize()
    replays = max(1, steps // n_copies)
    # median of 5 repeats of each timing (each repeat: `steps` launches in graph replays)
    med = lambda f: float(np.median([f() for _ in range(5)]))
    step_ms = med(lambda: graph_ms(torch, steps_body, n_copies, replays))
    gu_ms = med(lambda: graph_ms(torch, lambda: [gate_up(c) for c in copies], n_copies, replays))
    dn_ms = med(lambda: graph_ms(torch, lambda: [down(c) for c in copies], n_copies, replays))
    b_gu = linear_bytes(1, gu.d_out, gu.d_in, gu.group_size, False)
    b_dn = linear_bytes(1, dn.d_out, dn.d_in, dn.group_size, False)
    # the same gate/up weights with the SiLU(gate) * up epilogue (w4_gemv_glu): h has d_out / 2
    # values
    h_gu = torch.empty((1, gu.d_out // 2), dtype=torch.bfloat16, device=dev)

    def gate_up_glu(c):
        w4.w4_gemv_glu(x_gu, *c[0], None, gu.d_in, gu.group_size, out=h_gu)

    glu_ms = med(lambda: graph_ms(torch, lambda: [gate_up_glu(c) for c in copies], n_copies,
                                  replays))
    b_glu = b_gu - (gu.d_out // 2) * 2
    return dict(step_ms=step_ms, bytes_step=b_gu + b_dn, gu_ms=gu_ms, dn_ms=dn_ms, b_gu=b_gu,
                b_dn=b_dn, glu_ms=glu_ms, b_glu=b_glu, n_copies=n_copies,
                rotate_mb=n_copies * per_copy / 1e6, steps_timed=replays * n_copies)


def stream_ceilings_gbs(torch, nbytes=1 << 30, reps=20):
    """Measured streaming rates on the same GPU, bytes read + bytes written over the kernel time,
    for a 1 GiB buffer: torch's device copy, and torch's elementwise xor of int32 (the faster of
    torch's plain streaming kernels here; its reductions, read-only, run slower than either)."""
    a = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    out = {}
    for name, fn in (("copy", lambda: b.copy_(a)),
                     ("xor", lambda: torch.bitwise_xor(a, 1, out=b))):
        fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        out[name] = round(2 * nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9, 1)
    del a, b
    return out


def bench_c4(torch, w4, workloads, iters):
    cfg = workloads.C4
    dev = torch.device("cuda", 0)
    M = cfg.tokens[0]
    out = {}
    total_flop, total_ms, w8_ms = 0.0, 0.0, 0.0
    for li, lin in enumerate(cfg.linears):
        w = torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev)
        qw, sc, zr = w4.w4_pack(w, lin.group_size, lin.mode)
        del w
        x = torch.from_numpy(workloads.linear_x(cfg, li, M).view(np.int16)).view(
            torch.bfloat16).to(dev)
        y = torch.empty((M, lin.d_out), dtype=torch.bfloat16, device=dev)
        for _ in range(2):
            w4.w4_gemm(x, qw, sc, zr, None, lin.d_in, lin.group_size, out=y)
        torch.cuda.synchronize()
        timer = Timer(torch)
        for _ in range(iters):
            timer.start(lin.name)
            w4.w4_gemm(x, qw, sc, zr, None, lin.d_in, lin.group_size, out=y)
            timer.stop(lin.name)
        torch.cuda.synchronize()
        ms = timer.mean_ms(lin.name)
        flop = 2.0 * M * lin.d_out * lin.d_in
        total_flop += flop
        total_ms += ms
        out[lin.name] = dict(ms=round(ms, 4), tflops=round(flop / ms / 1e9, 1),
                             mfma_frac=round(flop / ms / 1e9 / BF16_MFMA_PEAK_TFLOPS, 4))
        del qw, sc, zr
        # W4A8 on the same shape: a per-row symmetric pack, act_quant_int8 + w4a8_gemm
        w = torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev)
        qw8, sw8, _ = w4.w4_pack(w, 0, w4.W4_SYM)
        del w
        q, s_x, _ = w4.act_quant_int8(x, lin.d_in, with_sum=False)
        for _ in range(2):
            w4.w4a8_gemm(q, s_x, qw8, sw8, None, lin.d_in, out=y)
        torch.cuda.synchronize()
        for _ in range(iters):
            timer.start("aq")
            w4.act_quant_int8(x, lin.d_in, with_sum=False, out=(q, s_x))
            timer.stop("aq")
            timer.start("w4a8")
            w4.w4a8_gemm(q, s_x, qw8, sw8, None, lin.d_in, out=y)
            timer.stop("w4a8")
        torch.cuda.synchronize()
        g_ms, aq_ms = timer.mean_ms("w4a8"), timer.mean_ms("aq")
        w8_ms += g_ms + aq_ms
        out[lin.name]["w4a8"] = dict(
            gemm_ms=round(g_ms, 4), tops=round(flop / g_ms / 1e9, 1),
            int8_mfma_frac=round(flop / g_ms / 1e9 / INT8_MFMA_PEAK_TOPS, 4),
            act_quant_ms=round(aq_ms, 4), path_ms=round(g_ms + aq_ms, 4))
        # context, not a ceiling of this library's kernels: the vendor GEMMs (hipBLASLt through
        # torch) on dense operands of the same shape, bf16 x bf16 and int8 x int8 (random values,
        # weights column-major), the forms a dequantize-then-GEMM path would call
        wd = torch.randn((lin.d_out, lin.d_in), device=dev, dtype=torch.bfloat16)
        xd = torch.randn((M, lin.d_in), device=dev, dtype=torch.bfloat16)
        qd = torch.randint(-127, 128, (M, lin.d_in), device=dev, dtype=torch.int8)
        wq = torch.randint(-8, 8, (lin.d_out, lin.d_in), device=dev, dtype=torch.int8)
        lib = {}
        for key, fn in (("bf16_tflops", lambda: torch.matmul(xd, wd.t())),
                        ("int8_tops", lambda: torch._int_mm(qd, wq.t()))):
            try:
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                for _ in range(iters):
                    timer.start(key)
                    fn()
                    timer.stop(key)
                torch.cuda.synchronize()
                lib[key] = round(flop / timer.mean_ms(key) / 1e9, 1)
            except RuntimeError:
                lib[key] = None
        out[lin.name]["vendor_gemm_same_shape"] = lib
        del qw8, sw8, q, s_x, x, y, wd, xd, qd, wq
    out["total"] = dict(gflop=round(total_flop / 1e9, 2), ms=round(total_ms, 4),
                        tflops=round(total_flop / total_ms / 1e9, 1),
                        mfma_frac=round(total_flop / total_ms / 1e9 / BF16_MFMA_PEAK_TFLOPS, 4),
                        w4a8_path_ms=round(w8_ms, 4),
                        w4a8_path_tops=round(total_flop / w8_ms / 1e9, 1))
    return out


def bench_c5(torch, w4, workloads, iters):
    cfg = workloads.C5
    dev = torch.device("cuda", 0)
    out = {}
    for li, lin in enumerate(cfg.linears):
        w = torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev)
        base = w4.w4_pack(w, 0, w4.W4_SYM)
        del w
        per_copy = base[0].numel() + base[1].numel() * 2
        n_copies = max(2, int(np.ceil(2 * INFINITY_CACHE_BYTES / per_copy)))
        copies = [base] + [tuple(None if t is None else t.clone() for t in base)
                           for _ in range(n_copies - 1)]
        x = torch.from_numpy(workloads.linear_x(cfg, li, 1).view(np.int16)).view(
            torch.bfloat16).to(dev)
        b = torch.from_numpy(workloads.linear_bias(cfg, li).view(np.int16)).view(
            torch.bfloat16).to(dev)
        y = torch.empty((1, lin.d_out), dtype=torch.bfloat16, device=dev)
        q, s_x, _ = w4.act_quant_int8(x, lin.d_in, with_sum=False)

        def gemvs():
            for c in copies:
                w4.w4a8_gemv(q, s_x, c[0], c[1], b, lin.d_in, out=y)

        def quants():
            for _ in copies:
                w4.act_quant_int8(x, lin.d_in, with_sum=False)

        def fused():  # the quantization folded into the GEMV (w4a8_linear)
            for c in copies:
                w4.w4a8_linear(x, c[0], c[1], b, lin.d_in, out=y)

        gemv_ms = graph_ms(torch, gemvs, n_copies, max(1, iters // n_copies))
        aq_ms = graph_ms(torch, quants, n_copies, max(1, iters // n_copies))
        fused_ms = graph_ms(torch, fused, n_copies, max(1, iters // n_copies))
        gb = linear_bytes(1, lin.d_out, lin.d_in, 0, False, bias=True, x_bytes=1) + 4
        aq_bytes = 2 * lin.d_in + lin.d_in + 4
        fb = linear_bytes(1, lin.d_out, lin.d_in, 0, False, bias=True, x_bytes=2)
        # a few tokens (the int8 matrix-core kernel: the weights read once per 16 tokens)
        few = {}
        for M in (4, 16):
            xm = torch.from_numpy(workloads.linear_x(cfg, li, M).view(np.int16)).view(
                torch.bfloat16).to(dev)
            qm, sm, _ = w4.act_quant_int8(xm, lin.d_in, with_sum=False)
            ym = torch.empty((M, lin.d_out), dtype=torch.bfloat16, device=dev)

            def gemvs_m(qm=qm, sm=sm, ym=ym):
                for c in copies:
                    w4.w4a8_gemv(qm, sm, c[0], c[1], b, lin.d_in, out=ym)

            ms = graph_ms(torch, gemvs_m, n_copies, max(1, iters // n_copies))
            mb = linear_bytes(M, lin.d_out, lin.d_in, 0, False, bias=True, x_bytes=1) + 4 * M
            few[f"M={M}"] = dict(gemv_us=round(ms * 1e3, 2), gemv_gbs=round(mb / ms / 1e6, 1),
                                 gemv_hbm_frac=round(mb / ms / 1e6 / HBM_PEAK_GBS, 4))
        out[f"{lin.d_out}x{lin.d_in}"] = dict(
            gemv_us=round(gemv_ms * 1e3, 2), gemv_gbs=round(gb / gemv_ms / 1e6, 1),
            gemv_hbm_frac=round(gb / gemv_ms / 1e6 / HBM_PEAK_GBS, 4),
            act_quant_us=round(aq_ms * 1e3, 2),
            path_gbs=round((gb + aq_bytes) / (gemv_ms + aq_ms) / 1e6, 1),
            fused_us=round(fused_ms * 1e3, 2), fused_gbs=round(fb / fused_ms / 1e6, 1),
            fused_hbm_frac=round(fb / fused_ms / 1e6 / HBM_PEAK_GBS, 4), few_tokens=few)
        del copies, base
    return out


def bench_qat(torch, w4, workloads, iters):
    """w4_qat_repack on the C4 gate/up shape (37888 x 3584, groups of 32): bf16 weights on the
    4-bit grid, generated on the GPU with a seeded torch generator (timing only; parity of the
    rule at full size is in the GPU tests).  HBM-bound: 2 B read and 0.5 B written per weight,
    plus one bf16 scale per group."""
    lin = workloads.C4.linears[1]
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(workloads.C4.seed)
    G = (lin.d_in + 31) // 32
    steps = torch.exp2(torch.rand((lin.d_out, G, 1), generator=gen, device=dev) * 4 - 10)
    steps = steps.to(torch.bfloat16).float()
    levels = torch.randn((lin.d_out, G, 32), generator=gen, device=dev).mul_(2.5).round_()
    w = (levels.clamp_(-8, 7) * steps).reshape(lin.d_out, G * 32)[:, :lin.d_in]
    w = w.to(torch.bfloat16).contiguous()
    del steps, levels
    for _ in range(2):
        w4.w4_qat_repack(w, lin.d_in)
    torch.cuda.synchronize()
    timer = Timer(torch)
    for _ in range(iters):
        timer.start("qat")
        w4.w4_qat_repack(w, lin.d_in)
        timer.stop("qat")
    torch.cuda.synchronize()
    ms = timer.mean_ms("qat")
    nbytes = 2 * lin.d_out * lin.d_in + lin.d_out * G * 16 + lin.d_out * G * 2
    _, _, m = w4.w4_qat_repack(w, lin.d_in, want_m=True)
    torch.cuda.synchronize()
    on_grid = float((m > 0).float().mean().item())
    del w, m
    return dict(shape=f"{lin.d_out}x{lin.d_in}", us=round(ms * 1e3, 2),
                gbs=round(nbytes / ms / 1e6, 1), hbm_frac=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                groups_on_grid=round(on_grid, 4))


def bench_gptq(torch, w4, workloads, iters):
    """GPTQ on the C4 q/k/v shape (4608 x 3584, g32 symmetric) with 2048 calibration tokens:
    the three calls timed separately (HIP events). Inputs are generated on the GPU with a seeded
    torch generator: N(0, 0.02^2) weights, activations with correlated channels (timing only;
    parity of the path is in the GPU tests)."""
    lin = workloads.C4.linears[0]
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(workloads.C4.seed)
    N = 2048
    w = torch.randn((lin.d_out, lin.d_in), generator=gen, device=dev) * 0.02
    lat = torch.randn((N, lin.d_in // 4), generator=gen, device=dev)
    mix = torch.randn((lin.d_in // 4, lin.d_in), generator=gen, device=dev) / 2
    x = (lat @ mix + 0.3 * torch.randn((N, lin.d_in), generator=gen, device=dev))
    x = x.to(torch.bfloat16).contiguous()
    del lat, mix
    timer = Timer(torch)
    for it in range(iters + 1):
        key = "warm" if it == 0 else ""
        timer.start("h" + key)
        h = w4.gptq_hessian(x, lin.d_in)
        timer.stop("h" + key)
        timer.start("f" + key)
        u, dead = w4.gptq_factor(h, 0.01)
        timer.stop("f" + key)
        wc = w.clone()
        timer.start("q" + key)
        w4.gptq_quantize(wc, u, dead, 32, w4.W4_SYM)
        timer.stop("q" + key)
    torch.cuda.synchronize()
    h_ms, f_ms, q_ms = timer.mean_ms("h"), timer.mean_ms("f"), timer.mean_ms("q")
    flop_h = 2.0 * N * lin.d_in * lin.d_in
    return dict(shape=f"{lin.d_out}x{lin.d_in}", calib_tokens=N, hessian_ms=round(h_ms, 3),
                hessian_tflops=round(flop_h / h_ms / 1e9, 1), factor_ms=round(f_ms, 3),
                quantize_ms=round(q_ms, 3), total_ms=round(h_ms + f_ms + q_ms, 3))


def bench_c1(torch, w4, workloads, replays=20, calls=50):
    """The tiny linear (128 x 256, g32 symmetric) at M = 1 and 4: the time of one call among
    `calls` back-to-back calls in a HIP graph (kernel time plus the gap between graph nodes),
    through w4_gemv and, at M = 4, also w4_gemm."""
    cfg = workloads.C1
    lin = cfg.linears[0]
    dev = torch.device("cuda", 0)
    w = torch.from_numpy(workloads.linear_weight(cfg, 0)).to(dev)
    qw, sc, zr = w4.w4_pack(w, lin.group_size, lin.mode)
    out = {}
    for M in cfg.tokens:
        x = torch.from_numpy(workloads.linear_x(cfg, 0, M).view(np.int16)).view(
            torch.bfloat16).to(dev)
        y = torch.empty((M, lin.d_out), dtype=torch.bfloat16, device=dev)
        def gemv():
            for _ in range(calls):
                w4.w4_gemv(x, qw, sc, zr, None, lin.d_in, lin.group_size, out=y)

        def gemm():
            for _ in range(calls):
                w4.w4_gemm(x, qw, sc, zr, None, lin.d_in, lin.group_size, out=y)

        r = dict(gemv_us=round(graph_ms(torch, gemv, calls, replays) * 1e3, 2))
        if M > 1:
            r["gemm_us"] = round(graph_ms(torch, gemm, calls, replays) * 1e3, 2)
        out[f"M={M}"] = r
    return out


def bench_c3(torch, w4, workloads, iters):
    """28 layers x {qkv, o, gate/up, down}, asymmetric g128, weights generated on the GPU with a
    seeded torch generator (timing only; parity of these shapes is in the GPU tests)."""
    cfg = workloads.C3
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    layers = []
    for _ in range(cfg.repeat_layers):
        packs = []
        for lin in cfg.linears:
            w = torch.randn((lin.d_out, lin.d_in), generator=gen, device=dev) * workloads.W_SIGMA
            packs.append(w4.w4_pack(w, lin.group_size, lin.mode))
            del w
        layers.append(packs)
    out = {}
    for M in cfg.tokens:
        xs = [torch.randn((M, lin.d_in), generator=gen, device=dev).to(torch.bfloat16)
              for lin in cfg.linears]
        ys = [torch.empty((M, lin.d_out), dtype=torch.bfloat16, device=dev)
              for lin in cfg.linears]
        # one workspace for every call of the step (the calls are ordered on one stream): the
        # library splits the reduction over column slices on the few-row matrices at M >= 2
        need = max(w4.w4_gemv_work_bytes(M, l.d_out, l.d_in, l.group_size) for l in cfg.linears)
        work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def step():
            for packs in layers:
                for lin, p, x, y in zip(cfg.linears, packs, xs, ys):
                    w4.w4_gemv_ws(x, *p, None, lin.d_in, lin.group_size, out=y, work=work)

        def step_no_workspace():
            for packs in layers:
                for lin, p, x, y in zip(cfg.linears, packs, xs, ys):
                    w4.w4_gemv(x, *p, None, lin.d_in, lin.group_size, out=y)

        ms = graph_ms(torch, step, 1, iters)
        ms_nows = graph_ms(torch, step_no_workspace, 1, iters) if need > 0 else ms
        nbytes = cfg.repeat_layers * sum(linear_bytes(M, l.d_out, l.d_in, l.group_size, True)
                                         for l in cfg.linears)
        # each linear alone (its 28 launches in one graph): per-call time and rate; their sum
        # next to the whole step's time shows what the back-to-back launches cost or save
        per_lin = {}
        for k, lin in enumerate(cfg.linears):
            def one(k=k, lin=lin):
                for packs in layers:
                    w4.w4_gemv_ws(xs[k], *packs[k], None, lin.d_in, lin.group_size, out=ys[k],
                                  work=work)
            lms = graph_ms(torch, one, cfg.repeat_layers, iters)
            lb = linear_bytes(M, lin.d_out, lin.d_in, lin.group_size, True)
            per_lin[lin.name] = dict(us=round(lms * 1e3, 2), gbs=round(lb / lms / 1e6, 1),
                                     hbm_frac=round(lb / lms / 1e6 / HBM_PEAK_GBS, 4))
        sum_us = cfg.repeat_layers * sum(v["us"] for v in per_lin.values())
        out[f"M={M}"] = dict(step_us=round(ms * 1e3, 1), gbs=round(nbytes / ms / 1e6, 1),
                             hbm_frac=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                             sum_of_linears_us=round(sum_us, 1), linears=per_lin,
                             step_us_without_workspace=round(ms_nows * 1e3, 1),
                             workspace_bytes=int(need))
    del layers
    return out


def bench_decode_g32(torch, w4, workloads, iters):
    """Decode at 1, 8 and 16 tokens on the C4 shapes with 32-column symmetric groups (the format
    the QAT page's repack produces), each linear over rotated weight copies in one HIP graph:
    per-call time and rate (timing only; parity of g32 decode is in the GPU tests)."""
    cfg = workloads.C4
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed + 32)
    copies = 6
    out = {}
    for lin in cfg.linears:
        packs = []
        for _ in range(copies):
            w = torch.randn((lin.d_out, lin.d_in), generator=gen, device=dev) * workloads.W_SIGMA
            packs.append(w4.w4_pack(w, lin.group_size, lin.mode))
            del w
        r = {}
        for M in (1, 8, 16):
            x = torch.randn((M, lin.d_in), generator=gen, device=dev).to(torch.bfloat16)
            y = torch.empty((M, lin.d_out), dtype=torch.bfloat16, device=dev)
            need = w4.w4_gemv_work_bytes(M, lin.d_out, lin.d_in, lin.group_size)
            work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

            def body(x=x, y=y, work=work):
                for p in packs:
                    w4.w4_gemv_ws(x, *p, None, lin.d_in, lin.group_size, out=y, work=work)

            ms = graph_ms(torch, body, copies, iters)
            b = linear_bytes(M, lin.d_out, lin.d_in, lin.group_size, False)
            r[f"M={M}"] = dict(us=round(ms * 1e3, 2), gbs=round(b / ms / 1e6, 1),
                               hbm_frac=round(b / ms / 1e6 / HBM_PEAK_GBS, 4))
        out[f"{lin.name} {lin.d_out}x{lin.d_in}"] = r
        del packs
    return out


def host_cpu():
    """The host's CPU model (from /proc/cpuinfo) and logical CPU count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(model=model, logical_cpus=os.cpu_count())


def _oracle_rate(fn, budget_s, max_calls=100000):
    """(calls, seconds) of repeated calls of fn within about budget_s (at least one call)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= max_calls:
            return n, el


def cpu_baseline(workloads, budget_s):
    """The oracle, as it stands, on the host's cores: the C2 step (M = 1) with all threads (the
    headline baseline), then every other config on a bounded sample, with all threads and, for
    C1, C2 and C5, with one thread."""
    import oracle
    threads = oracle.max_threads()
    per = {}

    # C2: the headline (the whole decode step, all threads), then one thread
    cfg = workloads.C2
    packs, xs = [], []
    for li, lin in enumerate(cfg.linears):
        w = workloads.linear_weight(cfg, li)
        packs.append(oracle.pack(w, lin.group_size, lin.mode))
        xs.append(workloads.linear_x(cfg, li, 1))
        del w
    nbytes = sum(linear_bytes(1, l.d_out, l.d_in, l.group_size, False) for l in cfg.linears)

    def c2_step():
        for (qw, sc, zr), x, lin in zip(packs, xs, cfg.linears):
            oracle.w4a16(x, qw, sc, zr, None, lin.d_in, lin.group_size)

    n, el = _oracle_rate(c2_step, 0.5 * budget_s, 2000)
    head = dict(value=round(nbytes * n / el / 1e9, 3), unit="GB/s", cores=threads, kind="oracle",
                sample=f"{n} full C2 decode steps (gate/up 37888x3584 + down 3584x18944, M=1) "
                       f"in {el:.1f} s, fp64 oracle with OpenMP over output rows")
    oracle.set_num_threads(1)
    n1, el1 = _oracle_rate(c2_step, 0.1 * budget_s, 100)
    oracle.set_num_threads(threads)
    per["C2"] = dict(step_ms=round(el / n * 1e3, 2), gbs=head["value"],
                     step_ms_1thread=round(el1 / n1 * 1e3, 2),
                     gbs_1thread=round(nbytes * n1 / el1 / 1e9, 3))
    del packs, xs

    # C1: the tiny linear at M = 1 and 4
    cfg = workloads.C1
    lin = cfg.linears[0]
    qw, sc, zr = oracle.pack(workloads.linear_weight(cfg, 0), lin.group_size, lin.mode)
    c1 = {}
    for M in cfg.tokens:
        x = workloads.linear_x(cfg, 0, M)
        fn = lambda: oracle.w4a16(x, qw, sc, zr, None, lin.d_in, lin.group_size)
        n, el = _oracle_rate(fn, 0.02 * budget_s)
        oracle.set_num_threads(1)
        n1, el1 = _oracle_rate(fn, 0.02 * budget_s)
        oracle.set_num_threads(threads)
        c1[f"M={M}"] = dict(us=round(el / n * 1e6, 2), us_1thread=round(el1 / n1 * 1e6, 2))
    per["C1"] = c1

    # C3: one layer's four linears (asymmetric g128) at M = 1 and 8, scaled to the 28 layers
    cfg = workloads.C3
    packs = [oracle.pack(workloads.linear_weight(cfg, li), l.group_size, l.mode)
             for li, l in enumerate(cfg.linears)]
    c3 = {}
    for M in (1, 8):
        xs = [workloads.linear_x(cfg, li, M) for li in range(len(cfg.linears))]

        def layer():
            for (qw, sc, zr), x, l in zip(packs, xs, cfg.linears):
                oracle.w4a16(x, qw, sc, zr, None, l.d_in, l.group_size)

        n, el = _oracle_rate(layer, 0.05 * budget_s, 50)
        layer_bytes = sum(linear_bytes(M, l.d_out, l.d_in, l.group_size, True)
                          for l in cfg.linears)
        c3[f"M={M}"] = dict(layer_ms=round(el / n * 1e3, 2),
                            step_ms_28_layers=round(el / n * 1e3 * cfg.repeat_layers, 1),
                            gbs=round(layer_bytes * n / el / 1e9, 3))
    c3["sample"] = "layer 0's four linears, timed whole; the 28-layer step is 28 x that"
    per["C3"] = c3
    del packs

    # C4: 16 of the 2048 tokens through each full weight (all rows), as GFLOP/s; the full
    # config's time at that rate
    cfg = workloads.C4
    c4, flop_all, t_all = {}, 0.0, 0.0
    for li, l in enumerate(cfg.linears):
        qw, sc, zr = oracle.pack(workloads.linear_weight(cfg, li), l.group_size, l.mode)
        x = workloads.linear_x(cfg, li, 16)
        n, el = _oracle_rate(lambda: oracle.w4a16(x, qw, sc, zr, None, l.d_in, l.group_size),
                             0.04 * budget_s, 20)
        rate = 2.0 * 16 * l.d_out * l.d_in * n / el
        c4[l.name] = dict(gflops=round(rate / 1e9, 2))
        flop = 2.0 * cfg.tokens[0] * l.d_out * l.d_in
        flop_all += flop
        t_all += flop / rate
        del qw, sc, zr
    c4["full_config_s_at_that_rate"] = round(t_all, 1)
    c4["gflops"] = round(flop_all / t_all / 1e9, 2)
    c4["sample"] = "16 of the 2048 tokens against all rows of each weight, fp64"
    per["C4"] = c4

    # C5: act_quant + W4A8 GEMV (per-row symmetric), M = 1, both shapes
    cfg = workloads.C5
    c5 = {}
    for li, l in enumerate(cfg.linears):
        qw, sw, _ = oracle.pack(workloads.linear_weight(cfg, li), 0, oracle.SYM)
        x = workloads.linear_x(cfg, li, 1)
        b = workloads.linear_bias(cfg, li)

        def path():
            q, s_x, _ = oracle.act_quant(x)
            oracle.w4a8(q, s_x, qw, sw, b, l.d_in)

        n, el = _oracle_rate(path, 0.04 * budget_s, 200)
        oracle.set_num_threads(1)
        n1, el1 = _oracle_rate(path, 0.02 * budget_s, 50)
        oracle.set_num_threads(threads)
        gb = linear_bytes(1, l.d_out, l.d_in, 0, False, bias=True, x_bytes=2)
        c5[f"{l.d_out}x{l.d_in}"] = dict(us=round(el / n * 1e6, 1),
                                         us_1thread=round(el1 / n1 * 1e6, 1),
                                         gbs=round(gb * n / el / 1e9, 3))
    per["C5"] = c5
    head["per_config"] = per
    head["host_cpu"] = host_cpu()
    return head


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--only", choices=["c1", "c2", "c3", "c4", "c5", "qat", "gptq", "g32"],
                    default=None,
                    help="time one workload only (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch

    import int4_weight_only_amd as w4
    import workloads

    torch.cuda.set_device(0)
    log("device", torch.cuda.get_device_name(0), "lib", w4.library_path())
    rotate = 2 * INFINITY_CACHE_BYTES + (64 << 20)

    secondary = {}
    if args.only in (None, "c2"):
        log("C2 decode step")
        r = bench_c2(torch, w4, workloads, args.steps, args.warmup, rotate)
    if args.only is not None:
        if args.only == "c1":
            secondary["C1_tiny"] = bench_c1(torch, w4, workloads)
        elif args.only == "c3":
            secondary["C3_decoder_step"] = bench_c3(torch, w4, workloads, 5)
        elif args.only == "c4":
            secondary["C4_prefill_gemm"] = bench_c4(torch, w4, workloads, 10)
        elif args.only == "c5":
            secondary["C5_w4a8"] = bench_c5(torch, w4, workloads, 100)
        elif args.only == "qat":
            secondary["qat_repack"] = bench_qat(torch, w4, workloads, 10)
        elif args.only == "gptq":
            secondary["gptq"] = bench_gptq(torch, w4, workloads, 3)
        elif args.only == "g32":
            secondary["decode_g32"] = bench_decode_g32(torch, w4, workloads, 10)
        if args.only != "c2":
            print(json.dumps(secondary), flush=True)
            return
    if not args.no_secondary and args.only is None:
        log("C1 tiny linear")
        secondary["C1_tiny"] = bench_c1(torch, w4, workloads)
        log("C4 prefill GEMM")
        secondary["C4_prefill_gemm"] = bench_c4(torch, w4, workloads, 10)
        log("C5 W4A8")
        secondary["C5_w4a8"] = bench_c5(torch, w4, workloads, 100)
        log("C3 decoder step")
        secondary["C3_decoder_step"] = bench_c3(torch, w4, workloads, 5)
        log("decode with 32-column groups")
        secondary["decode_g32"] = bench_decode_g32(torch, w4, workloads, 10)
        log("QAT repack")
        secondary["qat_repack"] = bench_qat(torch, w4, workloads, 10)
        log("GPTQ")
        secondary["gptq"] = bench_gptq(torch, w4, workloads, 3)

    secondary["C2_gate_up_silu_mul"] = dict(
        us=round(r["glu_ms"] * 1e3, 3), gbs=round(r["b_glu"] / r["glu_ms"] / 1e6, 1),
        hbm_frac=round(r["b_glu"] / r["glu_ms"] / 1e6 / HBM_PEAK_GBS, 4),
        plain_gate_up_us=round(r["gu_ms"] * 1e3, 3))
    value = r["bytes_step"] / r["step_ms"] / 1e6
    gu_gbs = r["b_gu"] / r["gu_ms"] / 1e6
    src = source_hash(*TRAFFIC_SOURCES)
    tr_gu = load_trace("gemv_c2_gate_up", src)
    tr_dn = load_trace("gemv_c2_down", source_hash(*DOWN_SOURCES))
    roofline = {
        "bound": "hbm",
        "kernel": "gemv_i8_kernel (C2 gate/up 37888x3584, M=1)",
        "achieved": round(gu_gbs, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
        "traffic": load_traffic("gemv_c2_gate_up", src),
        "algorithmic_bytes": r["b_gu"],
        "avg_launch_us": round(r["gu_ms"] * 1e3, 3),
        # the same kernel's average duration in the committed kernel trace (profiles/
        # kernel_trace.json, while its sources are unchanged) and the fraction it gives
        "trace_avg_launch_us": tr_gu,
        "frac_trace": round(r["b_gu"] / tr_gu / 1e3 / HBM_PEAK_GBS, 4) if tr_gu else None,
        "down_trace_avg_launch_us": tr_dn,
        "down_frac_trace": (round(r["b_dn"] / tr_dn / 1e3 / HBM_PEAK_GBS, 4)
                            if tr_dn else None),
        "down_avg_launch_us": round(r["dn_ms"] * 1e3, 3),
        "down_gbs": round(r["b_dn"] / r["dn_ms"] / 1e6, 1),
        **{f"stream_{k}_gbs": v for k, v in stream_ceilings_gbs(torch).items()},
    }
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8 x u4 -> i32 (gate/up: bf16 x as exact integer digits on MFMA), "
                 "f16 x f16 -> f32 (down); fp32 scaling",
        "data": "synthetic",
        "config": {
            "workload": "C2 MLP decode step at M=1: gate/up GEMV 37888x3584 + down GEMV "
                        "3584x18944, symmetric INT4 g128, 0.1% weight outliers, bf16 out",
            "tokens": 1,
            "bytes_per_step": r["bytes_step"],
            "weight_copies_rotated": r["n_copies"],
            "timing": "HIP graph replays of the library launches, HIP events on the stream",
            "rotated_mb": round(r["rotate_mb"], 1),
            "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        },
        "roofline": roofline,
    }
    if not args.no_cpu_baseline and args.only is None:
        log("CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(workloads, args.cpu_budget_s)
    if secondary:
        line["secondary"] = secondary
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
