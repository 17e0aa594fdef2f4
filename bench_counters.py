"""Hardware counters of the library's kernels, per workload, with rocprofv3 (one MI355X).

Each counter pass is a run of its own (rocprofv3 does not split counters over passes):

    rocprofv3 --kernel-trace --pmc VALUBusy MfmaUtil SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS \
        SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD --output-format csv -d <dir_sq> -o pmc \
        -- python3 bench_counters.py run <workload>
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o pmc -- python3 bench_counters.py run <workload>
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o pmc -- python3 bench_counters.py run <workload>
    python3 bench_counters.py summarize <workload> <dir_sq>/pmc_counter_collection.csv \
        <dir_sq>/pmc_kernel_trace.csv <dir_f>/pmc_counter_collection.csv <dir_w>/pmc_counter_collection.csv

Workloads: c2 (the decode step's gate/up and down GEMVs at M = 1, and the gate/up GEMV with the
SiLU * up epilogue), c3 (one decoder layer's four linears at M = 1, 8, 16, through w4_gemv_ws as
the bench calls them), c4 (the prefill GEMMs, W4A16 and W4A8, M = 2048), c5 (act_quant_int8 and
the W4A8 GEMV at one token, the fused W4A8 linear, act_quant_int8 and the W4A8 GEMV at 16 tokens).

`run` first copies a 256 MiB device buffer (known bytes: the calibration of FETCH_SIZE and
WRITE_SIZE, whose units this part counts differently), then launches each labelled call of the
workload REPS times in a row over rotated weight copies (so that weights come from HBM, not the
256 MB Infinity Cache), with a small torch fill between labels: the library's dispatches of a label
form one run, in the order of LABELS. `summarize` averages every counter per dispatch of each
label and derives:
  * VALU lane-operations per weight = SQ_INSTS_VALU * 64 / (d_out * d_in) (the plain-ALU budget
    at 70% of 8 TB/s is 3.5 per 4-bit weight: 64 lanes x 4 SIMDs per CU, 2.4 GHz);
  * VALUBusy and MfmaUtil (rocprofv3's own formulas);
  * the kernel-trace duration, and from it the algorithmic GB/s (or TFLOP/s);
  * calibrated HBM bytes per dispatch against the algorithmic bytes.
The summary is printed as a markdown table (profiles/ keeps it with this command line).

    python3 bench_counters.py trace <dir>/run_kernel_stats.csv

records the kernel-trace averages of the C2 GEMVs from `rocprofv3 --kernel-trace --stats --
python3 bench.py --only c2 ...` in profiles/kernel_trace.json (bench.py's trace-based fraction).
"""
import csv
import json
import os
import sys
from collections import OrderedDict, defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20
CALIB_COPIES = 4
REPS = 12
SQ_COUNTERS = ["VALUBusy", "MfmaUtil", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_VMEM_RD"]


def _labels(workload):
    """(label, d_out, d_in, M, algorithmic bytes, flops) of the calls `run` makes, in order."""
    import workloads
    from bench import linear_bytes

    out = []
    if workload == "c2":
        gu, dn = workloads.C2.linears
        out.append(("gate/up GEMV 37888x3584", gu.d_out, gu.d_in, 1,
                    linear_bytes(1, gu.d_out, gu.d_in, gu.group_size, False), 0))
        out.append(("down GEMV 3584x18944", dn.d_out, dn.d_in, 1,
                    linear_bytes(1, dn.d_out, dn.d_in, dn.group_size, False), 0))
        out.append(("gate/up GEMV + SiLU*up", gu.d_out, gu.d_in, 1,
                    linear_bytes(1, gu.d_out, gu.d_in, gu.group_size, False) - gu.d_out, 0))
    elif workload == "c3":
        for M in (1, 8, 16):
            for lin in workloads.C3.linears:
                out.append((f"{lin.name} M={M}", lin.d_out, lin.d_in, M,
                            linear_bytes(M, lin.d_out, lin.d_in, lin.group_size, True), 0))
    elif workload == "c4":
        M = workloads.C4.tokens[0]
        for lin in workloads.C4.linears:
            out.append((f"W4A16 GEMM {lin.name}", lin.d_out, lin.d_in, M, 0,
                        2 * M * lin.d_out * lin.d_in))
        for lin in workloads.C4.linears:
            out.append((f"act_quant {lin.name}", 0, lin.d_in, M, 3 * M * lin.d_in, 0))
            out.append((f"W4A8 GEMM {lin.name}", lin.d_out, lin.d_in, M, 0,
                        2 * M * lin.d_out * lin.d_in))
    elif workload == "c5":
        for lin in workloads.C5.linears:
            k32 = (lin.d_in + 31) // 32 * 32
            b = lin.d_out * k32 // 2 + 2 * lin.d_out + lin.d_in + 4 + 2 * lin.d_out + 2 * lin.d_out
            out.append((f"act_quant {lin.name}", 0, lin.d_in, 1, 3 * lin.d_in, 0))
            out.append((f"w4a8_gemv {lin.name}", lin.d_out, lin.d_in, 1, b, 0))
            out.append((f"w4a8_linear {lin.name}", lin.d_out, lin.d_in, 1, b + lin.d_in, 0))
            b16 = (lin.d_out * k32 // 2 + 2 * lin.d_out + 16 * (lin.d_in + 4) + 2 * lin.d_out
                   + 16 * 2 * lin.d_out)
            out.append((f"act_quant M=16 {lin.name}", 0, lin.d_in, 16, 16 * 3 * lin.d_in, 0))
            out.append((f"w4a8_gemv M=16 {lin.name}", lin.d_out, lin.d_in, 16, b16, 0))
    else:
        raise SystemExit(f"unknown workload {workload}")
    return out


def run(workload):
    import numpy as np
    import torch

    import int4_weight_only_amd as w4
    import workloads
    from bench import INFINITY_CACHE_BYTES

    dev = torch.device("cuda", 0)
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(3)
    for _ in range(CALIB_COPIES):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    rotate = 2 * INFINITY_CACHE_BYTES + (64 << 20)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    def copies_of(packed):
        per = sum(t.numel() * t.element_size() for t in packed if t is not None)
        n = max(2, -(-rotate // per))
        return [packed] + [tuple(None if t is None else t.clone() for t in packed)
                           for _ in range(n - 1)]

    def separator():
        torch.cuda.synchronize()
        torch.zeros(16, device=dev)  # a torch kernel between two labels' dispatches
        torch.cuda.synchronize()

    def repeat(fn, cps):
        for i in range(REPS):
            fn(cps[i % len(cps)])
        separator()

    if workload == "c2":
        cfg = workloads.C2
        gu, dn = cfg.linears
        pg = copies_of(w4.w4_pack(torch.from_numpy(workloads.linear_weight(cfg, 0)).to(dev),
                                  gu.group_size, gu.mode))
        pd = copies_of(w4.w4_pack(torch.from_numpy(workloads.linear_weight(cfg, 1)).to(dev),
                                  dn.group_size, dn.mode))
        xg, xd = bf16(workloads.linear_x(cfg, 0, 1)), bf16(workloads.linear_x(cfg, 1, 1))
        separator()
        repeat(lambda c: w4.w4_gemv(xg, *c, None, gu.d_in, gu.group_size), pg)
        repeat(lambda c: w4.w4_gemv(xd, *c, None, dn.d_in, dn.group_size), pd)
        repeat(lambda c: w4.w4_gemv_glu(xg, *c, None, gu.d_in, gu.group_size), pg)
    elif workload == "c3":
        cfg = workloads.C3
        packs = [copies_of(w4.w4_pack(torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev),
                                      lin.group_size, lin.mode))
                 for li, lin in enumerate(cfg.linears)]
        separator()
        for M in (1, 8, 16):
            # the bench's calls: w4_gemv_ws with one workspace (the column split where it applies)
            need = max(w4.w4_gemv_work_bytes(M, l.d_out, l.d_in, l.group_size) for l in cfg.linears)
            work = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            for li, lin in enumerate(cfg.linears):
                x = bf16(workloads.linear_x(cfg, li, M))
                repeat(lambda c: w4.w4_gemv_ws(x, *c, None, lin.d_in, lin.group_size, work=work),
                       packs[li])
    elif workload == "c4":
        cfg = workloads.C4
        M = cfg.tokens[0]
        xs = [bf16(workloads.linear_x(cfg, li, M)) for li in range(len(cfg.linears))]
        p16 = [w4.w4_pack(torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev),
                          lin.group_size, lin.mode) for li, lin in enumerate(cfg.linears)]
        p8 = [w4.w4_pack(torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev), 0, w4.W4_SYM)
              for li, lin in enumerate(cfg.linears)]
        separator()
        for li, lin in enumerate(cfg.linears):
            repeat(lambda c: w4.w4_gemm(xs[li], *c, None, lin.d_in, lin.group_size), [p16[li]])
        for li, lin in enumerate(cfg.linears):
            q, s, _ = w4.act_quant_int8(xs[li], with_sum=False)
            repeat(lambda c: w4.act_quant_int8(xs[li], with_sum=False, out=(q, s)), [None])
            repeat(lambda c: w4.w4a8_gemm(q, s, c[0], c[1], None, lin.d_in), [p8[li]])
    elif workload == "c5":
        cfg = workloads.C5
        for li, lin in enumerate(cfg.linears):
            pk = copies_of(w4.w4_pack(torch.from_numpy(workloads.linear_weight(cfg, li)).to(dev),
                                      lin.group_size, lin.mode))
            x = bf16(workloads.linear_x(cfg, li, 1))
            x16 = bf16(workloads.linear_x(cfg, li, 16))  # 16 tokens: the int8 matrix-core kernel
            bias = bf16(workloads.linear_bias(cfg, li))
            ldq = (lin.d_in + 15) // 16 * 16
            q = torch.empty((1, ldq), dtype=torch.int8, device=dev)
            s = torch.empty((1,), dtype=torch.float32, device=dev)
            q16 = torch.empty((16, ldq), dtype=torch.int8, device=dev)
            s16 = torch.empty((16,), dtype=torch.float32, device=dev)
            separator()
            repeat(lambda c: w4.act_quant_int8(x, with_sum=False, out=(q, s)), [None])
            repeat(lambda c: w4.w4a8_gemv(q, s, c[0], c[1], bias, lin.d_in), pk)
            repeat(lambda c: w4.w4a8_linear(x, c[0], c[1], bias, lin.d_in), pk)
            repeat(lambda c: w4.act_quant_int8(x16, with_sum=False, out=(q16, s16)), [None])
            repeat(lambda c: w4.w4a8_gemv(q16, s16, c[0], c[1], bias, lin.d_in), pk)
    else:
        raise SystemExit(f"unknown workload {workload}")
    torch.cuda.synchronize()
    print(f"ran {workload}: {len(_labels(workload))} labels x {REPS} calls", flush=True)


def _read(path, value_field="Counter_Value"):
    with open(path) as f:
        return list(csv.DictReader(f))


def _runs(rows, name_field):
    """Consecutive runs of the library's dispatches (kernel names in namespace w4, the set-up
    packs left out), split by any other dispatch; returns [([kernel names in order of first
    dispatch], [dispatch ids])]. A call that launches two kernels (the column-split GEMV and its
    reduction) puts both in its label's run."""
    order = sorted({(int(r["Dispatch_Id"]), r[name_field]) for r in rows})
    runs, cur = [], None
    for did, name in order:
        if "w4::" in name and "pack_kernel" not in name:  # (the set-up packs are not timed)
            if cur is None:
                cur = ([name], [did])
            else:
                if name not in cur[0]:
                    cur[0].append(name)
                cur[1].append(did)
        elif cur is not None:
            runs.append(cur)
            cur = None
    if cur is not None:
        runs.append(cur)
    return runs


def _copy_mean(rows, counter):
    vals = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                  if r["Counter_Name"] == counter and "copybuffer" in r["Kernel_Name"].lower())
    vals = [v for _, v in vals][:CALIB_COPIES]
    return sum(vals) / len(vals) if vals else None


def summarize(workload, sq_csv, trace_csv, fetch_csv, write_csv):
    labels = _labels(workload)
    per = OrderedDict((lab[0], defaultdict(list)) for lab in labels)
    for path in (sq_csv, fetch_csv, write_csv):
        rows = _read(path)
        runs = _runs(rows, "Kernel_Name")
        if len(runs) != len(labels):
            raise SystemExit(f"{path}: {len(runs)} dispatch runs for {len(labels)} labels")
        by_id = defaultdict(dict)
        for r in rows:
            by_id[int(r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
        for (lab, *_), (knames, ids) in zip(labels, runs):
            per[lab]["kernel"] = knames
            for did in ids:
                for c, v in by_id[did].items():
                    per[lab][c].append(v)
    trace = _read(trace_csv)
    truns = _runs(trace, "Kernel_Name")
    dur = {}
    by_tid = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
              for r in trace}
    wsum = {}  # duration-weighted means of the derived % metrics (VALUBusy, MfmaUtil)
    sq_by_id = defaultdict(dict)
    for r in _read(sq_csv):
        sq_by_id[int(r["Dispatch_Id"])][r["Counter_Name"]] = float(r["Counter_Value"])
    for (lab, *_), (knames, ids) in zip(labels, truns):
        dur[lab] = sum(by_tid[i] for i in ids) / REPS  # per call: every kernel the call launches
        tot = sum(by_tid[i] for i in ids)
        wsum[lab] = {c: sum(sq_by_id[i].get(c, 0.0) * by_tid[i] for i in ids) / tot
                     for c in ("VALUBusy", "MfmaUtil")}
    fscale = COPY_BYTES / (_copy_mean(_read(fetch_csv), "FETCH_SIZE") * 1024)
    wscale = COPY_BYTES / (_copy_mean(_read(write_csv), "WRITE_SIZE") * 1024)
    mean = lambda v: sum(v) / REPS if v else float("nan")  # per call (sum over its kernels)
    print(f"| call | kernel | us (trace) | rate | VALU lane-ops / weight | VALUBusy % | "
          f"MfmaUtil % | MFMA insts | LDS insts | LDS bank-conflict cycles | HBM bytes / "
          f"algorithmic |")
    print("|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    table = []
    for lab, d_out, d_in, M, algo, flops in labels:
        p = per[lab]
        us = dur[lab]
        valu = mean(p["SQ_INSTS_VALU"])
        weights = d_out * d_in if d_out else 0
        lane_ops = valu * 64 / weights if weights else float("nan")
        rd = mean(p["FETCH_SIZE"]) * 1024 * fscale
        wr = mean(p["WRITE_SIZE"]) * 1024 * wscale
        hbm = rd + wr
        if flops:
            rate = f"{flops / us / 1e6:.0f} TFLOP/s"
        else:
            rate = f"{algo / us / 1e3:.0f} GB/s"
        ratio = hbm / algo if algo else float("nan")
        kname = " + ".join(k.replace("(anonymous namespace)::", "").split("(")[0].replace(
            "void ", "") for k in p["kernel"])
        print(f"| {lab} | `{kname}` | {us:.2f} | {rate} | {lane_ops:.2f} | "
              f"{wsum[lab]['VALUBusy']:.1f} | {wsum[lab]['MfmaUtil']:.1f} | "
              f"{mean(p['SQ_INSTS_MFMA']):.0f} | {mean(p['SQ_INSTS_LDS']):.0f} | "
              f"{mean(p['SQ_LDS_BANK_CONFLICT']):.0f} | {ratio:.4f} |")
        table.append(dict(label=lab, kernel=kname, us=us, hbm_bytes=hbm, read_bytes=rd,
                          write_bytes=wr, fetch_kb_raw=mean(p["FETCH_SIZE"]),
                          write_kb_raw=mean(p["WRITE_SIZE"]), fetch_scale=fscale,
                          write_scale=wscale, dispatches=len(p["FETCH_SIZE"]),
                          calls=REPS,
                          algorithmic_bytes=algo, flops=flops, valu_lane_ops_per_weight=lane_ops,
                          valu_busy=wsum[lab]["VALUBusy"], mfma_util=wsum[lab]["MfmaUtil"]))
    print(f"\nFETCH_SIZE scale {fscale:.4f}, WRITE_SIZE scale {wscale:.4f} (256 MiB copy); "
          f"{REPS} calls per label, counters and durations summed over the kernels of a call")
    return table


def update_traffic(table):
    """Record the calibrated bytes of the C2 gate/up GEMV for bench.py's roofline.traffic."""
    from bench import TRAFFIC_SOURCES, source_hash

    row = table[0]
    out = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(out)) if os.path.exists(out) else {}
    data["gemv_c2_gate_up"] = {
        "kernel": row["kernel"] + " (C2 gate/up 37888x3584, M=1, bf16 out)",
        "source_hash": source_hash(*TRAFFIC_SOURCES),
        "bytes_per_launch": round(row["hbm_bytes"]),
        "read_bytes_per_launch": round(row["read_bytes"]),
        "write_bytes_per_launch": round(row["write_bytes"]),
        "algorithmic_bytes_per_launch": row["algorithmic_bytes"],
        "traffic_over_algorithmic": round(row["hbm_bytes"] / row["algorithmic_bytes"], 4),
        "fetch_kb_raw": round(row["fetch_kb_raw"], 1),
        "write_kb_raw": round(row["write_kb_raw"], 1),
        "fetch_scale": round(row["fetch_scale"], 4),
        "write_scale": round(row["write_scale"], 4),
        "calibration": f"{COPY_BYTES >> 20} MiB device copy, mean of {CALIB_COPIES} dispatches",
        "dispatches": row["dispatches"],
    }
    with open(out, "w") as fh:
        json.dump(data, fh, indent=2)


def update_trace(stats_csv):
    """Record the kernel-trace average durations of the C2 GEMVs (rocprofv3 --kernel-trace --stats
    of `bench.py --only c2`) for bench.py's trace-based roofline fraction."""
    from bench import DOWN_SOURCES, TRAFFIC_SOURCES, source_hash

    rows = _read(stats_csv)
    want = {"gemv_c2_gate_up": ("gemv_i8_kernel<1, false, 1, false>", TRAFFIC_SOURCES),
            "gemv_c2_down": ("gemv_w4a16_stream_kernel<1, 5, 1, 2, false, 2, 448>", DOWN_SOURCES)}
    out = os.path.join(ROOT, "profiles", "kernel_trace.json")
    data = json.load(open(out)) if os.path.exists(out) else {}
    for key, (kname, srcs) in want.items():
        for r in rows:
            if kname in r["Name"]:
                data[key] = {"kernel": kname, "source_hash": source_hash(*srcs),
                             "calls": int(r["Calls"]),
                             "avg_us": round(float(r["AverageNs"]) / 1e3, 3),
                             "min_us": round(float(r["MinNs"]) / 1e3, 3)}
    with open(out, "w") as fh:
        json.dump(data, fh, indent=2)


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "run":
        run(sys.argv[2])
    elif len(sys.argv) == 3 and sys.argv[1] == "trace":
        update_trace(sys.argv[2])
    elif len(sys.argv) == 7 and sys.argv[1] == "summarize":
        t = summarize(*sys.argv[2:7])
        if sys.argv[2] == "c2":
            update_traffic(t)
    else:
        raise SystemExit(__doc__)
