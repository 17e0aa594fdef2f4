"""HBM traffic of the decode GEMV, measured with rocprofv3 counters and calibrated on a copy.

bench.py reports `roofline.traffic` (HBM bytes per launch of the C2 gate/up GEMV) from
profiles/traffic.json, which this script writes.  Two counter passes are needed because one pass
cannot hold both derived counters:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o pmc -- python3 bench_traffic.py run
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o pmc -- python3 bench_traffic.py run
    python3 bench_traffic.py summarize <dir_f>/..._counter_collection.csv <dir_w>/..._counter_collection.csv

`run` launches, on the current weights source: a plain device copy of 256 MiB (known bytes:
256 MiB read, 256 MiB written) several times, then the C2 gate/up GEMV over rotated weight copies
(so that the weights come from memory, not from the 256 MB Infinity Cache).  `summarize` averages
the per-dispatch counters of each kernel, derives the scale factors (known copy bytes / counted
copy bytes, one for reads and one for writes) and writes the calibrated bytes per GEMV launch,
keyed by a hash of the kernel sources; bench.py reports the figure only while that hash matches.
"""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 256 << 20
CALIB_COPIES = 4
GEMV_KERNEL = "gemv_i8_kernel"


def run():
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

    cfg = workloads.C2
    gu = cfg.linears[0]
    w = torch.from_numpy(workloads.linear_weight(cfg, 0)).to(dev)
    qw, sc, zr = w4.w4_pack(w, gu.group_size, gu.mode)
    del w
    per_copy = qw.numel() + 2 * sc.numel()
    n_copies = max(2, -(-(2 * INFINITY_CACHE_BYTES + (64 << 20)) // per_copy))
    copies = [(qw.clone(), sc.clone()) for _ in range(n_copies)]
    x = torch.from_numpy(workloads.linear_x(cfg, 0, 1).view("int16")).view(torch.bfloat16).to(dev)
    y = torch.empty((1, gu.d_out), dtype=torch.bfloat16, device=dev)
    for i in range(2 * n_copies):
        c = copies[i % n_copies]
        w4.w4_gemv(x, c[0], c[1], None, None, gu.d_in, gu.group_size, out=y)
    torch.cuda.synchronize()
    print(f"ran {CALIB_COPIES} copies of {COPY_BYTES} B and {2 * n_copies} gate/up GEMVs "
          f"({n_copies} weight copies)", flush=True)


def per_kernel_mean(path, counter):
    """Mean counter value per dispatch of the calibration copies (the first CALIB_COPIES device
    copies of the run, issued before anything else) and of the GEMV kernel."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    copies = [v for _, name, v in rows if "copybuffer" in name.lower()][:CALIB_COPIES]
    gemv = [v for _, name, v in rows if GEMV_KERNEL in name]
    mean = lambda v: (sum(v) / len(v) if v else None, len(v))
    return {"copy": mean(copies), "gemv": mean(gemv)}


def summarize(fetch_csv, write_csv):
    from bench import TRAFFIC_SOURCES, linear_bytes, source_hash
    import workloads

    f = per_kernel_mean(fetch_csv, "FETCH_SIZE")
    w = per_kernel_mean(write_csv, "WRITE_SIZE")
    (copy_f_kb, n_cf), (gemv_f_kb, n_gf) = f["copy"], f["gemv"]
    (copy_w_kb, n_cw), (gemv_w_kb, n_gw) = w["copy"], w["gemv"]
    if None in (copy_f_kb, gemv_f_kb, copy_w_kb, gemv_w_kb):
        raise SystemExit(f"missing dispatches: fetch {f}, write {w}")
    scale_f = COPY_BYTES / (copy_f_kb * 1024)
    scale_w = COPY_BYTES / (copy_w_kb * 1024)
    read_b = gemv_f_kb * 1024 * scale_f
    write_b = gemv_w_kb * 1024 * scale_w
    gu = workloads.C2.linears[0]
    algo = linear_bytes(1, gu.d_out, gu.d_in, gu.group_size, False)
    entry = {
        "kernel": f"{GEMV_KERNEL} (C2 gate/up 37888x3584, M=1, bf16 out)",
        "source_hash": source_hash(*TRAFFIC_SOURCES),
        "bytes_per_launch": round(read_b + write_b),
        "read_bytes_per_launch": round(read_b),
        "write_bytes_per_launch": round(write_b),
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": round((read_b + write_b) / algo, 4),
        "fetch_kb_raw": round(gemv_f_kb, 1), "write_kb_raw": round(gemv_w_kb, 1),
        "copy_fetch_kb_raw": round(copy_f_kb, 1), "copy_write_kb_raw": round(copy_w_kb, 1),
        "fetch_scale": round(scale_f, 4), "write_scale": round(scale_w, 4),
        "dispatches": {"gemv_fetch": n_gf, "gemv_write": n_gw, "copy_fetch": n_cf,
                       "copy_write": n_cw},
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(out):
        with open(out) as fh:
            data = json.load(fh)
    data["gemv_c2_gate_up"] = entry
    with open(out, "w") as fh:
        json.dump(data, fh, indent=2)
    print(json.dumps(entry, indent=2))


if __name__ == "__main__":
    if len(sys.argv) >= 2 and sys.argv[1] == "run":
        run()
    elif len(sys.argv) == 4 and sys.argv[1] == "summarize":
        summarize(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
