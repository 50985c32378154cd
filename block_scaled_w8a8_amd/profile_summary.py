"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m block_scaled_w8a8_amd.profile_summary stats   <kernel_stats.csv> --command "..." --out FILE
  python -m block_scaled_w8a8_amd.profile_summary traffic --fetch <dir> --write <dir>
         --copy-fetch <dir> --copy-write <dir> --kernel SUBSTR --command "..." --out FILE

`traffic` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over the dispatches of one
kernel and scales each by what the same counter reads for a plain device copy of known size
(bytes moved by the copy / counter reading), so the result is HBM bytes per launch. It also
records a hash of the kernel sources, so bench.py can tell whether the counters still
describe the current kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/gemm_std.hip", "csrc/gemm_swapab.hip", "csrc/quant.hip",
                  "csrc/moe.hip", "csrc/device_common.h")


def source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path_or_dir, name):
    if os.path.isdir(path_or_dir):
        files = glob.glob(os.path.join(path_or_dir, "**", name), recursive=True)
    else:
        files = [path_or_dir]
    out = []
    for f in files:
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def cmd_stats(args):
    rows = _rows(args.csv, "*kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {args.command}",
             f"# kernel sources: {source_hash()}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total%':>7}  kernel"]
    for r in rows[: args.top]:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                     f"{float(r['Percentage']):7.2f}  {r['Name'][:150]}")
    if args.trace:
        trace = _rows(args.trace, "*kernel_trace.csv")
        groups = {}
        for r in trace:
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            g = groups.setdefault(key, [0, 0])
            g[0] += 1
            g[1] += d
        lines += ["", "# per (kernel, grid threads) from the kernel trace",
                  f"{'calls':>6} {'avg_us':>10} {'grid':>10}  kernel"]
        for (name, grid), (n, tot) in sorted(groups.items(), key=lambda kv: -kv[1][1])[: args.top]:
            lines.append(f"{n:6d} {tot / n / 1e3:10.2f} {grid:10d}  {name[:150]}")
    _write(args.out, lines)


def _counter_mean(rows, counter, kernel_sub, grids=None):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and kernel_sub in r["Kernel_Name"]
            and (grids is None or int(r["Grid_Size"]) in grids)]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def cmd_traffic(args):
    f_rows = _rows(args.fetch, "*counter_collection.csv")
    w_rows = _rows(args.write, "*counter_collection.csv")
    cf_rows = _rows(args.copy_fetch, "*counter_collection.csv")
    cw_rows = _rows(args.copy_write, "*counter_collection.csv")
    grids = {int(g) for g in args.grid_threads.split(",")} if args.grid_threads else None
    fetch, nf = _counter_mean(f_rows, "FETCH_SIZE", args.kernel, grids)
    write, nw = _counter_mean(w_rows, "WRITE_SIZE", args.kernel, grids)
    cfetch, _ = _counter_mean(cf_rows, "FETCH_SIZE", "copyBuffer")
    cwrite, _ = _counter_mean(cw_rows, "WRITE_SIZE", "copyBuffer")
    copy_kib = args.copy_bytes / 1024.0
    kf = copy_kib / cfetch
    kw = copy_kib / cwrite
    bytes_per_launch = (fetch * kf + write * kw) * 1024.0
    names = sorted({r["Kernel_Name"] for r in f_rows if args.kernel in r["Kernel_Name"]})
    lines = ["# HBM traffic per dispatch from rocprofv3 --pmc (FETCH_SIZE and WRITE_SIZE runs)",
             f"# command: {args.command}",
             f"kernel_sources {source_hash()}",
             f"kernel {names[0] if names else args.kernel}",
             f"grid_threads {args.grid_threads or ''}",
             f"dispatches_fetch {nf}", f"dispatches_write {nw}",
             f"fetch_kib_per_dispatch {fetch:.1f}", f"write_kib_per_dispatch {write:.1f}",
             f"copy_bytes {args.copy_bytes}",
             f"copy_fetch_kib {cfetch:.1f}", f"copy_write_kib {cwrite:.1f}",
             f"fetch_factor {kf:.4f}", f"write_factor {kw:.4f}",
             f"hbm_bytes_per_dispatch {bytes_per_launch:.0f}"]
    _write(args.out, lines)


def _write(path, lines):
    text = "\n".join(lines) + "\n"
    if path:
        os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
        with open(path, "w") as f:
            f.write(text)
    print(text, end="")


def read_traffic(path):
    """Parse a traffic summary written by `traffic` (key value per line)."""
    out = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, _, v = line.strip().partition(" ")
            out[k] = v
    return out


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", default="")
    s.add_argument("--out")
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--trace", help="kernel_trace.csv (or its directory) for per-grid averages")
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", type=int, default=1 << 30)
    t.add_argument("--kernel", required=True)
    t.add_argument("--grid-threads", default="", help="comma list of Grid_Size values to keep")
    t.add_argument("--command", default="")
    t.add_argument("--out")
    args = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic}[args.cmd](args)


if __name__ == "__main__":
    main()
