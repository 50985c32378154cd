"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

  python -m block_scaled_w8a8_amd.profile_summary stats   <kernel_stats.csv> --command "..." --out FILE
  python -m block_scaled_w8a8_amd.profile_summary traffic --fetch <dir> --write <dir>
         --copy-fetch <dir> --copy-write <dir> --kernel SUBSTR --command "..." --out FILE
  python -m block_scaled_w8a8_amd.profile_summary counters <dir> [<dir> ...] --kernel SUBSTR
         [--grid-threads G] --command "..." --out FILE

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


# Derived figures of the `counters` summary (each needs all its counters in the runs given):
#   clock_mhz       GRBM_GUI_ACTIVE / 8 XCDs / kernel duration (the engine clock under load)
#   mfma_busy       SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 256 CUs * 4 SIMDs)
#   vmem_wait       SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (share of wave cycles waiting on s_waitcnt)
#   vmem_in_flight  SQ_INST_LEVEL_VMEM / SQ_ACTIVE_INST_VMEM (vector-memory instructions in
#                   flight, per cycle with any in flight)
#   l1_l2_latency   TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum (cycles per L1->L2 read)
#   l1_l2_reads_mb  TCP_TCC_READ_REQ_sum * 128 B (L1 -> L2 read requests, 128-byte lines)
#   l2_hit          TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum)
#   l2_in_flight    TCC_EA0_RDREQ_LEVEL_sum / GRBM_GUI_ACTIVE * 8 (L2 -> memory reads in flight)
#   hbm_mb          FETCH_SIZE * fetch_factor + WRITE_SIZE (KiB -> MB), as in `traffic`
DERIVED = {
    "mfma_busy": (("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
                  lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8 * 256 * 4)),
    "vmem_wait": (("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
                  lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]),
    "vmem_in_flight": (("SQ_INST_LEVEL_VMEM", "SQ_ACTIVE_INST_VMEM"),
                       lambda c: c["SQ_INST_LEVEL_VMEM"] / c["SQ_ACTIVE_INST_VMEM"]),
    "lds_wait": (("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
                 lambda c: c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"]),
    "l1_l2_latency": (("TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum"),
                      lambda c: c["TCP_TCC_READ_REQ_LATENCY_sum"] / c["TCP_TCC_READ_REQ_sum"]),
    "l1_l2_reads_mb": (("TCP_TCC_READ_REQ_sum",), lambda c: c["TCP_TCC_READ_REQ_sum"] * 128 / 1e6),
    "l2_hit": (("TCC_HIT_sum", "TCC_MISS_sum"),
               lambda c: c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])),
    "l2_in_flight": (("TCC_EA0_RDREQ_LEVEL_sum", "GRBM_GUI_ACTIVE"),
                     lambda c: c["TCC_EA0_RDREQ_LEVEL_sum"] / c["GRBM_GUI_ACTIVE"] * 8),
}


def cmd_counters(args):
    """Per-dispatch means of every counter over one kernel's dispatches in several --pmc runs
    (each may also carry --kernel-trace for durations), plus the derived figures above."""
    means, n_disp, durs, names = {}, {}, [], set()
    for d in args.runs:
        rows = [r for r in _rows(d, "*counter_collection.csv") if args.kernel in r["Kernel_Name"]]
        if args.grid_threads:
            keep = {int(g) for g in args.grid_threads.split(",")}
            rows = [r for r in rows if int(r["Grid_Size"]) in keep]
        per = {}
        for r in rows:
            names.add(r["Kernel_Name"])
            per.setdefault(r["Counter_Name"], {}).setdefault(r.get("Dispatch_Id", r.get("Correlation_Id")), 0.0)
            per[r["Counter_Name"]][r.get("Dispatch_Id", r.get("Correlation_Id"))] += float(r["Counter_Value"])
        for cname, disp in per.items():
            means.setdefault(cname, []).extend(disp.values())
        for r in _rows(d, "*kernel_trace.csv"):
            if args.kernel in r["Kernel_Name"] and (not args.grid_threads or int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]) in keep):
                durs.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    c = {k: sum(v) / len(v) for k, v in means.items() if v}
    n_disp = {k: len(v) for k, v in means.items()}
    lines = ["# rocprofv3 --pmc counters per dispatch (mean over the kernel's dispatches)",
             f"# command: {args.command}",
             "# derived: clock_mhz = GRBM_GUI_ACTIVE/8/duration (overstated for kernels under ~100 us:",
             "#   GUI_ACTIVE also counts the dispatch around them); mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES",
             "#   / (GUI_ACTIVE/8 * 256 CUs * 4 SIMDs); l1_l2_latency = cycles per L1->L2 read request;",
             "#   l1_l2_reads_mb = L1->L2 read requests * 128 B; l2_hit = TCC hits / (hits + misses);",
             "#   hbm_mb = FETCH_SIZE * fetch_factor + WRITE_SIZE; durations are under counter collection",
             f"kernel_sources {source_hash()}",
             f"kernel {sorted(names)[0] if names else args.kernel}",
             f"grid_threads {args.grid_threads or ''}"]
    if durs:
        lines.append(f"duration_us {sum(durs) / len(durs) / 1e3:.2f}")
        if "GRBM_GUI_ACTIVE" in c:
            lines.append(f"clock_mhz {c['GRBM_GUI_ACTIVE'] / 8 / (sum(durs) / len(durs)) * 1e3:.0f}")
    if "FETCH_SIZE" in c and args.fetch_factor:
        lines.append(f"hbm_mb {(c['FETCH_SIZE'] * args.fetch_factor + c.get('WRITE_SIZE', 0.0)) * 1024 / 1e6:.1f}")
    for k, (need, fn) in DERIVED.items():
        if all(n in c for n in need):
            lines.append(f"{k} {fn(c):.4g}")
    lines.append("# raw (per dispatch; dispatches averaged)")
    for k in sorted(c):
        lines.append(f"{k} {c[k]:.6g}  n={n_disp[k]}")
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
    k = sub.add_parser("counters")
    k.add_argument("runs", nargs="+", help="rocprofv3 output directories, one per --pmc pass")
    k.add_argument("--kernel", required=True)
    k.add_argument("--grid-threads", default="")
    k.add_argument("--fetch-factor", type=float, default=2.0,
                   help="bytes per FETCH_SIZE byte, from a device copy of known size")
    k.add_argument("--command", default="")
    k.add_argument("--out")
    args = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.cmd](args)


if __name__ == "__main__":
    main()
