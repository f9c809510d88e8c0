"""Summaries of rocprofv3 output for the matvec kernels.

    python -m quantized_decode_matvec_amd.rocprof_summary stats KERNEL_STATS_CSV [--match SUBSTR]
    python -m quantized_decode_matvec_amd.rocprof_summary grid KERNEL_TRACE_CSV [--match SUBSTR]
    python -m quantized_decode_matvec_amd.rocprof_summary traffic --kernel SUBSTR --key NAME \\
        --fetch FETCH_CSV --write WRITE_CSV --calib-fetch CF_CSV --calib-write CW_CSV \\
        [--grid THREADS] [--sources FILE ...] [--calib-kernel copyBuffer] [--calib-bytes 1073741824] \\
        [--out profiles/traffic.json]

`grid` groups a kernel trace by kernel and launch grid (one line per distinct
launch shape, e.g. per token count of the MoE kernels) with the median and
minimum duration.

`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into HBM bytes per
dispatch: each counter is divided by what the same counter reads for a plain
device copy of known size (the calibration run), so the factor absorbs how
the counter is defined on this GPU. The record is keyed by the SHA-256 of the
matvec kernel sources, so a later kernel change invalidates it.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/matvec.hip", "csrc/qmv_device.h")   # the batch 1-2 matvec kernels


def kernel_source_hash(sources=None) -> str:
    """SHA-256 over the sources a kernel is built from (a counter record taken
    on other sources no longer describes the kernel)."""
    h = hashlib.sha256()
    sources = sources or KERNEL_SOURCES
    for rel in sources:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _per_kernel(path, counter, grid_size=None):
    """Counter values per kernel name; with `grid_size`, only dispatches of that
    total grid size (threads), e.g. one token count of the MoE kernels."""
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if grid_size is not None and int(r["Grid_Size"]) != grid_size:
            continue
        vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def _pick(vals, substr):
    hits = {k: v for k, v in vals.items() if substr in k}
    if len(hits) != 1:
        raise SystemExit("kernel match %r is not unique: %s" % (substr, list(hits)[:5]))
    (name, v), = hits.items()
    return name, sum(v) / len(v), len(v)


def stats(path, match=None):
    rows = list(csv.DictReader(open(path)))
    out = []
    for r in rows:
        if match and match not in r["Name"]:
            continue
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    return out


def grid(path, match=None):
    groups = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if match and match not in name:
            continue
        key = (name.split("(")[0], r["Grid_Size_X"], r["Grid_Size_Y"], r["Workgroup_Size_X"])
        groups[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = []
    for key, v in sorted(groups.items()):
        v.sort()
        out.append(key + (len(v), v[len(v) // 2], v[0]))
    return out


def window(path, match, last):
    """Durations of the last `last` dispatches of the kernels matching `match`
    (the timed region of a bench run comes last): mean, min, max in us, and
    the wall time from the first start to the last end divided by `last`."""
    rows = [r for r in csv.DictReader(open(path)) if match in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rows = rows[-last:]
    d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    wall = (int(rows[-1]["End_Timestamp"]) - int(rows[0]["Start_Timestamp"])) / 1e3 / len(rows)
    return len(d), sum(d) / len(d), min(d), max(d), wall


def traffic(args):
    fetch_name, fetch_kib, nf = _pick(_per_kernel(args.fetch, "FETCH_SIZE", args.grid), args.kernel)
    write_name, write_kib, nw = _pick(_per_kernel(args.write, "WRITE_SIZE", args.grid), args.kernel)
    _, cf_kib, _ = _pick(_per_kernel(args.calib_fetch, "FETCH_SIZE"), args.calib_kernel)
    _, cw_kib, _ = _pick(_per_kernel(args.calib_write, "WRITE_SIZE"), args.calib_kernel)
    known_kib = args.calib_bytes / 1024.0
    f_fac, w_fac = cf_kib / known_kib, cw_kib / known_kib
    read_b = fetch_kib / f_fac * 1024.0
    write_b = write_kib / w_fac * 1024.0
    rec = {
        "kernel": fetch_name,
        "grid_size": args.grid,
        "kernel_sources": list(args.sources),
        "kernel_source_sha256": kernel_source_hash(args.sources),
        "fetch_kib_per_dispatch": round(fetch_kib, 1), "fetch_dispatches": nf,
        "write_kib_per_dispatch": round(write_kib, 1), "write_dispatches": nw,
        "calibration": {"kernel": args.calib_kernel, "bytes": args.calib_bytes,
                        "fetch_kib": round(cf_kib, 1), "write_kib": round(cw_kib, 1),
                        "fetch_factor": round(f_fac, 5), "write_factor": round(w_fac, 5)},
        "hbm_read_bytes": int(round(read_b)), "hbm_write_bytes": int(round(write_b)),
        "traffic_bytes": int(round(read_b + write_b)),
    }
    db = {}
    if args.out and os.path.exists(args.out):
        db = json.load(open(args.out))
    db[args.key] = rec
    if args.out:
        with open(args.out, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)
            f.write("\n")
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--match")
    g = sub.add_parser("grid")
    g.add_argument("csv")
    g.add_argument("--match")
    w = sub.add_parser("window")
    w.add_argument("csv")
    w.add_argument("--match", required=True)
    w.add_argument("--last", type=int, required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--key", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--calib-fetch", required=True)
    t.add_argument("--calib-write", required=True)
    t.add_argument("--calib-kernel", default="copyBuffer")
    t.add_argument("--calib-bytes", type=int, default=1 << 30)
    t.add_argument("--grid", type=int, help="only dispatches of this total grid size (threads)")
    t.add_argument("--sources", nargs="+", default=list(KERNEL_SOURCES),
                   help="sources the kernel is built from, relative to the package")
    t.add_argument("--out")
    a = ap.parse_args()
    if a.cmd == "stats":
        print("| kernel | calls | avg us | min us | max us |")
        print("|---|---|---|---|---|")
        for name, calls, avg, mn, mx in stats(a.csv, a.match):
            print("| %s | %d | %.2f | %.2f | %.2f |" % (name[:110], calls, avg / 1e3, mn / 1e3, mx / 1e3))
    elif a.cmd == "window":
        n, avg, mn, mx, wall = window(a.csv, a.match, a.last)
        print("| dispatches | avg us | min us | max us | wall us per dispatch |")
        print("|---|---|---|---|---|")
        print("| %d | %.2f | %.2f | %.2f | %.2f |" % (n, avg, mn, mx, wall))
    elif a.cmd == "grid":
        print("| kernel | grid x (threads) | grid y | workgroup | calls | median us | min us |")
        print("|---|---|---|---|---|---|---|")
        for name, gx, gy, wg, n, med, mn in grid(a.csv, a.match):
            print("| %s | %s | %s | %s | %d | %.2f | %.2f |" % (name[:90], gx, gy, wg, n, med, mn))
    else:
        traffic(a)


if __name__ == "__main__":
    main()
