"""Summaries of rocprofv3 results (rocpd SQLite databases) for this library's kernels.

  python -m moe_grouped_gemm_e4m3_amd.profiling stats DIR
      per-kernel dispatch count and average/min/max duration (us), grouped by grid size
  python -m moe_grouped_gemm_e4m3_amd.profiling pmc DIR
      per-kernel average of every collected counter
  python -m moe_grouped_gemm_e4m3_amd.profiling traffic --fetch DIR1 --write DIR2 \
        --workload W --label L --kernel REGEX [--grid G] --out profiles/traffic.json
      HBM bytes per launch of one kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
      from two separate --pmc runs), each scaled by what the same counter reads for the
      reference copy kernel (a 256 MiB device-to-device copy, 256 MiB read and written).

Nothing here touches the GPU; it only reads the databases rocprofv3 wrote.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sqlite3
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 * 2 ** 20  # the reference copy: 64 Mi float32 elements


def source_hash() -> str:
    """Hash of the GEMM kernel sources; counter figures are valid only for this source."""
    h = hashlib.sha256()
    for f in ("gemm.hip", "dg_device.h"):
        with open(os.path.join(_PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _dbs(path: str):
    if path.endswith(".db"):
        return [path]
    return sorted(glob.glob(os.path.join(path, "**", "*.db"), recursive=True))


def _short(name: str) -> str:
    name = re.sub(r"\(anonymous namespace\)::|void |dg::", "", name)
    name = name.replace("(KParams)", "")
    return name if len(name) <= 100 else name[:97] + "..."


def kernel_stats(path: str):
    rows = []
    for db in _dbs(path):
        c = sqlite3.connect(db)
        rows += c.execute("select name, grid_x, workgroup_x, count(*), avg(end-start), min(end-start), "
                          "max(end-start) from kernels group by name, grid_x").fetchall()
    return rows


def pmc_stats(path: str):
    rows = []
    for db in _dbs(path):
        c = sqlite3.connect(db)
        rows += c.execute("select name, counter_name, avg(counter_value), count(*), avg(duration) "
                          "from pmc_events group by name, counter_name").fetchall()
    return rows


def _counter_per_kernel(path: str, counter: str, regex: str, grid=None, largest=False):
    vals = []
    for db in _dbs(path):
        c = sqlite3.connect(db)
        q = ("select p.name, p.counter_value, k.grid_x from pmc_events p left join kernels k "
             "on k.dispatch_id = p.dispatch_id where p.counter_name = ?")
        try:
            got = c.execute(q, (counter,)).fetchall()
        except sqlite3.OperationalError:
            got = [(n, v, None) for n, v in c.execute(
                "select name, counter_value from pmc_events where counter_name = ?", (counter,)).fetchall()]
        for name, v, g in got:
            if re.search(regex, name) and (grid is None or g is None or int(g) == int(grid)):
                vals.append(float(v))
    if not vals:
        raise SystemExit("no %s values for kernels matching %r in %s" % (counter, regex, path))
    if largest:  # the reference copy is the largest dispatch of its kernel
        return max(vals), 1
    return sum(vals) / len(vals), len(vals)


def traffic(args) -> dict:
    copy_re = r"__amd_rocclr_copyBuffer"
    f_copy, _ = _counter_per_kernel(args.fetch, "FETCH_SIZE", copy_re, largest=True)
    w_copy, _ = _counter_per_kernel(args.write, "WRITE_SIZE", copy_re, largest=True)
    f_k, nf = _counter_per_kernel(args.fetch, "FETCH_SIZE", args.kernel, args.grid)
    w_k, nw = _counter_per_kernel(args.write, "WRITE_SIZE", args.kernel, args.grid)
    f_scale = COPY_BYTES / (f_copy * 1024.0)
    w_scale = COPY_BYTES / (w_copy * 1024.0)
    rec = {"bytes_per_launch": f_k * 1024.0 * f_scale + w_k * 1024.0 * w_scale,
           "fetch_kib": f_k, "write_kib": w_k, "fetch_scale": f_scale, "write_scale": w_scale,
           "dispatches": [nf, nw], "kernel": args.kernel, "source_hash": source_hash()}
    data = {}
    if os.path.exists(args.out):
        with open(args.out) as fh:
            data = json.load(fh)
    data.setdefault(args.workload, {})[args.label] = rec
    with open(args.out, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    p = sub.add_parser("stats"); p.add_argument("path"); p.add_argument("--match", default="")
    p = sub.add_parser("pmc"); p.add_argument("path"); p.add_argument("--match", default="")
    p = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--workload", "--label", "--kernel", "--out"):
        p.add_argument(a, required=True)
    p.add_argument("--grid", type=int, default=None)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print("%7s %10s %10s %10s %9s %5s  %s" % ("calls", "avg_us", "min_us", "max_us", "grid", "wg", "kernel"))
        for name, grid, wg, n, avg, mn, mx in kernel_stats(args.path):
            if args.match and not re.search(args.match, name):
                continue
            print("%7d %10.3f %10.3f %10.3f %9d %5d  %s" % (n, avg / 1e3, mn / 1e3, mx / 1e3, grid, wg, _short(name)))
    elif args.cmd == "pmc":
        for name, counter, v, n, dur in pmc_stats(args.path):
            if args.match and not re.search(args.match, name):
                continue
            print("%-34s %18.1f  n=%-4d dur=%9.3fus  %s" % (counter, v, n, dur / 1e3, _short(name)))
    else:
        print(json.dumps(traffic(args), indent=1))


if __name__ == "__main__":
    main(sys.argv[1:])
