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

  python -m moe_grouped_gemm_e4m3_amd.profiling mfma DIR [--se 32] [--simds 1024]
      per kernel and grid: FP8 MFMA work counted by the hardware (SQ_INSTS_VALU_MFMA_MOPS_F8
      and _F6F4, 512 flops per unit), MFMA instructions, and the matrix-unit utilisation
      SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs), averaged over dispatches. The SQ
      counters read per shader engine; totals are scaled by the engine count (32 on MI355X:
      8 XCDs x 4), which the flop totals confirm against the algorithmic counts.

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


def _code_only(text: str) -> str:
    """C++ source without its comments and with whitespace runs collapsed (string and
    character literals kept as they are), so that editing a comment keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(texts=None) -> str:
    """Hash of the GEMM kernel sources' code (comments and layout excluded); counter figures
    are valid only for this code. `texts` (gemm.hip, dg_device.h contents) defaults to the
    files in csrc/."""
    if texts is None:
        texts = []
        for f in ("gemm.hip", "dg_device.h"):
            with open(os.path.join(_PKG, "csrc", f), encoding="utf-8") as fh:
                texts.append(fh.read())
    h = hashlib.sha256()
    for t in texts:
        h.update(_code_only(t).encode())
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


def mfma_stats(path: str):
    """{(kernel, grid): {counter: average per dispatch}, plus the dispatch count}."""
    acc = {}
    for db in _dbs(path):
        c = sqlite3.connect(db)
        rows = c.execute("select p.name, k.grid_x, p.counter_name, avg(p.counter_value), count(*) from pmc_events p "
                         "left join kernels k on k.dispatch_id = p.dispatch_id "
                         "group by p.name, k.grid_x, p.counter_name").fetchall()
        for name, grid, counter, v, n in rows:
            rec = acc.setdefault((name, grid), {})
            rec[counter] = v
            rec["n"] = max(rec.get("n", 0), n)
    return acc


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
    p = sub.add_parser("mfma"); p.add_argument("path"); p.add_argument("--match", default="")
    p.add_argument("--se", type=int, default=32)
    p.add_argument("--simds", type=int, default=1024)
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
    elif args.cmd == "mfma":
        print("%6s %9s %11s %11s %11s %12s %12s %7s  %s" % (
            "calls", "grid", "F8 GFLOP", "F6F4 GFLOP", "MFMA insts", "busy cyc/SE", "active cyc", "util %", "kernel"))
        for (name, grid), rec in sorted(mfma_stats(args.path).items(), key=lambda kv: _short(kv[0][0])):
            if args.match and not re.search(args.match, name):
                continue
            f8 = rec.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512 * args.se / 1e9
            f64 = rec.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0) * 512 * args.se / 1e9
            busy, act = rec.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), rec.get("GRBM_GUI_ACTIVE", 0.0)
            util = 100.0 * busy * args.se / (act * args.simds) if act else 0.0
            print("%6d %9s %11.3f %11.3f %11.0f %12.4g %12.4g %7.1f  %s" % (
                rec.get("n", 0), grid, f8, f64, rec.get("SQ_INSTS_VALU_MFMA_F8", 0.0) * args.se, busy, act, util,
                _short(name)))
    else:
        print(json.dumps(traffic(args), indent=1))


if __name__ == "__main__":
    main(sys.argv[1:])
