"""Text summaries of rocprofv3 output (kernel traces and HBM byte counters).

Kernel trace (a rocprofv3 --kernel-trace output folder, csv or rocpd database):

    python -m int8_gemm_linear_amd.profsum trace <dir>

Any counters of the GEMM kernels, per kernel, over one or more --pmc runs:

    python -m int8_gemm_linear_amd.profsum counters <dir> [<dir> ...]

HBM traffic per GEMM call, from two counter runs of the same bench command,
one with ``--pmc FETCH_SIZE`` and one with ``--pmc WRITE_SIZE`` (csv output),
each run also holding one plain copy of known size (``bench.py --copy-calib``)
that calibrates the counter to bytes:

    python -m int8_gemm_linear_amd.profsum traffic --fetch <dir> --write <dir> \
        --workload int8_1p7b_decode --out profiles/<name>.json

The traffic record carries a fingerprint of the kernel sources and the config
table, so a reader can tell whether the kernels have changed since the
counters were taken.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20          # the calibration copy of bench.py --copy-calib
COPY_TAG = "bitwise_not"        # its kernel is torch's elementwise bitwise_not


def fingerprint(table_path: str | None = None) -> str:
    """sha256 over the kernel sources and the config table in use."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(PKG, "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    tp = table_path or os.path.join(PKG, "configs", "qlin_mi355x.cfg")
    with open(tp, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _is_gemm(name: str) -> bool:
    return "qlin::k_stream" in name or "qlin::k_tile" in name or "qlin::k_gemv" in name


def _is_qlin(name: str) -> bool:
    return "qlin::" in name


def kernel_durations(folder: str, by_grid: bool = False) -> dict[str, list[float]]:
    """{kernel name (with " grid=x,y,z" when by_grid): [duration ns, ...]}
    from a kernel-trace folder."""
    out: dict[str, list[float]] = collections.OrderedDict()
    csvs = glob.glob(os.path.join(folder, "**", "*kernel_trace.csv"), recursive=True)
    if csvs:
        for p in csvs:
            with open(p, newline="") as f:
                for r in csv.DictReader(f):
                    d = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                    k = r["Kernel_Name"]
                    if by_grid:
                        k += " grid=%s,%s,%s" % (r.get("Grid_Size_X", "?"), r.get("Grid_Size_Y", "?"),
                                                 r.get("Grid_Size_Z", "?"))
                    out.setdefault(k, []).append(d)
        return out
    dbs = glob.glob(os.path.join(folder, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no kernel trace under {folder}")
    for p in dbs:
        db = sqlite3.connect(p)
        if by_grid:
            rows = db.execute("select name, duration, grid_size_x, grid_size_y, grid_size_z "
                              "from kernels")
            for name, d, gx, gy, gz in rows:
                out.setdefault(f"{name} grid={gx},{gy},{gz}", []).append(float(d))
        else:
            for name, d in db.execute("select name, duration from kernels"):
                out.setdefault(name, []).append(float(d))
    return out


def trace_summary(folder: str, by_grid: bool = False, match: str | None = None,
                  grid_z: int | None = None) -> str:
    agg = kernel_durations(folder, by_grid or grid_z is not None)
    if match:
        agg = collections.OrderedDict((k, v) for k, v in agg.items() if match in k)
    if grid_z is not None:
        agg = collections.OrderedDict((k, v) for k, v in agg.items()
                                      if k.rsplit(",", 1)[-1] == str(grid_z))
    lines = [f"{'calls':>6} {'avg_us':>9} {'min_us':>8} {'max_us':>8} {'total_ms':>9}  kernel"]
    for name, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(ds) / 1e3
        lines.append(f"{len(d):6d} {d.mean():9.3f} {d.min():8.3f} {d.max():8.3f} "
                     f"{d.sum() / 1e3:9.3f}  {name[:140]}")
    gemm = [k for k in agg if _is_gemm(k)]
    red = [k for k in agg if "qlin::k_reduce" in k]
    if gemm:
        g = np.concatenate([np.array(agg[k]) for k in gemm]) / 1e3
        tot = (g.sum() + sum(sum(agg[k]) for k in red) / 1e3)
        lines.append("")
        lines.append(f"GEMM kernels: {len(g)} launches, mean {g.mean():.3f} us/launch")
        lines.append(f"per GEMM call (GEMM kernel + its split-K reduce when two-pass): "
                     f"{tot / len(g):.3f} us/call")
    return "\n".join(lines)


def counter_values(folder: str, counter: str, with_grid: bool = False):
    """[(kernel name, value)] per dispatch, in dispatch order, from a --pmc csv
    run; with_grid adds the dispatch's grid size as a third field."""
    rows = []
    paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = collections.OrderedDict()
    for p in paths:
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = (p, int(r["Dispatch_Id"]))
                grid = "x".join(r[k] for k in sorted(r) if k and k.startswith("Grid_Size"))
                name, v, _ = per.get(key, (r["Kernel_Name"], 0.0, grid))
                per[key] = (name, v + float(r["Counter_Value"]), grid)
    for key in sorted(per, key=lambda k: (k[0], k[1])):
        rows.append(per[key] if with_grid else per[key][:2])
    return rows


def per_launch_table(folder: str, counter: str, factor: float) -> str:
    """Mean calibrated bytes per dispatch of every (qlin kernel, grid) pair."""
    agg = collections.OrderedDict()
    for n, v, g in counter_values(folder, counter, with_grid=True):
        if _is_qlin(n):
            agg.setdefault((n, g), []).append(v * 1024.0 * factor)
    lines = [f"{'calls':>6} {'mean_MB':>9} {'min_MB':>9} {'max_MB':>9}  grid  kernel"]
    for (n, g), vs in agg.items():
        a = np.array(vs) / 1e6
        lines.append(f"{len(a):6d} {a.mean():9.3f} {a.min():9.3f} {a.max():9.3f}  {g}  {n[:90]}")
    return "\n".join(lines)


def mfma_summary(folder: str, xcds: int = 8, simds: int = 1024) -> str:
    """Matrix-core utilisation per (GEMM kernel, grid) from a --pmc run with
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_*:
    busy fraction = MFMA busy cycles / (GPU cycles x SIMDs), where the GRBM
    count is summed over the XCDs; clock = GPU cycles / kernel duration;
    TFLOP/s from the MOPS counters (512 operations each)."""
    per = collections.OrderedDict()
    for p in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(p, newline="") as f:
            for r in csv.DictReader(f):
                key = (p, int(r["Dispatch_Id"]))
                d = per.setdefault(key, {"name": r["Kernel_Name"], "grid": r.get("Grid_Size", ""),
                                         "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    agg = collections.OrderedDict()
    for d in per.values():
        if not _is_gemm(d["name"]):
            continue
        agg.setdefault((d["name"], d["grid"]), []).append(d)
    lines = [f"{'calls':>5} {'avg_us':>9} {'clock_GHz':>9} {'mfma_busy':>9} {'TFLOP/s':>9}  grid  kernel"]
    for (n, g), ds in agg.items():
        us = np.mean([d["ns"] for d in ds]) / 1e3
        cyc = np.mean([d.get("GRBM_GUI_ACTIVE", 0.0) for d in ds]) / xcds
        busy = np.mean([d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds])
        mops = np.mean([d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0)
                        for d in ds])
        util = busy / (cyc * simds) if cyc else float("nan")
        lines.append(f"{len(ds):5d} {us:9.2f} {cyc / (us * 1e3):9.3f} {util:9.3f} "
                     f"{mops * 512 / (us * 1e-6) / 1e12:9.1f}  {g}  {n[:80]}")
    return "\n".join(lines)


def counters_summary(folders: list[str], skip_first: int = 1) -> str:
    """Mean value per dispatch of every counter of the GEMM kernels in one or
    more --pmc csv runs (one run per counter pass), per kernel, leaving out
    each kernel's first `skip_first` dispatches (cold code and TLBs); with
    the read-latency pair, also the mean L1->L2 read latency in cycles and
    the lines in flight per CU it implies (Little's law: requests per CU x
    latency / GPU cycles, the GRBM count being summed over 8 XCDs)."""
    per = collections.OrderedDict()
    for folder in folders:
        paths = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        if not paths:
            raise SystemExit(f"no counter_collection.csv under {folder}")
        for p in paths:
            disp = collections.OrderedDict()
            with open(p, newline="") as f:
                for r in csv.DictReader(f):
                    if not _is_gemm(r["Kernel_Name"]):
                        continue
                    d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
                    d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            seen = collections.Counter()
            for d in disp.values():
                seen[d["name"]] += 1
                if seen[d["name"]] <= skip_first:
                    continue
                k = per.setdefault(d["name"], collections.defaultdict(list))
                for c, v in d.items():
                    if c != "name":
                        k[c].append(v)
    lines = []
    for name, cs in per.items():
        m = {c: float(np.mean(v)) for c, v in cs.items()}
        lines.append(f"== {name[:100]}")
        req, lat = m.get("TCP_TCC_READ_REQ_sum"), m.get("TCP_TCC_READ_REQ_LATENCY_sum")
        if req and lat:
            line = f"   L1->L2 read latency {lat / req:.0f} cycles, {req / 256:.0f} read requests per CU"
            if m.get("GRBM_GUI_ACTIVE"):
                line += f", {req / 256 * (lat / req) / (m['GRBM_GUI_ACTIVE'] / 8):.0f} lines in flight per CU"
            lines.append(line)
        for c in sorted(m):
            lines.append(f"   {c:42s} {m[c]:.4g}  ({len(cs[c])} dispatches)")
    return "\n".join(lines)


def traffic(fetch_dir: str, write_dir: str, workload: str, table: str | None) -> dict:
    out = {"workload": workload, "fingerprint": fingerprint(table)}
    for tag, folder, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        vals = counter_values(folder, counter)
        copy = [v for n, v in vals if COPY_TAG in n]
        if len(copy) != 1:
            raise SystemExit(f"{counter}: expected one calibration copy, found {len(copy)}")
        factor = COPY_BYTES / (copy[0] * 1024.0)
        calls = [v for n, v in vals if _is_gemm(n)]
        qlin = [v for n, v in vals if _is_qlin(n)]
        if not calls:
            raise SystemExit(f"{counter}: no GEMM dispatches")
        per_call = sum(qlin) * 1024.0 * factor / len(calls)
        out[tag] = {"counter": counter, "calib_copy_kib": copy[0], "factor": round(factor, 5),
                    "gemm_calls": len(calls), "bytes_per_call": round(per_call, 1)}
    out["traffic_bytes_per_call"] = round(out["fetch"]["bytes_per_call"] + out["write"]["bytes_per_call"], 1)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("folder")
    t.add_argument("--by-grid", action="store_true", help="one line per (kernel, grid)")
    t.add_argument("--match", default=None, help="only kernels whose line contains this text")
    t.add_argument("--grid-z", type=int, default=None,
                   help="only launches with this grid.z (e.g. the expert count of grouped calls)")
    m = sub.add_parser("mfma")
    m.add_argument("folder")
    cs = sub.add_parser("counters")
    cs.add_argument("folders", nargs="+")
    c = sub.add_parser("traffic")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--table", default=None)
    c.add_argument("--alg-bytes-per-call", type=float, default=None)
    c.add_argument("--out", default=None)
    c.add_argument("--per-launch", action="store_true", help="also print per (kernel, grid) means")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_summary(a.folder, a.by_grid, a.match, a.grid_z))
        return
    if a.cmd == "mfma":
        print(mfma_summary(a.folder))
        return
    if a.cmd == "counters":
        print(counters_summary(a.folders))
        return
    rec = traffic(a.fetch, a.write, a.workload, a.table)
    if a.alg_bytes_per_call:
        rec["alg_bytes_per_call"] = a.alg_bytes_per_call
        rec["traffic_over_alg"] = round(rec["traffic_bytes_per_call"] / a.alg_bytes_per_call, 4)
    if a.per_launch:
        for tag, folder in (("fetch", a.fetch), ("write", a.write)):
            print(f"== {rec[tag]['counter']} (calibrated)")
            print(per_launch_table(folder, rec[tag]["counter"], rec[tag]["factor"]))
    s = json.dumps(rec, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(s + "\n")
    print(s)


if __name__ == "__main__":
    sys.exit(main())
