"""Summaries of rocprofv3 output for this library's kernels.

    python -m generative_recommender_sequence_amd.profiling trace DIR
    python -m generative_recommender_sequence_amd.profiling pmc DIR [--copy DIR]
    python -m generative_recommender_sequence_amd.profiling traffic WORKLOAD FETCH_DIR WRITE_DIR --copy DIR

`trace` reads the *_kernel_trace.csv under DIR (rocprofv3 --kernel-trace
--output-format csv) and prints per (kernel, grid size) the number of
dispatches and their average / min / max duration.  Grouping by grid size
separates a benchmark's timed requests from its set-up launches of the same
kernel (different shapes give different grids).

`pmc` reads the *_counter_collection.csv under DIR (rocprofv3 --pmc ...) and
prints per (kernel, grid size) the mean of every counter.  With --copy DIR2
(the same counters collected on a plain device copy of known size, e.g.
`bench.py --calibrate-copy BYTES`), FETCH_SIZE / WRITE_SIZE are also scaled
by the ratio between the bytes the copy moved and what the counter read for
it, giving HBM bytes per dispatch.

`traffic` prints one line for the attention-traffic table the benchmark
reads: the workload, the grid of its timed attention launch (the attention
grid with the most dispatches), the calibrated FETCH_SIZE and WRITE_SIZE bytes
per launch, and a hash of the sources that decide what that launch reads and
writes (code only: comments and whitespace are ignored).  The benchmark
reports the figure only while the hash still matches.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import sys

_PKG = os.path.dirname(os.path.abspath(__file__))
# the attention kernel and the host scheduler that sizes its work items
TRAFFIC_SOURCES = ("csrc/kernels/attention.hip", "csrc/kernels/common.h", "csrc/internal.h",
                   "csrc/hstu_abi.cpp")
TRAFFIC_TABLE = os.path.join(os.path.dirname(_PKG), "profiles", "attention_traffic.txt")


def _code_only(text: str) -> str:
    """Source text without comments and whitespace (a comment edit does not
    change what a launch reads or writes)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def sources_hash() -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(_PKG, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """Calibrated HBM bytes (fetch + write) of the workload's attention launch,
    or None when the table has no line for it or the sources changed since."""
    if not os.path.exists(TRAFFIC_TABLE):
        return None
    cur = sources_hash()
    for line in open(TRAFFIC_TABLE):
        f = line.split()
        if len(f) == 5 and not line.startswith("#") and f[0] == workload and f[4] == cur:
            return float(f[2]) + float(f[3])
    return None


def _files(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def _short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    n = n.split("(")[0]
    return n[:70]


def trace_summary(d: str):
    rows = []
    for f in _files(d, "kernel_trace.csv"):
        rows += list(csv.DictReader(open(f)))
    groups = collections.defaultdict(list)
    for r in rows:
        grid = int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0)
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups[(_short(r["Kernel_Name"]), grid)].append(dur)
    out = []
    for (k, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append((k, grid, len(ds), sum(ds) / len(ds) / 1000.0, min(ds) / 1000.0, max(ds) / 1000.0,
                    sum(ds) / 1000.0))
    return out


def pmc_summary(d: str):
    rows = []
    for f in _files(d, "counter_collection.csv"):
        rows += list(csv.DictReader(open(f)))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    for r in rows:
        key = (_short(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
        did = r["Dispatch_Id"]
        per[key][(did, r["Counter_Name"])] += float(r["Counter_Value"])
        disp[key].add(did)
    out = {}
    for key, vals in per.items():
        n = len(disp[key])
        agg = collections.defaultdict(float)
        for (_, name), v in vals.items():
            agg[name] += v / n
        out[key] = (n, dict(agg))
    return out


def copy_factor(d: str, counter: str, bytes_moved: int) -> float:
    """bytes the copy moved / what `counter` (KiB) read for it (largest dispatch)."""
    best = 0.0
    for (k, grid), (n, agg) in pmc_summary(d).items():
        if counter in agg:
            best = max(best, agg[counter])
    return bytes_moved / (best * 1024.0) if best else float("nan")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["trace", "pmc", "traffic"])
    ap.add_argument("dir", help="trace/pmc: the output directory; traffic: the workload name")
    ap.add_argument("more", nargs="*", help="traffic: FETCH_SIZE and WRITE_SIZE directories")
    ap.add_argument("--copy", default=None, help="pmc directory of the calibration copy")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    a = ap.parse_args(argv)
    if a.mode == "trace":
        print("| kernel | grid | dispatches | avg us | min us | max us | total us |")
        print("|---|---:|---:|---:|---:|---:|---:|")
        for k, grid, n, avg, mn, mx, tot in trace_summary(a.dir):
            print(f"| {k} | {grid} | {n} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {tot:.1f} |")
        return
    if a.mode == "traffic":
        fdir, wdir = a.more
        fac = {c: copy_factor(os.path.join(a.copy, c), c, a.copy_bytes) for c in ("FETCH_SIZE", "WRITE_SIZE")}
        per = {}
        for c, d in (("FETCH_SIZE", fdir), ("WRITE_SIZE", wdir)):
            for (k, grid), (n, agg) in pmc_summary(d).items():
                if "attn_bf16_kernel" in k and c in agg:
                    per.setdefault(grid, {"n": n})[c] = agg[c] * 1024 * fac[c]
        grid = max(per, key=lambda g: per[g]["n"])
        print(f"{a.dir} {grid} {per[grid]['FETCH_SIZE']:.0f} {per[grid]['WRITE_SIZE']:.0f} {sources_hash()}")
        return
    fac = {}
    if a.copy:
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            sub = os.path.join(a.copy, c) if os.path.isdir(os.path.join(a.copy, c)) else a.copy
            fac[c] = copy_factor(sub, c, a.copy_bytes)
        print("copy calibration factors (bytes moved / counter bytes):",
              {k: round(v, 4) for k, v in fac.items()})
    for (k, grid), (n, agg) in sorted(pmc_summary(a.dir).items()):
        line = f"{k} grid={grid} dispatches={n}: " + ", ".join(f"{c}={v:.6g}" for c, v in sorted(agg.items()))
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in agg and c in fac:
                line += f", {c}_bytes={agg[c] * 1024 * fac[c]:.6g}"
        print(line)


if __name__ == "__main__":
    sys.exit(main())
