"""Summarise a rocprofv3 kernel trace: per-kernel dispatch count and durations.

Usage:
    python -m streaming_causal_video_amd.profsum <results.db | kernel_trace.csv> [--last N]

``--last N`` restricts each kernel to its last N dispatches (the steady-state
part of a streamed run, after the ring has filled); ``--slice A:B`` to its
dispatches A..B-1 in launch order (for a run that launches the same kernel again
after the part of interest, e.g. bench.py's standalone HBM timings after the
step).  Reads the SQLite database
that rocprofv3 writes by default or the CSV kernel trace of
``--output-format csv``.
"""

from __future__ import annotations

import argparse
import csv
import re
import sqlite3
import statistics
import sys


def short_name(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"\(.*", "", n)
    return n[:60]


def load(path: str):
    """[(kernel name, start_ns, end_ns)] in dispatch order."""
    if path.endswith(".db"):
        con = sqlite3.connect(path)
        rows = con.execute("select name, start, end from kernels order by start").fetchall()
        return [(r[0], int(r[1]), int(r[2])) for r in rows]
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((r["Kernel_Name"], int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    out.sort(key=lambda t: t[1])
    return out


def summarise(rows, last=None, window=None):
    by = {}
    for name, s, e in rows:
        by.setdefault(name, []).append((e - s) / 1e3)
    res = []
    for name, d in by.items():
        sel = d[window[0]:window[1]] if window else (d[-last:] if last else d)
        if not sel:
            continue
        res.append((short_name(name), len(d), len(sel), sum(sel), statistics.mean(sel),
                    statistics.median(sel), min(sel), max(sel)))
    res.sort(key=lambda r: -r[3])
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("trace")
    ap.add_argument("--last", type=int, default=None)
    ap.add_argument("--slice", default=None, help="A:B, dispatches A..B-1 of each kernel")
    a = ap.parse_args(argv)
    window = tuple(int(x) for x in a.slice.split(":")) if a.slice else None
    rows = summarise(load(a.trace), a.last, window)
    tot = sum(r[3] for r in rows)
    print(f"{'kernel':60s} {'calls':>6s} {'used':>5s} {'avg_us':>10s} {'median_us':>10s} "
          f"{'min_us':>9s} {'max_us':>9s} {'pct':>6s}")
    for n, calls, used, s, avg, med, mn, mx in rows:
        print(f"{n:60s} {calls:6d} {used:5d} {avg:10.2f} {med:10.2f} {mn:9.2f} {mx:9.2f} "
              f"{100 * s / tot:6.2f}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
