"""Summaries of rocprofv3 results (the rocpd SQLite database it writes) per kernel and grid size.

    python -m memory_bound_amd.profsum trace  <results.db>   # dispatch durations
    python -m memory_bound_amd.profsum pmc    <results.db>   # hardware counter values

rocprofv3's own --stats table groups dispatches by kernel name only; the same kernel
instantiation runs at several shapes here (the [2048,4096] and [16384,4096] Add+LayerNorm share
one), so the tables below also split by grid size.  Durations are in microseconds; counter values
are what rocprofv3 reports per dispatch (FETCH_SIZE and WRITE_SIZE in KiB).
"""
from __future__ import annotations

import sqlite3
import statistics
import sys
from collections import defaultdict


def short_name(name: str) -> str:
    i = name.rfind(">(")
    n = name[: i + 1] if i > 0 else name.split("(")[0]
    return n.replace("void ", "").replace("fuse::", "").replace("(anonymous namespace)::", "").replace("(DT)", "")


def trace(db_path: str) -> list[dict]:
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, grid_x, workgroup_x, duration from kernels order by start").fetchall()
    g = defaultdict(list)
    for name, gx, wx, dur in rows:
        g[(short_name(name), gx, wx)].append(dur / 1e3)
    out = []
    for (n, gx, wx), d in g.items():
        q = statistics.quantiles(d, n=10, method="inclusive") if len(d) > 1 else [d[0]] * 9
        out.append({"kernel": n, "grid": gx, "wg": wx, "calls": len(d), "mean_us": statistics.mean(d),
                    "median_us": statistics.median(d), "p10_us": q[0], "p90_us": q[8],
                    "min_us": min(d), "max_us": max(d)})
    return out


def pmc(db_path: str) -> list[dict]:
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, grid_size, workgroup_size, counter_name, value "
                      "from counters_collection order by dispatch_id").fetchall()
    g = defaultdict(list)
    for name, grid, wg, cname, val in rows:
        g[(short_name(name), grid, wg, cname)].append(val)
    out = []
    for (n, grid, wg, cname), v in g.items():
        out.append({"kernel": n, "grid": grid, "wg": wg, "counter": cname, "calls": len(v),
                    "mean": statistics.mean(v), "median": statistics.median(v), "min": min(v), "max": max(v)})
    return out


def main(argv):
    mode, path = argv[1], argv[2]
    if mode == "trace":
        print(f"{'kernel':64s} {'grid':>9s} {'wg':>4s} {'calls':>5s} {'mean_us':>9s} {'median_us':>9s} "
              f"{'p10_us':>8s} {'p90_us':>8s} {'min_us':>8s} {'max_us':>8s}")
        for r in trace(path):
            print(f"{r['kernel'][:64]:64s} {r['grid']:9d} {r['wg']:4d} {r['calls']:5d} {r['mean_us']:9.3f} "
                  f"{r['median_us']:9.3f} {r['p10_us']:8.3f} {r['p90_us']:8.3f} {r['min_us']:8.3f} "
                  f"{r['max_us']:8.3f}")
    elif mode == "pmc":
        print(f"{'kernel':64s} {'grid':>9s} {'counter':>11s} {'calls':>5s} {'mean':>12s} {'median':>12s}")
        for r in pmc(path):
            print(f"{r['kernel'][:64]:64s} {r['grid']:9d} {r['counter']:>11s} {r['calls']:5d} {r['mean']:12.2f} "
                  f"{r['median']:12.2f}")
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
