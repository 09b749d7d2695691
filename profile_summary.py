#!/usr/bin/env python3
"""Text summary of rocprofv3 result databases (SQLite, rocpd schema) written by bench runs.

  python3 profile_summary.py trace <run_results.db>
      per-kernel launches, total and average duration
  python3 profile_summary.py pmc <run_results.db> [kernel-substring]
      per-kernel average of each collected counter per dispatch
"""
import sqlite3
import sys


def trace(db):
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, count(*), sum(end - start), avg(end - start) from kernels group by name "
                          "order by sum(end - start) desc"))
    total = sum(r[2] for r in rows) or 1
    print(f"{'kernel':64s} {'calls':>6s} {'total_ms':>10s} {'avg_us':>10s} {'pct':>6s}")
    for name, n, tot, avg in rows:
        print(f"{name[:64]:64s} {n:6d} {tot / 1e6:10.3f} {avg / 1e3:10.2f} {100.0 * tot / total:6.1f}")


def pmc(db, pat=None):
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, counter_name, avg(counter_value), count(*) from pmc_events "
                          "group by name, counter_name order by name"))
    print(f"{'kernel':64s} {'counter':>12s} {'avg_per_dispatch':>18s} {'dispatches':>10s}")
    for name, cn, v, n in rows:
        if pat is None or pat in name:
            print(f"{name[:64]:64s} {cn:>12s} {v:18.1f} {n:10d}")


if __name__ == "__main__":
    mode, db = sys.argv[1], sys.argv[2]
    if mode == "trace":
        trace(db)
    else:
        pmc(db, sys.argv[3] if len(sys.argv) > 3 else None)
