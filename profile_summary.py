#!/usr/bin/env python3
"""Text summary of rocprofv3 result databases (SQLite, rocpd schema) written by bench runs.

  python3 profile_summary.py trace <run_results.db>
      per-kernel launches, total and average duration
  python3 profile_summary.py pmc <run_results.db> [kernel-substring]
      per-kernel average of each collected counter per dispatch
  python3 profile_summary.py sq <run_results.db> <kernel-substring>
      per-dispatch totals of SQ counters (one row per shader engine, 32 on MI355X) and GRBM_GUI_ACTIVE (one row
      per XCD, 8), with the vector-ALU busy fraction (a wave64 VALU instruction occupies a 16-lane SIMD for 4
      cycles; 1024 SIMDs), the share of wave cycles spent waiting, and LDS bank-conflict cycles per LDS instruction
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


def sq(db, pat):
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, counter_name, avg(counter_value), count(*) from pmc_events "
                          "group by name, counter_name order by name"))
    rows = [r for r in rows if pat in r[0]]
    if not rows:
        raise SystemExit(f"{db}: no kernel matching {pat!r}")
    name = rows[0][0]
    vals = {}
    for n, cn, v, cnt in rows:
        if n != name:
            continue
        per = 32 if cn.startswith("SQ_") else 8 if cn.startswith("GRBM_") else 1
        vals[cn] = (v * per if cn.startswith("SQ_") else v, cnt // per)
    print(f"kernel: {name}")
    for cn, (tot, nd) in sorted(vals.items()):
        print(f"{cn}: {tot:.4g}  (per dispatch, {nd} dispatches)")
    if "SQ_INSTS_VALU" in vals and "GRBM_GUI_ACTIVE" in vals:
        busy = vals["SQ_INSTS_VALU"][0] * 4 / (vals["GRBM_GUI_ACTIVE"][0] * 1024)
        print(f"derived valu_busy_fraction: {busy:.3f}  (SQ_INSTS_VALU x 4 cycles / (GRBM_GUI_ACTIVE x 1024 SIMDs))")
    if "SQ_WAIT_INST_ANY" in vals and "SQ_WAVE_CYCLES" in vals:
        print(f"derived wait_fraction: {vals['SQ_WAIT_INST_ANY'][0] / vals['SQ_WAVE_CYCLES'][0]:.3f}  "
              f"(SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)")
    if "SQ_LDS_BANK_CONFLICT" in vals and "SQ_INSTS_LDS" in vals and vals["SQ_INSTS_LDS"][0] > 0:
        print(f"derived lds_conflict_cycles_per_lds_inst: "
              f"{vals['SQ_LDS_BANK_CONFLICT'][0] / vals['SQ_INSTS_LDS'][0]:.2f}")


def _avg(db, counter, pat):
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, avg(counter_value), count(*) from pmc_events where counter_name = ? "
                          "group by name", (counter,)))
    rows = [r for r in rows if pat in r[0]]
    if len(rows) != 1:
        raise SystemExit(f"{db}: expected one kernel matching {pat!r} with {counter}, got {rows}")
    return rows[0][1], rows[0][2]


def traffic(kernel_pat, fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes, source_hash):
    """HBM bytes per dispatch of one kernel from FETCH_SIZE and WRITE_SIZE passes (KiB per dispatch), each
    scaled by what the same counter reads for a device copy of copy_bytes bytes."""
    f, nf = _avg(fetch_db, "FETCH_SIZE", kernel_pat)
    w, nw = _avg(write_db, "WRITE_SIZE", kernel_pat)
    cf, _ = _avg(copy_fetch_db, "FETCH_SIZE", "copyBuffer")
    cw, _ = _avg(copy_write_db, "WRITE_SIZE", "copyBuffer")
    kf = copy_bytes / (cf * 1024.0)
    kw = copy_bytes / (cw * 1024.0)
    print(f"kernel_pattern: {kernel_pat}")
    print(f"fetch_kib_per_dispatch: {f:.1f}  (dispatches {nf})")
    print(f"write_kib_per_dispatch: {w:.1f}  (dispatches {nw})")
    print(f"copy_fetch_kib_per_dispatch: {cf:.1f}")
    print(f"copy_write_kib_per_dispatch: {cw:.1f}")
    print(f"copy_bytes: {copy_bytes}")
    print(f"fetch_factor: {kf:.4f}")
    print(f"write_factor: {kw:.4f}")
    print(f"traffic_bytes_per_dispatch: {f * 1024.0 * kf + w * 1024.0 * kw:.0f}")
    print(f"source_sha256_16: {source_hash}")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "trace":
        trace(sys.argv[2])
    elif mode == "pmc":
        pmc(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else None)
    elif mode == "sq":
        sq(sys.argv[2], sys.argv[3])
    elif mode == "traffic":
        traffic(sys.argv[2], *sys.argv[3:7], int(sys.argv[7]), sys.argv[8])
