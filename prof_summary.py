"""Summaries of rocprofv3 runs of bench.py, written under profiles/.

  python prof_summary.py stats DIR OUT.txt --cmd "..."
      per-kernel dispatch counts and durations from a --kernel-trace run
  python prof_summary.py counters DIR[,DIR2] OUT.txt --kernel NAME --cmd "..." [--units U --unit-name S]
      per-dispatch averages of every counter a --pmc run collected for one kernel,
      by grid size, with the LDS bank-conflict and matrix-core busy fractions
  python prof_summary.py traffic FETCH_DIR WRITE_DIR OUT.json --workload NAME --cmd "..."
      HBM bytes per phase-A launch (and per finish launch) from two --pmc runs
      (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads for
      bench.py's known-size copy

DIR holds the rocpd SQLite database(s) rocprofv3 wrote (-d DIR).
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import re
import sqlite3
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
PHASE_A = "phase_a_kernel"
FINISH = "finish_kernel"
CALIB = "neg"                     # bench.calibration_copy: torch.neg over 1 GiB of float32
CALIB_BYTES = 1 << 30


def short(name: str) -> str:
    n = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("rtp::", "")
    return re.sub(r"\(.*", "", n)


def dbs(d: str):
    out = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not out:
        sys.exit(f"no rocpd database under {d}")
    return out


def kernel_rows(d: str):
    rows = []
    for db in dbs(d):
        con = sqlite3.connect(db)
        rows += con.execute("select name, grid_x / workgroup_x, duration from kernels").fetchall()
    return rows


def counter_rows(d: str, counter: str):
    """(kernel name, value in KiB) per dispatch, summed over the device's instances."""
    per = defaultdict(float)
    names = {}
    for db in dbs(d):
        con = sqlite3.connect(db)
        q = ("select k.dispatch_id, k.name, c.value from counters_collection c "
             "join kernels k on c.dispatch_id = k.dispatch_id where c.counter_name = ?")
        for did, name, v in con.execute(q, (counter,)).fetchall():
            per[(db, did)] += v
            names[(db, did)] = name
    return [(names[k], v) for k, v in per.items()]


def cmd_stats(a):
    rows = kernel_rows(a.dir)
    agg = defaultdict(list)
    for name, grid, dur in rows:
        agg[(short(name), grid)].append(dur)
    total = sum(sum(v) for v in agg.values())
    lines = [f"# rocprofv3 kernel trace: {a.title}", "", "command:", f"    {a.cmd}", "",
             f"{'kernel':60s} {'grid':>8s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for (n, g), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{n[:60]:60s} {g:8d} {len(v):6d} {sum(v) / len(v) / 1e3:9.2f} {min(v) / 1e3:9.2f} "
                     f"{max(v) / 1e3:9.2f} {100 * sum(v) / total:6.2f}")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


CUS, SIMDS, CLOCK_HZ = 256, 1024, 2.4e9
WAVE_SLOTS = 4 * SIMDS            # the decode kernels are built for 4 waves per SIMD (128 VGPRs)


def cmd_counters(a):
    """Averages per dispatch (counters summed over the device's instances)."""
    per = defaultdict(float)
    info = {}
    for db in [x for d in a.dir.split(",") for x in dbs(d)]:
        con = sqlite3.connect(db)
        q = ("select c.dispatch_id, k.name, k.grid_x / k.workgroup_x, k.duration, c.counter_name, c.value "
             "from counters_collection c join kernels k on c.dispatch_id = k.dispatch_id")
        for did, name, grid, dur, cn, v in con.execute(q).fetchall():
            if a.kernel not in name:
                continue
            per[(db, did, cn)] += v
            info[(db, did)] = (grid, dur)
    groups = defaultdict(lambda: defaultdict(list))
    for (db, did, cn), v in per.items():
        groups[info[(db, did)][0]][cn].append(v)
    for grid, dur in info.values():
        groups[grid]["_dur"].append(dur)
    lines = [f"# rocprofv3 counters: {a.title or a.kernel}", "", "command:", f"    {a.cmd}", "",
             "per dispatch, averaged over the dispatches of each grid size; fractions use",
             f"{CUS} CUs / {SIMDS} SIMDs at {CLOCK_HZ / 1e9:.1f} GHz over the dispatch's duration", ""]
    for grid in sorted(groups):
        c = groups[grid]
        dur_ns = sum(c["_dur"]) / len(c["_dur"])
        cyc = dur_ns * 1e-9 * CLOCK_HZ
        lines.append(f"{a.kernel}  grid {grid} workgroups  ({len(c['_dur'])} dispatches, avg {dur_ns / 1e6:.3f} ms)")
        for cn in sorted(k for k in c if k != "_dur"):
            lines.append(f"    {cn:32s} {sum(c[cn]) / len(c[cn]):14.4g}")
        if "SQ_LDS_BANK_CONFLICT" in c:
            v = sum(c["SQ_LDS_BANK_CONFLICT"]) / len(c["SQ_LDS_BANK_CONFLICT"])
            lines.append(f"    LDS bank-conflict stall / CU cycles  {v / CUS / cyc:.3f}")
        # SQ_WAVE_CYCLES and SQ_ACTIVE_INST_* count in units of 4 cycles (one wave64
        # VALU instruction occupies a 16-lane SIMD for 4 cycles)
        if "SQ_ACTIVE_INST_VALU" in c:
            v = sum(c["SQ_ACTIVE_INST_VALU"]) / len(c["SQ_ACTIVE_INST_VALU"])
            lines.append(f"    VALU busy / SIMD cycles              {4 * v / SIMDS / cyc:.3f}")
        if "SQ_ACTIVE_INST_LDS" in c:
            v = sum(c["SQ_ACTIVE_INST_LDS"]) / len(c["SQ_ACTIVE_INST_LDS"])
            lines.append(f"    LDS instruction issue / SIMD cycles  {4 * v / SIMDS / cyc:.3f}")
        if "SQ_WAVE_CYCLES" in c:
            v = sum(c["SQ_WAVE_CYCLES"]) / len(c["SQ_WAVE_CYCLES"])
            lines.append(f"    mean resident waves                  {4 * v / cyc:.0f} "
                         f"(of {WAVE_SLOTS} at 4 waves per SIMD: {4 * v / cyc / WAVE_SLOTS:.3f})")
        if "SQ_INSTS_VALU" in c and a.units:
            v = sum(c["SQ_INSTS_VALU"]) / len(c["SQ_INSTS_VALU"])
            lines.append(f"    VALU lane-instructions per {a.unit_name:10s} {64 * v / a.units:.1f}")
            for cn in ("SQ_INSTS_VALU_FMA_F64", "SQ_INSTS_VALU_CVT", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD"):
                if cn in c:
                    v = sum(c[cn]) / len(c[cn])
                    lines.append(f"    {cn + ' lanes per ' + a.unit_name:38s} {64 * v / a.units:.2f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            v = sum(c["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(c["SQ_VALU_MFMA_BUSY_CYCLES"])
            lines.append(f"    matrix-core busy / SIMD cycles       {v / SIMDS / cyc:.3f}")
        lines.append("")
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def mean_kib(rows, pred):
    v = [x for n, x in rows if pred(short(n))]
    if not v:
        return None, 0
    return sum(v) / len(v), len(v)


def cmd_traffic(a):
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash

    fetch = counter_rows(a.fetch_dir, "FETCH_SIZE")
    write = counter_rows(a.write_dir, "WRITE_SIZE")
    is_pa = lambda n: n.startswith(PHASE_A)
    is_cal = lambda n: "elementwise" in n and CALIB in n and "FillFunctor" not in n
    f_pa, nf = mean_kib(fetch, is_pa)
    w_pa, nw = mean_kib(write, is_pa)
    f_cal, ncf = mean_kib(fetch, is_cal)
    w_cal, ncw = mean_kib(write, is_cal)
    if None in (f_pa, w_pa, f_cal, w_cal):
        sys.exit(f"missing dispatches: phase A {nf}/{nw}, calibration copy {ncf}/{ncw}")
    s_fetch = CALIB_BYTES / (f_cal * 1024)
    s_write = CALIB_BYTES / (w_cal * 1024)
    rd = f_pa * 1024 * s_fetch
    wr = w_pa * 1024 * s_write
    out = {"kernel": PHASE_A, "workload": a.workload, "kernel_source_hash": kernel_source_hash(),
           "fetch_kib_per_launch": round(f_pa, 1), "write_kib_per_launch": round(w_pa, 1),
           "launches": [nf, nw],
           "calibration": {"kernel": "torch.neg over 1 GiB float32 (reads 1 GiB, writes 1 GiB)",
                           "fetch_kib": round(f_cal, 1), "write_kib": round(w_cal, 1),
                           "fetch_scale": round(s_fetch, 4), "write_scale": round(s_write, 4)},
           "read_bytes_per_launch": int(rd), "write_bytes_per_launch": int(wr),
           "bytes_per_launch": int(rd + wr), "commands": a.cmd}
    # the step's other kernel, from the same passes and scales
    f_fi, nff = mean_kib(fetch, lambda n: n.startswith(FINISH))
    w_fi, nfw = mean_kib(write, lambda n: n.startswith(FINISH))
    if f_fi is not None and w_fi is not None:
        out["other_kernels"] = {FINISH: {"launches": [nff, nfw], "fetch_kib_per_launch": round(f_fi, 1),
                                         "write_kib_per_launch": round(w_fi, 1),
                                         "read_bytes_per_launch": int(f_fi * 1024 * s_fetch),
                                         "write_bytes_per_launch": int(w_fi * 1024 * s_write)}}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    sp = ap.add_subparsers(dest="what", required=True)
    s = sp.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    c = sp.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("out")
    c.add_argument("--kernel", required=True)
    c.add_argument("--units", type=float, default=0.0, help="work units per dispatch (e.g. indexer scores)")
    c.add_argument("--unit-name", default="unit")
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", default="")
    t = sp.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("out")
    t.add_argument("--workload", required=True)
    t.add_argument("--cmd", action="append", required=True)
    a = ap.parse_args()
    {"stats": cmd_stats, "counters": cmd_counters, "traffic": cmd_traffic}[a.what](a)


if __name__ == "__main__":
    main()
