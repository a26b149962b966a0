"""Summarise rocprofv3 results of bench.py runs into short text files.

Reads the SQLite databases rocprofv3 writes (``<dir>/run_results.db``) for
  * a ``--kernel-trace --stats`` run  -> per-kernel calls / average duration,
  * a ``--pmc FETCH_SIZE`` run and a ``--pmc WRITE_SIZE`` run -> KiB per dispatch.
The HBM counters are scaled by what they read for a device copy of known size
made by the same bench command (``--calib-copy-mib``): the copy kernel with the
largest WRITE_SIZE is taken as the calibration dispatch, its expected read and
write sizes are the calibration size.

The bench command is expected to measure one workload (``--secondary none``);
the decode kernel with the largest total time in the trace is the one
summarised.  Writes ``profiles/<kernel>_<workload>.md`` and
``profiles/traffic_<workload>.json`` (HBM bytes per launch, keyed by the
kernel-source hash printed by bench.py so that stale counters are not used).

With ``--sq DIR ...`` (runs with SQ / GRBM counters, ``--command-sq`` giving
their commands in the same order) it adds, for the same kernel, the MFMA
pipes' busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs times the
kernel's cycles, GRBM_GUI_ACTIVE / 8 XCDs), the MFMA flops counted by
SQ_INSTS_VALU_MFMA_MOPS_* (units of 512), the share of LDS cycles lost to bank
conflicts, and where the waves spent their cycles.

usage: python profile_summary.py --stats DIR --fetch DIR
       --write DIR --bench-log FILE --calib-mib N --out profiles --command-stats "..."
       --command-fetch "..." --command-write "..." [--sq DIR ... --command-sq "..." ...]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sqlite3

def _db(d):
    p = os.path.join(d, "run_results.db")
    if not os.path.exists(p):
        cands = [f for f in os.listdir(d) if f.endswith(".db")]
        p = os.path.join(d, cands[0])
    return sqlite3.connect(p)


def kernel_stats(d):
    cur = _db(d).cursor()
    return cur.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels order by total_duration desc").fetchall()


def counter_avgs(d, counter):
    cur = _db(d).cursor()
    rows = cur.execute("select kernel_name, count(*), avg(value), max(value) from "
                       "counters_collection where counter_name = ? group by kernel_name",
                       (counter,)).fetchall()
    return {r[0]: dict(n=r[1], avg=r[2], max=r[3]) for r in rows}


def all_counters(d):
    cur = _db(d).cursor()
    rows = cur.execute("select kernel_name, counter_name, avg(value) from counters_collection "
                       "group by kernel_name, counter_name").fetchall()
    out = {}
    for k, c, v in rows:
        out.setdefault(k, {})[c] = v
    return out


N_XCD, N_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def sq_section(kname, sq_dirs, commands, flops, avg_us):
    """Markdown lines of the SQ / GRBM counters of kernel kname (per dispatch,
    averaged over the dispatches of each run)."""
    c = {}
    for d in sq_dirs:
        for k, vals in all_counters(d).items():
            if kname in k:
                c.update(vals)
    if not c:
        return []
    lines = ["", "## Matrix cores, LDS and wave states of `%s` (per launch)" % kname, "",
             "Counter commands (one pass each):", ""] + ["    " + x for x in commands] + [
             "", "| quantity | value |", "|---|---|"]
    for name in sorted(c):
        lines.append("| %s | %.4g |" % (name, c[name]))
    cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
    busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES")
    derived = []
    if cyc > 0 and busy is not None:
        derived.append(("kernel cycles (GRBM_GUI_ACTIVE / %d XCDs)" % N_XCD, "%.0f" % cyc))
        derived.append(("MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x cycles)" % N_SIMD,
                        "%.1f %%" % (100.0 * busy / (N_SIMD * cyc))))
        if c.get("SQ_INSTS_MFMA"):
            derived.append(("busy cycles per MFMA instruction", "%.1f" % (busy / c["SQ_INSTS_MFMA"])))
    mops = sum(v for k, v in c.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    if mops:
        derived.append(("MFMA flops counted (MOPS x 512)", "%.4g" % (mops * 512)))
        if flops:
            derived.append(("algorithmic flops of the launch", "%.4g" % flops))
        if avg_us:
            derived.append(("MFMA TFLOP/s at the traced duration", "%.1f" % (mops * 512 / avg_us / 1e6)))
    if c.get("SQ_LDS_IDX_ACTIVE"):
        derived.append(("LDS bank-conflict cycles / LDS active cycles", "%.1f %%" % (
            100.0 * c.get("SQ_LDS_BANK_CONFLICT", 0.0) / c["SQ_LDS_IDX_ACTIVE"])))
    wc = c.get("SQ_WAVE_CYCLES")
    if wc:
        for k in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_ANY",
                  "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
            if k in c:
                derived.append(("%s / SQ_WAVE_CYCLES" % k, "%.1f %%" % (100.0 * c[k] / wc)))
    if derived:
        lines += ["", "| derived | value |", "|---|---|"]
        lines += ["| %s | %s |" % d for d in derived]
    return lines


def short(name):
    m = re.search(r"(mla_[a-z0-9_]+_kernel(<[^>]*>)?)", name)
    if m:
        return m.group(1)
    return name if len(name) <= 100 else name[:100] + "..."


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--bench-log", required=True)
    ap.add_argument("--calib-mib", type=int, required=True)
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--command-stats", required=True)
    ap.add_argument("--command-fetch", required=True)
    ap.add_argument("--command-write", required=True)
    ap.add_argument("--sq", nargs="*", default=[])
    ap.add_argument("--command-sq", nargs="*", default=[])
    args = ap.parse_args()

    bench = None
    for line in open(args.bench_log):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            bench = json.loads(line)
    sha = bench["config"].get("kernel_sha") if bench else None

    stats = kernel_stats(args.stats)
    fetch = counter_avgs(args.fetch, "FETCH_SIZE")
    write = counter_avgs(args.write, "WRITE_SIZE")
    calib_kib = args.calib_mib * 1024.0
    copy_f = max((v for k, v in fetch.items() if "copyBuffer" in k), key=lambda v: v["max"])
    copy_w = max((v for k, v in write.items() if "copyBuffer" in k), key=lambda v: v["max"])
    f_scale = calib_kib / copy_f["max"]
    w_scale = calib_kib / copy_w["max"]

    os.makedirs(args.out, exist_ok=True)
    table = ["| kernel | calls | avg us | total us | % |", "|---|---|---|---|---|"]
    for name, calls, tot, avg, pct in stats:
        table.append("| `%s` | %d | %.2f | %.1f | %.1f |" % (short(name), calls, avg, tot, pct))

    workload = bench["config"]["workload"]
    decode = [st for st in stats if "mla_decode_" in st[0]]
    if decode:
        kname = short(max(decode, key=lambda st: st[2])[0])
        full = [n for n in fetch if kname in n]
        if not full:
            raise SystemExit("no counters for " + kname)
        fk = fetch[full[0]]
        wk = write.get(full[0])
        avg_us = [s[3] for s in stats if kname in s[0]]
        fetch_b = fk["avg"] * f_scale * 1024.0
        write_b = (wk["avg"] * w_scale * 1024.0) if wk else 0.0
        alg = bench["config"]["algorithmic_bytes"]
        lines = [
            "# `%s` on `%s`" % (kname, workload), "",
            "rocprofv3 summaries of `bench.py` runs on one MI355X (gfx950).", "",
            "Kernel trace + stats command:", "", "    " + args.command_stats, "",
            "Counter commands (one pass each):", "", "    " + args.command_fetch,
            "    " + args.command_write, "",
            "## Kernel durations (kernel-trace --stats, all kernels of the run)", "",
        ] + table + [
            "",
            "## HBM traffic of `%s` (per launch)" % kname, "",
            "| quantity | value |", "|---|---|",
            "| average duration (us) | %s |" % ("%.2f" % avg_us[0] if avg_us else "n/a"),
            "| FETCH_SIZE raw (KiB / dispatch) | %.1f |" % fk["avg"],
            "| WRITE_SIZE raw (KiB / dispatch) | %.1f |" % (wk["avg"] if wk else 0.0),
            "| calibration: %d MiB device copy reads FETCH_SIZE | %.1f KiB (scale %.4f) |"
            % (args.calib_mib, copy_f["max"], f_scale),
            "| calibration: same copy WRITE_SIZE | %.1f KiB (scale %.4f) |"
            % (copy_w["max"], w_scale),
            "| HBM bytes read (scaled) | %.0f |" % fetch_b,
            "| HBM bytes written (scaled) | %.0f |" % write_b,
        ]
        lines.append("| algorithmic bytes (inputs + outputs once) | %d |" % alg)
        lines.append("| traffic / algorithmic | %.3f |" % ((fetch_b + write_b) / alg))
        lines += sq_section(kname, args.sq, args.command_sq, bench["config"].get("flops"),
                            avg_us[0] if avg_us else None)
        lines.append("")
        lines.append("kernel source hash (bench.py `kernel_sha`): `%s`" % sha)
        with open(os.path.join(args.out, "%s_%s.md" % (re.sub(r"[^a-z0-9_]", "", kname.split("<")[0]),
                                                        workload)), "w") as f:
            f.write("\n".join(lines) + "\n")
        with open(os.path.join(args.out, "traffic_%s.json" % workload), "w") as f:
            json.dump({"kernel": kname, "workload": workload, "kernel_sha": sha,
                       "hbm_read_bytes_per_launch": round(fetch_b),
                       "hbm_write_bytes_per_launch": round(write_b),
                       "hbm_bytes_per_launch": round(fetch_b + write_b),
                       "fetch_scale": f_scale, "write_scale": w_scale,
                       "avg_duration_us": avg_us[0] if avg_us else None}, f, indent=1)
        print("wrote", kname, workload)


if __name__ == "__main__":
    main()
