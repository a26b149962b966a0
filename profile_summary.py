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

usage: python profile_summary.py --stats DIR --fetch DIR
       --write DIR --bench-log FILE --calib-mib N --out profiles --command-stats "..."
       --command-fetch "..." --command-write "..."
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
