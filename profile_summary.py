"""Condense rocprofv3 CSV output into the short summaries kept under profiles/.

    # per-kernel durations of a --kernel-trace --stats run
    python profile_summary.py stats \\
        --csv OUT_kernel_stats.csv --command "rocprofv3 ..." --out profiles/NAME.md

    # HBM bytes per launch of one kernel from two --pmc runs (FETCH_SIZE, then
    # WRITE_SIZE), each scaled by what the same counter reads for a plain
    # device copy of known size (bench.py --copy-calibration MIB)
    python profile_summary.py counters \\
        --fetch A_counter_collection.csv --write B_counter_collection.csv \\
        --copy-fetch C_counter_collection.csv --copy-write D_counter_collection.csv \\
        --copy-bytes BYTES --kernel SUBSTRING --key NAME --algorithmic-bytes N \\
        --commands "cmd1" "cmd2" "cmd3" "cmd4" [--sources scan_fwd.hip ...] \\
        --out-json profiles/hbm_counters.json --out profiles/NAME.md

FETCH_SIZE and WRITE_SIZE are reported in KiB per dispatch.  The JSON entry
names the library sources the kernel is built from (--sources, file names
under csrc/; default: all) and carries their hash with the compile flags;
bench.py uses it only while that hash matches the current sources.
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import statistics
import sys


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name, width=110):
    return name if len(name) <= width else name[:width - 3] + "..."


def cmd_stats(a):
    rows = _rows(a.csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# %s" % a.title, "", "Command (from the repository root):", "",
             "```", a.command, "```", "",
             "| kernel | calls | avg us | min us | max us | share % |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:a.top]:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    _write(a.out, "\n".join(lines) + "\n")


def _counter_per_dispatch(path, counter, match):
    vals = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter or match not in r.get("Kernel_Name", ""):
            continue
        d = r["Dispatch_Id"]
        vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def cmd_counters(a):
    fetch = _counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)
    write = _counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)
    cf = _counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw = _counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    if not (fetch and write and cf and cw):
        sys.exit("no matching dispatches (kernel %r, copy %r)" % (a.kernel, a.copy_kernel))
    # scale: true bytes per counter KiB, from the copy of known size
    fscale = a.copy_bytes / (statistics.median(cf) * 1024.0)
    wscale = a.copy_bytes / (statistics.median(cw) * 1024.0)
    fb = statistics.median(fetch) * 1024.0 * fscale
    wb = statistics.median(write) * 1024.0 * wscale
    total = fb + wb
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from selective_state_space_59_amd import build
    sources = sorted(a.sources) if a.sources else None
    entry = dict(source_hash=build.source_hash(sources), sources=sources, kernel=a.kernel,
                 bytes_per_launch=round(total),
                 fetch_bytes=round(fb), write_bytes=round(wb), fetch_scale=round(fscale, 4),
                 write_scale=round(wscale, 4), dispatches=len(fetch),
                 algorithmic_bytes_per_launch=a.algorithmic_bytes)
    rec = {}
    if os.path.exists(a.out_json):
        with open(a.out_json) as f:
            rec = json.load(f)
    rec[a.key] = entry
    _write(a.out_json, json.dumps(rec, indent=1, sort_keys=True) + "\n")
    lines = ["# HBM traffic of `%s` (%s)" % (_short(a.kernel, 80), a.key), "",
             "Commands (from the repository root):", "", "```"] + list(a.commands) + [
             "```", "",
             "| quantity | value |", "|---|---:|",
             "| FETCH_SIZE per dispatch (KiB, median of %d) | %.0f |" % (len(fetch), statistics.median(fetch)),
             "| WRITE_SIZE per dispatch (KiB, median of %d) | %.0f |" % (len(write), statistics.median(write)),
             "| copy calibration: bytes copied | %d |" % a.copy_bytes,
             "| copy calibration: FETCH_SIZE (KiB) | %.0f |" % statistics.median(cf),
             "| copy calibration: WRITE_SIZE (KiB) | %.0f |" % statistics.median(cw),
             "| fetch scale (bytes per counted byte) | %.4f |" % fscale,
             "| write scale (bytes per counted byte) | %.4f |" % wscale,
             "| HBM bytes read per launch | %.0f |" % fb,
             "| HBM bytes written per launch | %.0f |" % wb,
             "| HBM bytes per launch | %.0f |" % total,
             "| algorithmic bytes per launch | %d |" % a.algorithmic_bytes,
             "| traffic / algorithmic | %.4f |" % (total / a.algorithmic_bytes),
             "| hash of the kernel's sources (%s; code only) and flags | %s |"
             % (", ".join(sources) if sources else "all library sources", entry["source_hash"])]
    _write(a.out, "\n".join(lines) + "\n")


def _write(path, text):
    d = os.path.dirname(path)
    if d:
        os.makedirs(d, exist_ok=True)
    with open(path, "w") as f:
        f.write(text)
    print("wrote", path)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="Kernel durations (rocprofv3 --kernel-trace --stats)")
    s.add_argument("--top", type=int, default=12)
    c = sub.add_parser("counters")
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--kernel", "--key",
              "--out-json", "--out"):
        c.add_argument(k, required=True)
    c.add_argument("--copy-kernel", default="copyBuffer")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--algorithmic-bytes", type=int, required=True)
    c.add_argument("--commands", nargs="+", required=True)
    c.add_argument("--sources", nargs="+", default=None,
                   help="library sources the kernel is built from (file names under csrc/)")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
