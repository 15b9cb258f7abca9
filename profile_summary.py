"""Condense rocprofv3 CSV output into the short summaries kept under profiles/.

    # per-kernel durations of a --kernel-trace --stats run
    python profile_summary.py stats \\
        --csv OUT_kernel_stats.csv --command "rocprofv3 ..." --out profiles/NAME.md

    # HBM bytes per step from two --pmc runs (FETCH_SIZE, then WRITE_SIZE), each
    # scaled by what the same counter reads for a plain device copy of known size
    # (bench.py --copy-calibration MIB); with several --kernel substrings the
    # step's kernels are summed (median per dispatch of each)
    python profile_summary.py counters \\
        --fetch A_counter_collection.csv --write B_counter_collection.csv \\
        --copy-fetch C_counter_collection.csv --copy-write D_counter_collection.csv \\
        --copy-bytes BYTES --kernel SUBSTRING [SUBSTRING ...] --key NAME \\
        --algorithmic-bytes N --commands "cmd1" "cmd2" "cmd3" "cmd4" \\
        [--sources scan_fwd.hip ...] --out-json profiles/hbm_counters.json --out profiles/NAME.md

    # per (kernel, grid, workgroup) durations of a --kernel-trace run
    python profile_summary.py dispatches --csv OUT_kernel_trace.csv [--match SUBSTRING ...] \\
        --title "..." --command "rocprofv3 ..." --out profiles/NAME.md

    # instruction and wait counters (SQ block) of one kernel, with per-update figures
    python profile_summary.py sq --csv A_counter_collection.csv [B_...csv] \\
        --kernel SUBSTRING --updates N --duration-us T --title "..." \\
        --commands "cmd1" ["cmd2"] --out profiles/NAME.md

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
    fetch = [_counter_per_dispatch(a.fetch, "FETCH_SIZE", k) for k in a.kernel]
    write = [_counter_per_dispatch(a.write, "WRITE_SIZE", k) for k in a.kernel]
    cf = _counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    cw = _counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    if not (all(fetch) and all(write) and cf and cw):
        sys.exit("no matching dispatches (kernel %r, copy %r)" % (a.kernel, a.copy_kernel))
    # scale: true bytes per counter KiB, from the copy of known size
    fscale = a.copy_bytes / (statistics.median(cf) * 1024.0)
    wscale = a.copy_bytes / (statistics.median(cw) * 1024.0)
    fmed = [statistics.median(v) for v in fetch]
    wmed = [statistics.median(v) for v in write]
    fb = sum(fmed) * 1024.0 * fscale
    wb = sum(wmed) * 1024.0 * wscale
    total = fb + wb
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from selective_state_space_59_amd import build
    sources = sorted(a.sources) if a.sources else None
    entry = dict(source_hash=build.source_hash(sources), sources=sources,
                 kernel=a.kernel[0] if len(a.kernel) == 1 else list(a.kernel),
                 bytes_per_launch=round(total),
                 fetch_bytes=round(fb), write_bytes=round(wb), fetch_scale=round(fscale, 4),
                 write_scale=round(wscale, 4), dispatches=len(fetch[0]),
                 algorithmic_bytes_per_launch=a.algorithmic_bytes)
    rec = {}
    if os.path.exists(a.out_json):
        with open(a.out_json) as f:
            rec = json.load(f)
    rec[a.key] = entry
    _write(a.out_json, json.dumps(rec, indent=1, sort_keys=True) + "\n")
    title = " + ".join("`%s`" % _short(k, 80) for k in a.kernel)
    lines = ["# HBM traffic of %s (%s)" % (title, a.key), "",
             "Commands (from the repository root):", "", "```"] + list(a.commands) + [
             "```", "",
             "| quantity | value |", "|---|---:|"]
    for k, fv, wv, fm, wm in zip(a.kernel, fetch, write, fmed, wmed):
        lines += ["| FETCH_SIZE per dispatch of `%s` (KiB, median of %d) | %.0f |" % (_short(k, 60), len(fv), fm),
                  "| WRITE_SIZE per dispatch of `%s` (KiB, median of %d) | %.0f |" % (_short(k, 60), len(wv), wm)]
    lines += ["| copy calibration: bytes copied | %d |" % a.copy_bytes,
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


def cmd_dispatches(a):
    """Per (kernel, grid, workgroup) durations from a --kernel-trace CSV: launches of one
    kernel instance with different shapes (different workloads) are kept apart."""
    import collections
    groups = collections.OrderedDict()
    for r in _rows(a.csv):
        if a.match and not any(m in r["Kernel_Name"] for m in a.match):
            continue
        key = (r["Kernel_Name"], r.get("Grid_Size_X", ""), r.get("Workgroup_Size_X", ""))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# %s" % a.title, "", "Command (from the repository root):", "", "```", a.command, "```", "",
             "| kernel | grid (work-items) | workgroup | launches | median us | mean us | min us | max us |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    for (name, grid, wg), v in groups.items():
        lines.append("| `%s` | %s | %s | %d | %.2f | %.2f | %.2f | %.2f |" % (
            _short(name, 90), grid, wg, len(v), statistics.median(v), sum(v) / len(v), min(v), max(v)))
    if a.note:
        lines += ["", a.note]
    _write(a.out, "\n".join(lines) + "\n")


SQ_NOTES = {
    "SQ_WAVES": "waves launched",
    "SQ_INSTS_VALU": "vector ALU instructions issued (per wave, all kinds)",
    "SQ_INSTS_VALU_TRANS_F32": "of which fp32 transcendentals (exp, rcp, ...)",
    "SQ_ACTIVE_INST_VALU": "wave-cycles executing VALU instructions",
    "SQ_WAVE_CYCLES": "wave-cycles resident",
    "SQ_WAIT_ANY": "wave-cycles waiting for anything",
    "SQ_WAIT_INST_LDS": "wave-cycles waiting to issue LDS instructions",
    "SQ_WAIT_INST_ANY": "wave-cycles waiting to issue any instruction",
    "SQ_INSTS_LDS": "LDS instructions",
    "SQ_LDS_BANK_CONFLICT": "LDS bank-conflict cycles",
    "SQ_INSTS_MFMA": "matrix-core instructions",
    "SQ_INSTS_SALU": "scalar ALU instructions",
    "SQ_INSTS_VMEM_RD": "vector memory reads",
}


def cmd_sq(a):
    vals = {}
    for path in a.csv:
        names = sorted({r["Counter_Name"] for r in _rows(path) if a.kernel in r.get("Kernel_Name", "")})
        for n in names:
            v = _counter_per_dispatch(path, n, a.kernel)
            if v:
                vals[n] = (statistics.median(v), len(v))
    if not vals:
        sys.exit("no dispatches of %r" % a.kernel)
    g = lambda n: vals[n][0] if n in vals else None
    lines = ["# %s" % a.title, "", "Commands (from the repository root):", "", "```"] + list(a.commands) + [
             "```", "", "Kernel: `%s`. Counters are per dispatch (median over dispatches), summed over "
             "the GPU." % _short(a.kernel, 100), "",
             "| counter | value | meaning |", "|---|---:|---|"]
    saturated = [n for n in sorted(vals) if abs(vals[n][0] - 2.0 ** 31) < 2.0]  # a 32-bit counter at its limit
    for n in sorted(vals):
        if n not in saturated:
            lines.append("| %s | %.4g | %s |" % (n, vals[n][0], SQ_NOTES.get(n, "")))
    if saturated:
        lines += ["", "Not shown, read at the 32-bit limit (2^31): %s." % ", ".join(saturated)]
    lines += ["", "| derived | value |", "|---|---:|"]
    if a.updates and g("SQ_INSTS_VALU") is not None:
        lines.append("| state updates per dispatch | %d |" % a.updates)
        lines.append("| VALU instructions per update (64 lanes each) | %.3f |"
                     % (g("SQ_INSTS_VALU") * 64 / a.updates))
        if g("SQ_INSTS_VALU_TRANS_F32") is not None:
            lines.append("| fp32 transcendentals per update (one exp is the core) | %.3f |"
                         % (g("SQ_INSTS_VALU_TRANS_F32") * 64 / a.updates))
        if g("SQ_INSTS_MFMA") is not None:
            lines.append("| MFMA instructions per update | %.4f |" % (g("SQ_INSTS_MFMA") * 64 / a.updates))
    if g("SQ_WAVE_CYCLES"):
        for n in ("SQ_WAIT_ANY", "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU"):
            if g(n) is not None:
                lines.append("| %s / SQ_WAVE_CYCLES | %.3f |" % (n, g(n) / g("SQ_WAVE_CYCLES")))
    if a.duration_us and g("SQ_INSTS_VALU") is not None:
        # issue cost model from microbenchmarks on gfx950 (4 waves per SIMD):
        # ~2 cycles per wave64 fp32 VALU instruction, 8 per fp32 transcendental;
        # 1024 SIMDs at 2.4 GHz
        trans = g("SQ_INSTS_VALU_TRANS_F32") or 0.0
        cyc = (g("SQ_INSTS_VALU") - trans) * 2.0 + trans * 8.0
        avail = 1024 * a.duration_us * 1e-6 * 2.4e9
        lines.append("| kernel duration (us, from the kernel trace) | %.2f |" % a.duration_us)
        lines.append("| VALU issue cycles / SIMD cycles (2 per instruction, 8 per transcendental) | %.3f |"
                     % (cyc / avail))
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
    for k in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--key", "--out-json", "--out"):
        c.add_argument(k, required=True)
    c.add_argument("--kernel", nargs="+", required=True,
                   help="kernel name substrings; the step's kernels are summed")
    c.add_argument("--copy-kernel", default="copyBuffer")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--algorithmic-bytes", type=int, required=True)
    c.add_argument("--commands", nargs="+", required=True)
    c.add_argument("--sources", nargs="+", default=None,
                   help="library sources the kernel is built from (file names under csrc/)")
    q = sub.add_parser("sq")
    q.add_argument("--csv", nargs="+", required=True)
    q.add_argument("--kernel", required=True)
    q.add_argument("--updates", type=int, default=0, help="state updates per dispatch")
    q.add_argument("--duration-us", type=float, default=0.0)
    q.add_argument("--title", required=True)
    q.add_argument("--commands", nargs="+", required=True)
    q.add_argument("--out", required=True)
    dd = sub.add_parser("dispatches")
    dd.add_argument("--csv", required=True, help="the kernel_trace.csv of a --kernel-trace run")
    dd.add_argument("--match", nargs="*", default=None, help="kernel name substrings to keep")
    dd.add_argument("--title", required=True)
    dd.add_argument("--command", required=True)
    dd.add_argument("--note", default="")
    dd.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "counters": cmd_counters, "sq": cmd_sq, "dispatches": cmd_dispatches}[a.cmd](a)


if __name__ == "__main__":
    main()
