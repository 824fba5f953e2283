"""Summaries of rocprofv3 output for the committed profiles.

    python -m learned_kv_chunk_amd.profiling stats DIR --command "..." [--out FILE]
        per-kernel durations from a `rocprofv3 --kernel-trace --stats` run
        (DIR/run_kernel_stats.csv), as a Markdown table

    python -m learned_kv_chunk_amd.profiling traffic --kernel NAME --workload W \
            --source FILE --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
            --copy-bytes N --command "..." [--out-json FILE] [--out FILE]
        HBM-side bytes per launch of kernel NAME from two `--pmc` runs
        (FETCH_SIZE, then WRITE_SIZE; rocprofv3 reports both in KiB per
        dispatch), each scaled by what the same counter reads for a plain copy
        kernel that reads and writes N bytes per launch

    python -m learned_kv_chunk_amd.profiling counters DIR --kernel NAME ... --command "..."
        per-dispatch averages of every counter of a `--pmc` run for the named
        kernels, as a Markdown table (LDS bank conflicts, matrix-core busy
        cycles, ...)

All read only rocprofv3's CSV files.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def short_name(name: str) -> str:
    """Kernel name without namespaces and argument lists."""
    base = name.replace("(anonymous namespace)::", "").replace("lsa::", "")
    base = base.split("(")[0]
    return base[len("void "):] if base.startswith("void ") else base


def stats_table(run_dir: str) -> list[dict]:
    rows = _rows(os.path.join(run_dir, "run_kernel_stats.csv"))
    out = []
    for r in rows:
        out.append(dict(kernel=short_name(r["Name"]), calls=int(r["Calls"]),
                        avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                        max_us=float(r["MaxNs"]) / 1e3, pct=float(r["Percentage"])))
    return out


def counter_per_dispatch(run_dir: str, counter: str, kernel: str) -> list[float]:
    """Values of `counter` for every dispatch of kernels whose name contains
    `kernel` (the CSV holds one row per dispatch and counter)."""
    vals = []
    for r in _rows(os.path.join(run_dir, "run_counter_collection.csv")):
        if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel '{kernel}' in {run_dir}")
    return vals


def kernel_sources(kernel_file: str) -> list[str]:
    """A kernel's source file and every header it includes from this
    repository, recursively (first-seen order): a traffic record is valid
    only while all of them are unchanged."""
    import re

    out, todo = [], [kernel_file]
    while todo:
        f = todo.pop(0)
        if f in out or not os.path.exists(f):
            continue
        out.append(f)
        base = os.path.dirname(os.path.abspath(f))
        with open(f) as fh:
            for inc in re.findall(r'^\s*#\s*include\s+"([^"]+)"', fh.read(), flags=re.M):
                todo.append(os.path.relpath(os.path.normpath(os.path.join(base, inc))))
    return out


def source_hash(paths) -> str:
    """First 16 hex digits of the SHA-256 of the files' contents, in order."""
    if isinstance(paths, str):
        paths = [paths]
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cmd_stats(a) -> None:
    t = stats_table(a.dir)
    lines = [f"# Kernel durations: {a.title}", "", "Command:", "", "```", a.command, "```", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | share of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in t:
        lines.append(f"| {r['kernel']} | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['pct']:.1f}% |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def cmd_traffic(a) -> None:
    kib = 1024.0
    fetch = statistics.median(counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel)) * kib
    write = statistics.median(counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel)) * kib
    cf = statistics.median(counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)) * kib
    cw = statistics.median(counter_per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_kernel)) * kib
    f_scale = a.copy_bytes / cf      # true bytes per counted byte, reads
    w_scale = a.copy_bytes / cw      # and writes
    rec = {
        "kernel": a.kernel,
        "workload": a.workload,
        "kernel_source": [os.path.relpath(p) for p in kernel_sources(a.source)],
        "kernel_source_sha256_16": source_hash(kernel_sources(a.source)),
        "fetch_bytes_counted": fetch,
        "write_bytes_counted": write,
        "copy_calibration": {"bytes_read": a.copy_bytes, "bytes_written": a.copy_bytes,
                             "fetch_counted": cf, "write_counted": cw,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "read_bytes_per_launch": fetch * f_scale,
        "write_bytes_per_launch": write * w_scale,
        "bytes_per_launch": fetch * f_scale + write * w_scale,
        "command": a.command,
    }
    if a.out_json:
        with open(a.out_json, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    lines = [f"# HBM traffic of {a.kernel} on {a.workload}", "", "Commands:", "", "```",
             a.command, "```", "",
             "| quantity | bytes per launch |", "|---|---:|",
             f"| FETCH_SIZE (counted) | {fetch:.4g} |", f"| WRITE_SIZE (counted) | {write:.4g} |",
             f"| copy kernel FETCH_SIZE for {a.copy_bytes:.4g} B read | {cf:.4g} |",
             f"| copy kernel WRITE_SIZE for {a.copy_bytes:.4g} B written | {cw:.4g} |",
             f"| reads, calibrated (x{f_scale:.4f}) | {rec['read_bytes_per_launch']:.4g} |",
             f"| writes, calibrated (x{w_scale:.4f}) | {rec['write_bytes_per_launch']:.4g} |",
             f"| total | {rec['bytes_per_launch']:.4g} |", "",
             f"Kernel sources {', '.join(rec['kernel_source'])}: sha256[:16] of their "
             f"contents in that order = {rec['kernel_source_sha256_16']}."]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def cmd_counters(a) -> None:
    rows = _rows(os.path.join(a.dir, "run_counter_collection.csv"))
    table = {}
    for r in rows:
        name = short_name(r["Kernel_Name"])
        if not any(k in r["Kernel_Name"] for k in a.kernel):
            continue
        table.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(
            float(r["Counter_Value"]))
    counters = sorted({c for v in table.values() for c in v})
    lines = [f"# Counters: {a.title}", "", "Command:", "", "```", a.command, "```", "",
             "Per-dispatch averages as rocprofv3 reports them (summed over the device).", "",
             "| kernel | dispatches | " + " | ".join(counters) + " |",
             "|---|---:|" + "---:|" * len(counters)]
    for name, v in sorted(table.items()):
        n = max(len(x) for x in v.values())
        cells = [f"{statistics.mean(v[c]):.4g}" if c in v else "" for c in counters]
        lines.append(f"| {name} | {n} | " + " | ".join(cells) + " |")
    ratios = []
    for name, v in sorted(table.items()):
        if "SQ_LDS_BANK_CONFLICT" in v and "SQ_LDS_IDX_ACTIVE" in v:
            ratios.append(f"* {name}: LDS bank-conflict cycles / LDS active cycles = "
                          f"{statistics.mean(v['SQ_LDS_BANK_CONFLICT']) / max(1.0, statistics.mean(v['SQ_LDS_IDX_ACTIVE'])):.4f}")
    if ratios:
        lines += ["", "Ratios of the averages:", ""] + ratios
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", default="")
    s.add_argument("--command", required=True)
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="copy_kernel")
    t.add_argument("--workload", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--out-json")
    t.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--command", required=True)
    c.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        cmd_stats(a)
    elif a.cmd == "counters":
        cmd_counters(a)
    else:
        cmd_traffic(a)


if __name__ == "__main__":
    main()
