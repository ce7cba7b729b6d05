"""Summaries of rocprofv3 output for the committed profiles.

    python -m paged_kv_prefill_amd.prof stats --csv RUN_kernel_stats.csv \\
        --bench-log LOG --cmd "..." --title "..." --out profiles/NAME.txt
    python -m paged_kv_prefill_amd.prof hbm --fetch-csv A_counter_collection.csv \\
        --write-csv B_counter_collection.csv --bench-log LOG \\
        --cmd-fetch "..." --cmd-write "..." --out profiles/NAME.txt

`stats` turns a --kernel-trace --stats summary into per-kernel call counts and
durations.  `hbm` turns two --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per
dispatch) into HBM bytes per attention launch, each counter scaled by what it
reads for the calibration gather in the same run (pa_gather_kv of a known
number of bytes, read once and written once).  The library build id is taken
from the bench JSON line in the log, so a summary names the exact build it
describes.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import statistics


def bench_library(log_path: str) -> str:
    lib = "unknown"
    for line in open(log_path, errors="replace"):
        line = line.strip()
        if line.startswith("{") and '"library"' in line:
            lib = json.loads(line)["library"]
    return lib


def bench_line(log_path: str) -> dict:
    for line in open(log_path, errors="replace"):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    return {}


def short_name(name: str) -> str:
    name = name.replace("void ", "")
    return name[:110]


def stats_summary(args) -> str:
    rows = list(csv.DictReader(open(args.csv)))
    out = [f"# {args.title}", f"command: {args.cmd}", f"library: {bench_library(args.bench_log)}",
           "", f"{'kernel':<112s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"{short_name(r['Name']):<112s} {int(r['Calls']):>6d} {float(r['AverageNs']) / 1e3:>10.1f} "
                   f"{float(r['MinNs']) / 1e3:>10.1f} {float(r['MaxNs']) / 1e3:>10.1f} "
                   f"{float(r['Percentage']):>6.1f}")
    b = bench_line(args.bench_log)
    if b:
        rl = b.get("roofline", {})
        out += ["", "bench (same command, HIP events on the launch stream):",
                f"  attention kernel alone: {rl.get('kernel_ms', 0) * 1e3:.1f} us per launch, "
                f"{rl.get('achieved', 0):.1f} TFLOP/s ({rl.get('frac', 0) * 100:.1f} % of the dense peak)",
                f"  whole call (V image pass + attention): {rl.get('call_ms', 0) * 1e3:.1f} us"]
    return "\n".join(out) + "\n"


def pmc_by_kernel(path: str, counter: str):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def pick(vals, key: str):
    hits = {k: v for k, v in vals.items() if key in k}
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {key!r}, found {list(hits)}")
    (name, v), = hits.items()
    return name, v


def hbm_summary(args) -> str:
    lib_f, lib_w = bench_library(args.bench_log_fetch), bench_library(args.bench_log_write)
    if lib_f != lib_w:
        raise SystemExit(f"the two counter runs used different builds: {lib_f} / {lib_w}")
    calib = bench_line(args.bench_log_fetch).get("calib_copy_bytes")
    if not calib:
        raise SystemExit("the fetch run has no calibration gather (run bench.py with --calib-copy)")
    f_vals = pmc_by_kernel(args.fetch_csv, "FETCH_SIZE")
    w_vals = pmc_by_kernel(args.write_csv, "WRITE_SIZE")
    ga, gf = pick(f_vals, "gather_kernel")
    _, gw = pick(w_vals, "gather_kernel")
    an, af = pick(f_vals, "attn_kernel")
    _, aw = pick(w_vals, "attn_kernel")
    ff = calib / (statistics.median(gf) * 1024)     # bytes per counted byte, reads
    fw = calib / (statistics.median(gw) * 1024)     # same, writes
    fetch_b = statistics.median(af) * 1024 * ff
    write_b = statistics.median(aw) * 1024 * fw
    out = ["# HBM bytes of the bf16 attention kernel, 20k-context 2,048-token chunk (head_dim 256)",
           f"command_fetch: {args.cmd_fetch}", f"command_write: {args.cmd_write}",
           f"library: {lib_f}", f"kernel: {short_name(an)}",
           f"calibration: {short_name(ga)} moving {calib} bytes; FETCH_SIZE median "
           f"{statistics.median(gf):.1f} KiB, WRITE_SIZE median {statistics.median(gw):.1f} KiB; "
           f"scale factors {ff:.4f} (fetch) {fw:.4f} (write)",
           f"attention FETCH_SIZE: median {statistics.median(af):.1f} KiB over {len(af)} dispatches "
           f"(min {min(af):.1f}, max {max(af):.1f})",
           f"attention WRITE_SIZE: median {statistics.median(aw):.1f} KiB over {len(aw)} dispatches "
           f"(min {min(aw):.1f}, max {max(aw):.1f})",
           f"fetch_bytes_per_launch: {fetch_b:.0f}",
           f"write_bytes_per_launch: {write_b:.0f}",
           f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}"]
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--bench-log", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    h = sub.add_parser("hbm")
    h.add_argument("--fetch-csv", required=True)
    h.add_argument("--write-csv", required=True)
    h.add_argument("--bench-log-fetch", required=True)
    h.add_argument("--bench-log-write", required=True)
    h.add_argument("--cmd-fetch", required=True)
    h.add_argument("--cmd-write", required=True)
    h.add_argument("--out", required=True)
    a = ap.parse_args()
    text = stats_summary(a) if a.what == "stats" else hbm_summary(a)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
