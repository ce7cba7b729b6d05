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
number of bytes, read once and written once).  `passes` does the same for every
library kernel of a run over all arms, with each kernel's mean duration from
a kernel trace of the same command, as GB/s against the 8 TB/s HBM peak.
`mfma` turns a --pmc run of MFMA counters into, per attention kernel instance
and grid size: MFMA busy share of the SIMD cycles, the effective shader clock,
and the matrix operations the hardware counted (in TFLOP/s and against the
data-sheet peak).  The library build id is taken from the bench JSON line in
the log, so a summary names the exact build it describes.

    python -m paged_kv_prefill_amd.prof passes --fetch-csv ... --write-csv ... \
        --trace-csv RUN_kernel_stats.csv --bench-log-fetch ... --bench-log-write ... \
        --cmd-fetch ... --cmd-write ... --cmd-trace ... --out profiles/NAME.txt
    python -m paged_kv_prefill_amd.prof mfma --csv A_counter_collection.csv \
        --bench-log LOG --cmd "..." --out profiles/NAME.txt
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


PEAK_HBM_BYTES_S = 8.0e12
PEAK_MFMA_TFLOPS = {"bf16/f16": 2500.0, "i8": 5000.0}
N_SIMD = 1024         # 256 CUs x 4 SIMDs
N_XCD = 8


def calib_factors(f_vals, w_vals, calib):
    _, gf = pick(f_vals, "gather_kernel")
    _, gw = pick(w_vals, "gather_kernel")
    return calib / (statistics.median(gf) * 1024), calib / (statistics.median(gw) * 1024)


def passes_summary(args) -> str:
    lib_f, lib_w = bench_library(args.bench_log_fetch), bench_library(args.bench_log_write)
    if lib_f != lib_w:
        raise SystemExit(f"the two counter runs used different builds: {lib_f} / {lib_w}")
    calib = bench_line(args.bench_log_fetch).get("calib_copy_bytes")
    if not calib:
        raise SystemExit("the fetch run has no calibration gather (run bench.py with --calib-copy)")
    f_vals = pmc_by_kernel(args.fetch_csv, "FETCH_SIZE")
    w_vals = pmc_by_kernel(args.write_csv, "WRITE_SIZE")
    ff, fw = calib_factors(f_vals, w_vals, calib)
    durs = {r["Name"]: float(r["AverageNs"]) for r in csv.DictReader(open(args.trace_csv))}
    out = ["# HBM bytes and bandwidth of every library kernel over the bench's arms",
           f"command_fetch: {args.cmd_fetch}", f"command_write: {args.cmd_write}",
           f"command_trace: {args.cmd_trace}", f"library: {lib_f}",
           f"calibration: pa_gather_kv of {calib} bytes; scale factors {ff:.4f} (fetch) {fw:.4f} (write)",
           "bytes are per dispatch (median over its dispatches); time is the mean kernel duration of the trace run",
           "", f"{'kernel':<70s} {'n':>4s} {'read_MB':>9s} {'write_MB':>9s} {'avg_us':>9s} "
               f"{'GB/s':>8s} {'of_8TB/s':>9s}"]
    for name in sorted(set(f_vals) & set(w_vals)):
        if not name.startswith(("pa::", "void pa::")) or "probe" in name:
            continue
        rb = statistics.median(f_vals[name]) * 1024 * ff
        wb = statistics.median(w_vals[name]) * 1024 * fw
        key = next((k for k in durs if k.replace("void ", "") == name.replace("void ", "")), None)
        t = durs.get(key, 0.0) * 1e-9 if key else 0.0
        gbs = (rb + wb) / t * 1e-9 if t else 0.0
        out.append(f"{short_name(name)[:70]:<70s} {len(f_vals[name]):>4d} {rb / 1e6:>9.1f} {wb / 1e6:>9.1f} "
                   f"{t * 1e6:>9.1f} {gbs:>8.0f} {gbs * 1e9 / PEAK_HBM_BYTES_S:>9.3f}")
    out.append("")
    out.append("Attention kernels (MFMA-bound) are listed for their traffic only; one kernel name can")
    out.append("cover several workloads (the headline, batched and fp8 arms share the bf16 kernel).")
    return "\n".join(out) + "\n"


def mfma_summary(args) -> str:
    rows = [r for r in csv.DictReader(open(args.csv)) if "attn_kernel" in r["Kernel_Name"]]
    disp = collections.defaultdict(dict)
    for r in rows:
        d = disp[int(r["Dispatch_Id"])]
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        d["dur"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        d["name"] = r["Kernel_Name"]
        d["grid"] = r.get("Grid_Size", r.get("Grid_Size_X", "?"))
    groups = collections.defaultdict(list)
    for d in disp.values():
        groups[(d["name"], d["grid"])].append(d)
    out = [f"# MFMA utilisation of the attention kernels over the bench's arms",
           f"command: {args.cmd}", f"library: {bench_library(args.bench_log)}",
           "busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); clock = (GRBM_GUI_ACTIVE / 8) / duration;",
           "ops = SQ_INSTS_VALU_MFMA_MOPS_{BF16,F16,I8} x 512 (hardware-counted, masked tile work included); medians over dispatches",
           "", f"{'kernel':<52s} {'grid':>8s} {'n':>3s} {'avg_us':>8s} {'busy':>6s} {'GHz':>6s} "
               f"{'bf16/f16 TF/s':>13s} {'i8 TOP/s':>9s} {'of_peak':>8s}"]
    for (name, grid), ds in sorted(groups.items(), key=lambda kv: kv[0]):
        med = lambda f: statistics.median([f(d) for d in ds])
        dur = med(lambda d: d["dur"])
        busy = med(lambda d: d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / N_SIMD / (d.get("GRBM_GUI_ACTIVE", 1) / N_XCD))
        clk = med(lambda d: d.get("GRBM_GUI_ACTIVE", 0) / N_XCD / d["dur"] * 1e-9)
        hf = med(lambda d: (d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0)) * 512 / d["dur"] * 1e-12)
        i8 = med(lambda d: d.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0) * 512 / d["dur"] * 1e-12)
        # time share of each kind at its own peak: the fraction of the blended peak
        frac = hf / PEAK_MFMA_TFLOPS["bf16/f16"] + i8 / PEAK_MFMA_TFLOPS["i8"]
        out.append(f"{short_name(name).replace('pa::attn_kernel', 'attn_kernel')[:52]:<52s} {grid:>8s} {len(ds):>3d} "
                   f"{dur * 1e6:>8.1f} {busy:>6.3f} {clk:>6.2f} {hf:>13.1f} {i8:>9.1f} {frac:>8.3f}")
    out += ["", "Template arguments: <head_dim, kind (0 bf16, 1 int8 exact-QK, 3 int8-QK), bf16 output, fast path>."]
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
    q = sub.add_parser("passes")
    for n in ("--fetch-csv", "--write-csv", "--trace-csv", "--bench-log-fetch", "--bench-log-write",
              "--cmd-fetch", "--cmd-write", "--cmd-trace", "--out"):
        q.add_argument(n, required=True)
    m = sub.add_parser("mfma")
    for n in ("--csv", "--bench-log", "--cmd", "--out"):
        m.add_argument(n, required=True)
    a = ap.parse_args()
    text = {"stats": stats_summary, "hbm": hbm_summary, "passes": passes_summary, "mfma": mfma_summary}[a.what](a)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
