"""Summaries of rocprofv3 output for this library's kernels.

    # per-kernel call counts and durations from a --kernel-trace --stats run
    # (--skip N also averages each kernel's calls after its first N, e.g.
    # the benchmark's warm-up calls)
    python -m block_sparse_video_fp32_amd.profiling stats DIR [--skip N]

    # HBM bytes per attend launch from two --pmc runs (FETCH_SIZE, then
    # WRITE_SIZE) of a command that also ran a plain device copy of
    # COPY_BYTES bytes: each counter is scaled by the ratio of the copy's true
    # bytes to what the same counter reported for the copy
    python -m block_sparse_video_fp32_amd.profiling traffic FETCH_DIR WRITE_DIR \\
        --kernel attend_kernel --copy-bytes 268435456 --out FILE.json

    # MFMA work and MFMA-pipe utilisation of one kernel from one --pmc run of
    # SQ_INSTS_VALU_MFMA_BF16 SQ_INSTS_VALU_MFMA_MOPS_BF16
    # SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32
    # SQ_INSTS_LDS SQ_BUSY_CYCLES GRBM_GUI_ACTIVE, set against the JSON line
    # bench.py printed in the same run (selected FLOPs, expected MFMA count)
    python -m block_sparse_video_fp32_amd.profiling mfma PMC_DIR BENCH.json \\
        --kernel "attend_kernel<128, 2, false, false>" --out FILE.json

    # any counters of one kernel from one --pmc run, per dispatch, and per
    # CU-cycle of one XCD's GRBM_GUI_ACTIVE when that counter is in the run
    python -m block_sparse_video_fp32_amd.profiling counters PMC_DIR \\
        --kernel "attend_kernel<128, 2, false, false>" --out FILE.json

    # the launches of one stretch of a trace in start order, e.g. the
    # Spark-Reblock partition of the last reblock call: from the last launch
    # whose name holds FIRST up to the next one whose name holds STOP
    python -m block_sparse_video_fp32_amd.profiling sequence DIR \
        --first gram_kernel --stop pool_q_kernel

The directories are rocprofv3 ``-d`` output directories written with
``--output-format csv``.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def _find(dirname: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(dirname, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirname}")
    return hits[0]


def kernel_stats(dirname: str, skip: int = 0):
    """Rows (name, calls, total_ns, avg_ns, min_ns, max_ns, avg_ns after the
    first `skip` calls or None) from a kernel trace, calls in start order."""
    path = _find(dirname, "kernel_trace.csv")
    per = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append((int(r["Start_Timestamp"]),
                                          int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows = []
    for name, calls in per.items():
        d = [x for _, x in sorted(calls)]
        rest = d[skip:]
        rows.append((name, len(d), sum(d), sum(d) / len(d), min(d), max(d),
                     sum(rest) / len(rest) if skip and rest else None))
    rows.sort(key=lambda r: -r[2])
    return rows


def launch_sequence(dirname: str, first: str, stop: str):
    """[(short name, grid, duration_ns)] of the launches from the last one
    whose name holds `first` up to (not including) the next one whose name
    holds `stop`, in start order; grid is the x, y, z grid size in threads."""
    path = _find(dirname, "kernel_trace.csv")
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if first in r["Kernel_Name"]]
    if not starts:
        raise RuntimeError(f"no launch of {first}")
    out = []
    for r in rows[starts[-1]:]:
        name = r["Kernel_Name"]
        if out and stop in name:
            break
        short = name.replace("void ", "").replace("sa::(anonymous namespace)::", "").split("(")[0]
        grid = tuple(int(r.get(f"Grid_Size_{a}", 1) or 1) for a in "XYZ")
        out.append((short, grid, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    return out


def counter_per_dispatch(dirname: str, counter: str, kernel_substr: str):
    """{dispatch_id: summed counter value} for dispatches whose name matches."""
    path = _find(dirname, "counter_collection.csv")
    out = collections.defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
                continue
            out[r["Dispatch_Id"]] += float(r["Counter_Value"])
            names[r["Dispatch_Id"]] = r["Kernel_Name"]
    return out, names


def kernel_source_hash(kernel: str = "attend_kernel") -> str:
    """Hash of the source file that holds `kernel` (the dense path's kernel
    has a file of its own; every other kernel of the path is in
    sparse_attn_kernels.hip) without comment lines, end of line comments and
    blank lines, so that edits of comments alone do not mark the recorded
    counters as stale."""
    name = "dense_attend_kernels.hip" if kernel.startswith("dense_attend") else "sparse_attn_kernels.hip"
    lines = []
    with open(os.path.join(HERE, "csrc", name), encoding="utf-8") as f:
        for line in f:
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int):
    res = {"kernel": kernel, "copy_bytes": copy_bytes, "kernel_source_sha256_16": kernel_source_hash(kernel)}
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals, _ = counter_per_dispatch(d, counter, kernel)
        copies, _ = counter_per_dispatch(d, counter, "copy")
        if not vals:
            raise RuntimeError(f"{counter}: no dispatch of {kernel}")
        if not copies:
            raise RuntimeError(f"{counter}: no copy kernel dispatch to calibrate against")
        kib = sum(vals.values()) / len(vals)
        copy_kib = max(copies.values())  # the large calibration copy
        factor = copy_bytes / (copy_kib * 1024.0)
        nbytes = kib * 1024.0 * factor
        res[counter] = {
            "kib_per_dispatch": kib,
            "dispatches": len(vals),
            "copy_kib": copy_kib,
            "scale": factor,
            "bytes_per_launch": nbytes,
        }
        total += nbytes
    res["bytes_per_launch"] = total
    return res


MFMA_COUNTERS = (
    "SQ_INSTS_VALU_MFMA_BF16",
    "SQ_INSTS_VALU_MFMA_MOPS_BF16",
    "SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_INSTS_VALU",
    "SQ_INSTS_VALU_TRANS_F32",
    "SQ_INSTS_LDS",
    "SQ_BUSY_CYCLES",
    "GRBM_GUI_ACTIVE",
)
N_XCD = 8       # MI355X: GRBM_GUI_ACTIVE is summed over its 8 XCDs
N_SIMD = 1024   # 256 CUs x 4 SIMDs; SQ_VALU_MFMA_BUSY_CYCLES is summed over them
PEAK_BF16_TFLOPS = 2500.0


def dispatch_durations(dirname: str, kernel_substr: str):
    """{dispatch_id: ns} from the timestamps of a counter collection."""
    path = _find(dirname, "counter_collection.csv")
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel_substr in r["Kernel_Name"]:
                out[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    return out


def mfma(pmc_dir: str, bench_line: dict, kernel: str):
    """Executed MFMA work and MFMA-pipe busy share of a kernel, per launch.

    The MOPS counter counts bf16 MFMA work in units of 512 FLOPs.  The busy
    share divides the summed per-SIMD MFMA busy cycles by the SIMD count times
    the active cycles of one XCD."""
    per = {}
    for c in MFMA_COUNTERS:
        vals, _ = counter_per_dispatch(pmc_dir, c, kernel)
        if not vals:
            raise RuntimeError(f"{c}: no dispatch of {kernel}")
        per[c] = sum(vals.values()) / len(vals)
        ndisp = len(vals)
    dur = dispatch_durations(pmc_dir, kernel)
    dur_ns = sum(dur.values()) / len(dur)
    gui_xcd = per["GRBM_GUI_ACTIVE"] / N_XCD
    flops_exec = per["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    sel = bench_line["selected_tflop_per_call"] * 1e12
    expected = bench_line.get("attend_mfma_per_launch")
    res = {
        "kernel": kernel,
        "kernel_source_sha256_16": kernel_source_hash(kernel),
        "dispatches": ndisp,
        "counters_per_dispatch": per,
        "duration_us": dur_ns / 1e3,
        "clock_ghz": gui_xcd / dur_ns,
        "mfma_instructions": per["SQ_INSTS_VALU_MFMA_BF16"],
        "mfma_instructions_expected": expected,
        "executed_mfma_tflop": flops_exec / 1e12,
        "selected_tflop": sel / 1e12,
        "flop_per_mfma": flops_exec / per["SQ_INSTS_VALU_MFMA_BF16"],
        "mfma_busy_frac": per["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * gui_xcd),
        "mfma_busy_cycles_per_mfma": per["SQ_VALU_MFMA_BUSY_CYCLES"] / per["SQ_INSTS_VALU_MFMA_BF16"],
        "executed_tflops": flops_exec / (dur_ns * 1e-9) / 1e12,
        "selected_tflops": sel / (dur_ns * 1e-9) / 1e12,
        "executed_frac_of_peak": flops_exec / (dur_ns * 1e-9) / 1e12 / PEAK_BF16_TFLOPS,
        "selected_frac_of_peak": sel / (dur_ns * 1e-9) / 1e12 / PEAK_BF16_TFLOPS,
        "trans_per_mfma": per["SQ_INSTS_VALU_TRANS_F32"] / per["SQ_INSTS_VALU_MFMA_BF16"],
        "valu_per_mfma": per["SQ_INSTS_VALU"] / per["SQ_INSTS_VALU_MFMA_BF16"],
        "lds_per_mfma": per["SQ_INSTS_LDS"] / per["SQ_INSTS_VALU_MFMA_BF16"],
    }
    if expected:
        res["mfma_instructions_ratio"] = per["SQ_INSTS_VALU_MFMA_BF16"] / expected
    return res


N_CU = 256  # MI355X compute units


def counters(pmc_dir: str, kernel: str):
    """Per-dispatch averages of every counter collected for a kernel.  SQ
    counters are also given per CU-cycle (summed value / (256 CUs x the
    active cycles of one XCD)); SQ_WAVE_CYCLES counts quad-cycles, so
    4 x its per-CU-cycle figure is the mean number of resident waves per CU."""
    path = _find(pmc_dir, "counter_collection.csv")
    names = set()
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                names.add(r["Counter_Name"])
    if not names:
        raise RuntimeError(f"no dispatch of {kernel}")
    per = {}
    for c in sorted(names):
        vals, _ = counter_per_dispatch(pmc_dir, c, kernel)
        per[c] = sum(vals.values()) / len(vals)
        ndisp = len(vals)
    dur = dispatch_durations(pmc_dir, kernel)
    res = {"kernel": kernel, "kernel_source_sha256_16": kernel_source_hash(kernel), "dispatches": ndisp,
           "counters_per_dispatch": per, "duration_us": sum(dur.values()) / len(dur) / 1e3}
    if "GRBM_GUI_ACTIVE" in per:
        gx = per["GRBM_GUI_ACTIVE"] / N_XCD
        res["clock_ghz"] = gx / (res["duration_us"] * 1e3)
        res["per_cu_cycle"] = {c: v / (N_CU * gx) for c, v in per.items() if c.startswith("SQ_")}
        if "SQ_WAVE_CYCLES" in per:
            res["resident_waves_per_cu"] = 4.0 * per["SQ_WAVE_CYCLES"] / (N_CU * gx)
    return res


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--skip", type=int, default=0, help="also average each kernel's calls after its first N")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--kernel", default="attend_kernel")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--out")
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("bench_json", help="file holding the JSON line bench.py printed in the counter run")
    m.add_argument("--kernel", default="attend_kernel<128, 2, false, false>")
    m.add_argument("--out")
    q = sub.add_parser("sequence")
    q.add_argument("dir")
    q.add_argument("--first", required=True)
    q.add_argument("--stop", required=True)
    c = sub.add_parser("counters")
    c.add_argument("pmc_dir")
    c.add_argument("--kernel", default="attend_kernel<128, 2, false, false>")
    c.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        extra = f" {'avg_us>' + str(args.skip):>10}" if args.skip else ""
        print(f"{'calls':>6} {'avg_us':>10}{extra} {'min_us':>10} {'max_us':>10} {'total_ms':>10}  kernel")
        for name, n, tot, avg, mn, mx, rest in kernel_stats(args.dir, args.skip):
            ex = (f" {rest / 1e3:10.2f}" if rest is not None else f" {'-':>10}") if args.skip else ""
            print(f"{n:6d} {avg / 1e3:10.2f}{ex} {mn / 1e3:10.2f} {mx / 1e3:10.2f} {tot / 1e6:10.3f}  {name[:110]}")
    elif args.cmd == "sequence":
        seq = launch_sequence(args.dir, args.first, args.stop)
        print(f"{'us':>9}  {'grid (threads)':>22}  kernel")
        for name, grid, ns in seq:
            print(f"{ns / 1e3:9.1f}  {str(grid):>22}  {name}")
        print(f"{sum(ns for _, _, ns in seq) / 1e3:9.1f}  {'total':>22}")
    else:
        if args.cmd == "counters":
            res = counters(args.pmc_dir, args.kernel)
        elif args.cmd == "mfma":
            with open(args.bench_json) as f:
                line = [x for x in f.read().splitlines() if x.startswith("{")][-1]
            res = mfma(args.pmc_dir, json.loads(line), args.kernel)
        else:
            res = traffic(args.fetch_dir, args.write_dir, args.kernel, args.copy_bytes)
        text = json.dumps(res, indent=2)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    sys.exit(main())
