"""Summaries of rocprofv3 output for this library's kernels.

    # per-kernel call counts and durations from a --kernel-trace --stats run
    python -m block_sparse_video_fp32_amd.profiling stats DIR

    # HBM bytes per attend launch from two --pmc runs (FETCH_SIZE, then
    # WRITE_SIZE) of a command that also ran a plain device copy of
    # COPY_BYTES bytes: each counter is scaled by the ratio of the copy's true
    # bytes to what the same counter reported for the copy
    python -m block_sparse_video_fp32_amd.profiling traffic FETCH_DIR WRITE_DIR \\
        --kernel attend_kernel --copy-bytes 268435456 --out FILE.json

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


def kernel_stats(dirname: str):
    """Rows (name, calls, total_ns, avg_ns, min_ns, max_ns) from a kernel trace."""
    path = _find(dirname, "kernel_trace.csv")
    per = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            per[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    rows = []
    for name, d in per.items():
        rows.append((name, len(d), sum(d), sum(d) / len(d), min(d), max(d)))
    rows.sort(key=lambda r: -r[2])
    return rows


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


def kernel_source_hash() -> str:
    """Hash of the attend kernel's source file without comment lines, end of
    line comments and blank lines, so that edits of comments alone do not
    mark the recorded counters as stale."""
    lines = []
    with open(os.path.join(HERE, "csrc", "sparse_attn_kernels.hip"), encoding="utf-8") as f:
        for line in f:
            code = line.split("//", 1)[0].rstrip()
            if code.strip():
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def traffic(fetch_dir: str, write_dir: str, kernel: str, copy_bytes: int):
    res = {"kernel": kernel, "copy_bytes": copy_bytes, "kernel_source_sha256_16": kernel_source_hash()}
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


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_dir")
    b.add_argument("write_dir")
    b.add_argument("--kernel", default="attend_kernel")
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10}  kernel")
        for name, n, tot, avg, mn, mx in kernel_stats(args.dir):
            print(f"{n:6d} {avg / 1e3:10.2f} {mn / 1e3:10.2f} {mx / 1e3:10.2f} {tot / 1e6:10.3f}  {name[:110]}")
    else:
        res = traffic(args.fetch_dir, args.write_dir, args.kernel, args.copy_bytes)
        text = json.dumps(res, indent=2)
        if args.out:
            with open(args.out, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    sys.exit(main())
