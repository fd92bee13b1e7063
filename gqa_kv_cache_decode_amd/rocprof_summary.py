"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

Two summaries:

* ``stats``: the kernel-trace statistics of a run (calls, average / min / max
  duration per kernel), from ``<run>_kernel_stats.csv``.
* ``traffic``: HBM bytes per launch of the decode kernel from two counter
  runs (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, in KiB per dispatch).
  Each counter is scaled by what it reads for the largest copy kernel in the
  same run (a device-to-device copy of a known number of bytes, 1 GiB in
  ``bench.py --calibrate-copy``), and the result is stamped with a hash of
  the kernel sources so that a later source change invalidates it.

Usage:
  python -m gqa_kv_cache_decode_amd.rocprof_summary stats CSV OUT --command CMD [--trace TRACE_CSV]
  python -m gqa_kv_cache_decode_amd.rocprof_summary traffic FETCH_CSV WRITE_CSV OUT \\
      --kernel decode_matrix_kernel --copy-bytes 1073741824 --algorithmic-bytes N --command CMD
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))


# The sources the decode kernels are built from; a change to any of them may
# change the decode kernel's traffic. The projection and append-only sources
# and the host-side entry points do not.
DECODE_SOURCES = ("gqa_internal.hpp", "schedule.hpp", "decode_stream.hip", "decode_matrix.hip",
                  "decode_vector_kernel.hpp", "decode_vector.hip", "decode_vector_paged.hip",
                  "decode_vector_multi.hip", "decode_vector_multi_paged.hip", "merge_partials.hip")


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that a comment edit keeps the stamp."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def stats_summary(csv_path: str, command: str) -> str:
    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}",
             f"# kernel sources: {kernel_source_hash()}", "",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'share_%':>8}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.3f} {float(r['MinNs']) / 1e3:10.3f} "
                     f"{float(r['MaxNs']) / 1e3:10.3f} {float(r['Percentage']):8.2f}  {r['Name'][:140]}")
    return "\n".join(lines) + "\n"


def by_grid_summary(trace_csv: str) -> str:
    """Durations per (kernel, grid size) from ``<run>_kernel_trace.csv``: separates the
    launches of one kernel with different shapes (the layer's two projections)."""
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        key = (r["Kernel_Name"][:110], int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["", "# per launch shape (kernel trace)",
             f"{'calls':>6} {'avg_us':>9} {'p10_us':>9} {'p50_us':>9} {'p90_us':>9} {'min_us':>9} {'max_us':>9} "
             f"{'wgs':>7}  kernel"]
    for (name, wgs), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        q = statistics.quantiles(d, n=10) if len(d) > 1 else [d[0]] * 9
        lines.append(f"{len(d):6d} {statistics.mean(d):9.3f} {q[0]:9.3f} {q[4]:9.3f} {q[8]:9.3f} {min(d):9.3f} "
                     f"{max(d):9.3f} {wgs:7d}  {name}")
    return "\n".join(lines) + "\n"


def _per_kernel(csv_path: str):
    out = {}
    for r in csv.DictReader(open(csv_path)):
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def traffic_summary(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int, algorithmic: float,
                    command: str, workload: str) -> str:
    f, w = _per_kernel(fetch_csv), _per_kernel(write_csv)

    def pick(d, key):
        names = [n for n in d if key in n]
        if not names:
            raise SystemExit(f"no kernel matching {key!r} in counter output")
        return [v for n in names for v in d[n]]

    cf = max(pick(f, "copyBuffer"))  # the 1 GiB copy is the largest copy dispatch
    cw = max(pick(w, "copyBuffer"))
    kf_fetch = copy_bytes / (cf * 1024.0)
    kf_write = copy_bytes / (cw * 1024.0)
    fetch_kib = statistics.mean(pick(f, kernel))
    write_kib = statistics.mean(pick(w, kernel))
    hbm = fetch_kib * 1024 * kf_fetch + write_kib * 1024 * kf_write
    lines = [
        "# HBM traffic per decode launch from rocprofv3 counters",
        f"# fetch run: {command.replace('PMC', 'FETCH_SIZE')}",
        f"# write run: {command.replace('PMC', 'WRITE_SIZE')}",
        "# Each counter is scaled by what it reads for a device copy of copy_bytes.",
        f"workload = {workload}",
        f"kernel = {kernel}",
        f"kernel_source_hash = {kernel_source_hash()}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {cf:.1f}",
        f"copy_write_kib = {cw:.1f}",
        f"fetch_scale = {kf_fetch:.4f}",
        f"write_scale = {kf_write:.4f}",
        f"kernel_fetch_kib_per_dispatch = {fetch_kib:.1f}",
        f"kernel_write_kib_per_dispatch = {write_kib:.1f}",
        f"hbm_read_bytes_per_launch = {fetch_kib * 1024 * kf_fetch:.0f}",
        f"hbm_write_bytes_per_launch = {write_kib * 1024 * kf_write:.0f}",
        f"hbm_bytes_per_launch = {hbm:.0f}",
        f"algorithmic_bytes_per_launch = {algorithmic:.0f}",
        f"traffic_over_algorithmic = {hbm / algorithmic:.4f}",
    ]
    return "\n".join(lines) + "\n"


def read_traffic(path: str):
    try:
        text = open(path).read()
    except OSError:
        return None
    rec = {}
    for line in text.splitlines():
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    return rec


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--command", required=True)
    a.add_argument("--trace", default=None, help="kernel_trace.csv: add a breakdown per launch shape")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--kernel", default="decode_matrix_kernel")
    b.add_argument("--copy-bytes", type=int, default=1 << 30)
    b.add_argument("--algorithmic-bytes", type=float, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--command", required=True)
    args = ap.parse_args()
    if args.cmd == "stats":
        text = stats_summary(args.csv, args.command)
        if args.trace:
            text += by_grid_summary(args.trace)
    else:
        text = traffic_summary(args.fetch_csv, args.write_csv, args.kernel, args.copy_bytes,
                               args.algorithmic_bytes, args.command, args.workload)
    with open(args.out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main()
