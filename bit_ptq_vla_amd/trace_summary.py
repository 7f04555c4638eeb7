"""Plain-text summary of a rocprofv3 ``--kernel-trace --stats`` CSV folder:
calls, mean / min / max duration and share of GPU time per kernel.

  python3 -m bit_ptq_vla_amd.trace_summary OUT_DIR
"""

from __future__ import annotations

import csv
import glob
import os
import sys


def summarize(folder: str) -> None:
    files = glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {folder}")
    rows = [r for f in files for r in csv.DictReader(open(f))]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print(f"{'calls':>6s} {'mean_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}  kernel")
    for r in rows:
        name = r["Name"].split("(qlin::")[0].split("(int,")[0]
        print(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
              f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}  {name[:120]}")


if __name__ == "__main__":
    summarize(sys.argv[1])
