"""HBM traffic of the projection step's kernels from rocprofv3 counters.

Two parts:

  run        a short program to launch under ``rocprofv3 --pmc``: a plain
             device copy of known size (the calibration reference), then a few
             steps of the M = 816 backbone MLP block.
  summarize  reads the FETCH_SIZE and WRITE_SIZE collections of two such runs
             and prints a text summary: per kernel, the mean KiB per dispatch
             of each counter, scaled by the factor that maps the copy's
             counter reading onto its known byte count.

Usage (each counter in a run of its own):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- \\
      python3 -m bit_ptq_vla_amd.profile_step run
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- \\
      python3 -m bit_ptq_vla_amd.profile_step run
  python3 -m bit_ptq_vla_amd.profile_step summarize OUT/fetch OUT/write > summary.txt

The summary records the SHA-256 of the GEMM source it measured; a reader of
the figures (bench.py) treats them as stale once that source changes.
"""

from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
GEMM_SOURCE = os.path.join(HERE, "csrc", "gemm_i8.hip")
COPY_BYTES = 256 * 2 ** 20   # read once and written once by the calibration copy


def gemm_source_sha256() -> str:
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def run(steps: int) -> None:
    import torch

    from bit_ptq_vla_amd.workload import MlpBlock

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    block = MlpBlock(dev)
    torch.cuda.synchronize()
    for _ in range(steps):
        block.step()
    torch.cuda.synchronize()
    print(f"profile_step: copy x3 ({COPY_BYTES} bytes) and {steps} steps done", flush=True)


def _read_counter(folder: str, counter: str):
    """({kernel name: [values per dispatch]}, [calibration copy values]) of one
    counter (KiB per dispatch)."""
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    per = collections.defaultdict(float)
    names = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, r["Dispatch_Id"])
            per[key] += float(r["Counter_Value"])   # summed over dimensions (XCDs, channels)
            names[key] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    # the calibration copies: the first three copy dispatches of each run
    first = collections.defaultdict(list)
    for key in sorted(per, key=lambda kk: (kk[0], int(kk[1]))):
        if "copy" in names[key].lower() and len(first[key[0]]) < 3:
            first[key[0]].append(per[key])
    return out, [v for vs in first.values() for v in vs]


def _short(name: str) -> str:
    """Kernel name without its parameter list, spaces removed (one column)."""
    return name.split("(qlin::")[0].split("(int,")[0].replace(" ", "")[:110]


def summarize(fetch_dir: str, write_dir: str) -> None:
    fetch, copy_f = _read_counter(fetch_dir, "FETCH_SIZE")
    write, copy_w = _read_counter(write_dir, "WRITE_SIZE")
    if not copy_f or not copy_w:
        raise SystemExit("calibration copy kernel not found in the collections")
    kib = COPY_BYTES / 1024
    f_fac = kib / (sum(copy_f) / len(copy_f))
    w_fac = kib / (sum(copy_w) / len(copy_w))
    print("# HBM traffic per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch)")
    print(f"# copy calibration: {COPY_BYTES} bytes read and written; FETCH_SIZE reads "
          f"{sum(copy_f) / len(copy_f):.1f} KiB (factor {f_fac:.4f}), WRITE_SIZE reads "
          f"{sum(copy_w) / len(copy_w):.1f} KiB (factor {w_fac:.4f})")
    print(f"gemm_source_sha256: {gemm_source_sha256()}")
    print(f"{'kernel':110s} {'calls':>5s} {'fetch_KiB':>11s} {'write_KiB':>11s} {'bytes_scaled':>14s}")
    for name in sorted(set(fetch) | set(write)):
        fv, wv = fetch.get(name, []), write.get(name, [])
        if not fv or not wv:
            continue
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        scaled = (fk * f_fac + wk * w_fac) * 1024
        print(f"{_short(name):110s} {len(fv):5d} {fk:11.1f} {wk:11.1f} {scaled:14.0f}")


def read_traffic(summary_path: str, kernel_tag: str):
    """Scaled bytes per dispatch of the kernel whose summary line starts with
    kernel_tag (a name as _short prints it), or None when the summary is
    missing or its GEMM source hash differs from the current source."""
    if not os.path.exists(summary_path):
        return None
    sha = None
    for line in open(summary_path):
        if line.startswith("gemm_source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif sha is not None and line.startswith(kernel_tag):
            if sha != gemm_source_sha256():
                return None
            return int(float(line.split()[-1]))
    return None


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--steps", type=int, default=3)
    s = sub.add_parser("summarize")
    s.add_argument("fetch_dir")
    s.add_argument("write_dir")
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.steps)
    else:
        summarize(a.fetch_dir, a.write_dir)


if __name__ == "__main__":
    main(sys.argv[1:])
