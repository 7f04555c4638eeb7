"""Counter profiles of the projection path's kernels (rocprofv3 --pmc).

Two parts:

  run        a short program to launch under ``rocprofv3 --pmc``: a plain
             device copy of known size (the calibration reference for the
             traffic counters), then a few repetitions of one workload:
               mlp     the M = 816 backbone MLP block step
               sweep   one layer of the 18-layer backbone sweep at --m tokens
               gemm    integer GEMMs at the sweep shapes (--m tokens); the
                       *_e2m3 ones take codes from the E2M3 quantizers
               gemv    the batch-1 W4A16 GEMVs of a 7B-decoder layer, weight
                       copies cycled so that the weights stream from HBM
  summarize  reads the FETCH_SIZE and WRITE_SIZE collections of two such runs
             and prints a text summary: per kernel, the mean KiB per dispatch
             of each counter, scaled by the factor that maps the copy's
             counter reading onto its known byte count.
  counters   reads any number of counter collections (one rocprofv3 pass
             each) and prints, per kernel, the mean of every counter per
             dispatch and the derived rates: the MFMA unit's busy fraction,
             VALU and LDS instructions per MFMA, LDS bank conflicts per LDS
             instruction, and the share of wave cycles spent waiting.

Usage (each counter set in a run of its own, from the repository root):

  rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o run -- \\
      python3 -m bit_ptq_vla_amd.profile_step run --workload sweep --m 52224
  rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o run -- \\
      python3 -m bit_ptq_vla_amd.profile_step run --workload sweep --m 52224
  python3 -m bit_ptq_vla_amd.profile_step summarize OUT/fetch OUT/write > summary.txt

  rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE ... \\
      --output-format csv -d OUT/pmc1 -o run -- python3 -m bit_ptq_vla_amd.profile_step run ...
  python3 -m bit_ptq_vla_amd.profile_step counters OUT/pmc1 OUT/pmc2 ... > counters.txt

A summary records the SHA-256 of the GEMM source it measured; a reader of the
figures (bench.py) treats them as stale once that source changes.
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

# MI355X: 256 CUs x 4 SIMDs; GRBM_GUI_ACTIVE counts GPU-busy cycles once per XCD
SIMDS = 256 * 4
XCDS = 8


def gemm_source_sha256() -> str:
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _copy_reference(dev):
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


SWEEP_GEMMS = {  # name: (n, k, scheme) of the sweep's projections
    "qkv": (6144, 2048, "w4a4"), "o": (2048, 2048, "w8a8"), "gate_up": (32768, 2048, "geglu"),
    "down": (2048, 16384, "w8a8"), "gate_up_w4a8": (32768, 2048, "w4a8"),
    "qkv_e2m3": (6144, 2048, "e2m3"), "gate_up_e2m3": (32768, 2048, "geglu_e2m3"),
}


def run(workload: str, steps: int, m: int, gemms) -> None:
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    _copy_reference(dev)
    if workload == "mlp":
        from bit_ptq_vla_amd.workload import MlpBlock

        block = MlpBlock(dev)
        for _ in range(steps):
            block.step()
    elif workload == "sweep":
        from bit_ptq_vla_amd.workload import SweepModel

        model = SweepModel(dev, m, layers=1)
        for _ in range(steps):
            model.step(m)
    elif workload == "gemm":
        import bit_ptq_vla_amd as q
        from bit_ptq_vla_amd import synth

        for name in gemms:
            n, k, sch = SWEEP_GEMMS[name]
            if sch in ("e2m3", "geglu_e2m3"):
                # E2M3 codes from the library's quantizers on synthetic rows
                x = synth.device_normal(0, f"prof/x/{name}", (m, k), dev, dtype="bf16")
                w = synth.device_normal(0, f"prof/w/{name}", (n, k), dev, std=0.02, dtype="f16")
                xq, xs = q.qlin_rotate_quant_act(x, had_block=128, bits=q.QLIN_BITS_E2M3)
                wq, ws = q.qlin_quantize_weights(w, had_block=128, bits=q.QLIN_BITS_E2M3)
                del x, w
                for _ in range(steps):
                    if sch == "geglu_e2m3":
                        q.qlin_gemm_geglu(q.QLIN_W4A4_E2M3, xq, xs, wq, ws, k)
                    else:
                        q.qlin_gemm_e2m3(xq, xs, wq, ws, k)
                torch.cuda.synchronize()
                del xq, wq
                torch.cuda.empty_cache()
                continue
            abits = 8 if sch in ("w8a8", "w4a8") else 4
            wbits = 8 if sch == "w8a8" else 4
            a = synth.device_normal(0, f"prof/a/{name}", (m, k), dev).clamp(-7, 7).round().to(torch.int8)
            b = synth.device_normal(0, f"prof/b/{name}", (n, k), dev).clamp(-7, 7).round().to(torch.int8)
            if abits == 4:   # two codes per byte, even k in the low nibble
                a = ((a[:, 0::2] & 0xF) | (a[:, 1::2] << 4)).view(torch.uint8).contiguous()
            if wbits == 4:
                b = ((b[:, 0::2] & 0xF) | (b[:, 1::2] << 4)).view(torch.uint8).contiguous()
            sx = torch.full((m,), 1e-3, device=dev)
            sw = torch.full((n,), 1e-3, device=dev)
            for _ in range(steps):
                if sch == "geglu":
                    q.qlin_gemm_w4a4_geglu(a, sx, b, sw, k)
                else:
                    f = {"w4a4": q.qlin_gemm_w4a4, "w8a8": q.qlin_gemm_w8a8, "w4a8": q.qlin_gemm_w4a8}[sch]
                    ws = q.gemm_workspace({"w4a4": 0, "w8a8": 1, "w4a8": 2}[sch], m, n, k, dev)
                    f(a, sx, b, sw, k, workspace=ws)
            torch.cuda.synchronize()
            del a, b
            torch.cuda.empty_cache()
    elif workload == "gemv":
        import bit_ptq_vla_amd as q
        from bit_ptq_vla_amd import synth

        wl = synth.CFG4
        layer = []
        for p in wl.projs:
            w = synth.weight(wl, p).to(dev)
            layer.append((p,) + q.qlin_quantize_weights(w, bits=4, group=128))
            del w
        layer_bytes = sum(p.n * p.k // 2 for p, _, _ in layer)
        copies = max(1, -(-512 * 2 ** 20 // layer_bytes) + 1)
        layers = [layer] + [[(p, a.clone(), b.clone()) for p, a, b in layer] for _ in range(copies - 1)]
        xs = {k: synth.normal_tensor(wl.seed, f"gemv_x/{k}", (1, k), dtype="f16").to(dev) for k in (4096, 11008)}
        for _ in range(steps):
            for L in layers:
                for p, wq, ws in L:
                    q.qlin_gemv_w4a16(xs[p.k], wq, ws)
    else:
        raise SystemExit(f"unknown workload {workload}")
    torch.cuda.synchronize()
    print(f"profile_step: copy x3 ({COPY_BYTES} bytes) and {steps} repetitions of {workload} done", flush=True)


def _collections(folder: str):
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    return files


def _read_all(folder: str):
    """{counter: {(file, dispatch): value}} and {(file, dispatch): kernel name},
    values summed over the counter's dimensions (XCDs, channels, SEs)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for f in _collections(folder):
        for r in csv.DictReader(open(f)):
            key = (f, int(r["Dispatch_Id"]))
            vals[r["Counter_Name"]][key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    return vals, names


def _read_counter(folder: str, counter: str):
    """({kernel name: [values per dispatch]}, [calibration copy values]) of one
    counter (KiB per dispatch)."""
    vals, names = _read_all(folder)
    per = vals.get(counter, {})
    out = collections.defaultdict(list)
    for key, v in per.items():
        out[names[key]].append(v)
    # the calibration copies: the first three copy dispatches of each run
    first = collections.defaultdict(list)
    for key in sorted(per, key=lambda kk: (kk[0], kk[1])):
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


def counters(dirs) -> None:
    """Per kernel: mean per dispatch of every counter found, and derived rates."""
    table = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        vals, names = _read_all(d)
        for counter, per in vals.items():
            for key, v in per.items():
                table[names[key]][counter].append(v)
    print("# rocprofv3 --pmc counters, mean per dispatch (summed over the counter's dimensions)")
    print(f"gemm_source_sha256: {gemm_source_sha256()}")
    for name in sorted(table):
        if "copy" in name.lower() or "Fill" in name:
            continue
        c = {k: sum(v) / len(v) for k, v in table[name].items()}
        calls = max(len(v) for v in table[name].values())
        print(f"\n{_short(name)}  (dispatches per counter: {calls})")
        for k in sorted(c):
            print(f"  {k:32s} {c[k]:18.1f}")
        mf = c.get("SQ_INSTS_MFMA")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c and c["GRBM_GUI_ACTIVE"] > 0:
            busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / XCDS * SIMDS)
            print(f"  -> MFMA busy fraction of kernel cycles (all SIMDs): {busy:.3f}")
        if mf:
            for k, label in (("SQ_INSTS_VALU", "VALU per MFMA"), ("SQ_INSTS_LDS", "LDS instructions per MFMA"),
                             ("SQ_INSTS_VMEM_RD", "vector-memory reads per MFMA"), ("SQ_INSTS_SALU", "SALU per MFMA")):
                if k in c:
                    # SQ_INSTS_VALU counts MFMAs as VALU instructions too
                    v = c[k] - mf if k == "SQ_INSTS_VALU" else c[k]
                    print(f"  -> {label}: {v / mf:.2f}")
        if "SQ_LDS_BANK_CONFLICT" in c and "SQ_LDS_IDX_ACTIVE" in c and c["SQ_LDS_IDX_ACTIVE"] > 0:
            print(f"  -> LDS bank-conflict cycles / LDS active cycles: "
                  f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_LDS_IDX_ACTIVE']:.3f}")
        if "SQ_WAIT_ANY" in c and "SQ_WAVE_CYCLES" in c and c["SQ_WAVE_CYCLES"] > 0:
            print(f"  -> wave cycles waiting (any): {c['SQ_WAIT_ANY'] / c['SQ_WAVE_CYCLES']:.3f}")
        if "SQ_WAIT_INST_LDS" in c and "SQ_WAVE_CYCLES" in c and c["SQ_WAVE_CYCLES"] > 0:
            print(f"  -> wave cycles waiting on LDS instructions: {c['SQ_WAIT_INST_LDS'] / c['SQ_WAVE_CYCLES']:.3f}")


def read_traffic(summary_path: str, kernel_tag: str):
    """Scaled bytes per dispatch of the first kernel whose summary line
    contains kernel_tag, or None when the summary is missing or its GEMM
    source hash differs from the current source."""
    if not os.path.exists(summary_path):
        return None
    sha = None
    for line in open(summary_path):
        if line.startswith("gemm_source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        elif sha is not None and kernel_tag in line.split(" ")[0]:
            if sha != gemm_source_sha256():
                return None
            return int(float(line.split()[-1]))
    return None


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", choices=["mlp", "sweep", "gemm", "gemv"], default="mlp")
    r.add_argument("--steps", type=int, default=3)
    r.add_argument("--m", type=int, default=52224)
    r.add_argument("--gemms", default="qkv,o,gate_up,down", help="comma list of " + ",".join(SWEEP_GEMMS))
    s = sub.add_parser("summarize")
    s.add_argument("fetch_dir")
    s.add_argument("write_dir")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run(a.workload, a.steps, a.m, [g for g in a.gemms.split(",") if g])
    elif a.cmd == "summarize":
        summarize(a.fetch_dir, a.write_dir)
    else:
        counters(a.dirs)


if __name__ == "__main__":
    main(sys.argv[1:])
