#!/usr/bin/env python3
"""Throughput of the quantized linear projection on one MI355X.

A step is one pass of the whole hot path over one batch: the backbone-shaped
MLP block at M = 816 tokens (hidden 2048, gate|up 2 x 16384, down 2048):

  rotate+quantize X (bf16, fold, Hadamard 128, int4)
  -> gate|up W4A4 GEMM (816 x 32768 x 2048) with GeGLU in its epilogue
     (gate/up weight rows interleaved in blocks of 32) -> h bf16 [816][16384]
  -> fold + Hadamard 128 + int8 quantize of h
  -> down W8A8 GEMM (816 x 2048 x 16384) -> bf16

(--unfused: the gate|up GEMM writes both halves and the int8 quantizer
applies GeGLU on the way in.)

Weights are quantized once before timing (offline).  Inputs are synthetic,
seeded, resident in HBM before the timed region.  Before the W warm-up steps
the step runs untimed for 0.5 s so that the GPU clocks settle; the timed
region is bracketed by HIP events created without a system-scope fence.  value = integer GEMM ops of
the step (2*M*N*K summed) / step time, in TOPS.  Also reported: the
batch-1 W4A16 GEMV of a 7B-decoder layer (hidden 4096, MLP 11008) in GB/s
with distinct weight copies rotated to defeat the 256 MB Infinity Cache, the
W4A8 GEMM (int8 activations x int4 weights) at the gate|up shape, one layer
of the 18-layer backbone sweep at M = 6528 and 52224 (the compute-bound
regime), the action expert's projections over 10 denoising steps (W4A4 with
per-token scales, W4A4 with per-step static tables, W4A16), the dominant
kernel's roofline fraction, the activation stage with the SVD-Hadamard
composite rotation against the block Hadamard, and the CPU oracle on a row
sample.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
# FETCH_SIZE / WRITE_SIZE summary of the step's kernels and the gate|up GEMM's name in it
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_mlp_block_m816.txt")
GATE_UP_KERNEL = {True: "voidqlin::(anonymousnamespace)::gemm_i8_kernel<128,256,2,3,true,17,false>",
                  False: "voidqlin::(anonymousnamespace)::gemm_i8_kernel<128,256,2,3,true,1,false>"}
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=256, help="token rows of the oracle's CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--unfused", action="store_true", help="GeGLU in the int8 quantizer, not the GEMM epilogue")
    ap.add_argument("--no-sweep", action="store_true", help="skip the sweep-layer and action-expert legs")
    return ap.parse_args()


from bit_ptq_vla_amd.profile_step import read_traffic  # noqa: E402
from bit_ptq_vla_amd.workload import MlpBlock  # noqa: E402


class HipEvent:
    """A HIP event on the launch stream, created with hipEventDisableSystemFence:
    recording it adds no system-scope cache flush between the kernels it
    brackets (a default event's flush slows the next kernel measurably)."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, stream):
        import ctypes

        if HipEvent._hip is None:
            HipEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        self.stream = ctypes.c_void_p(stream)
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)):
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        if HipEvent._hip.hipEventRecord(self.ev, self.stream):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end) -> float:
        ms = self._ct.c_float()
        if HipEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if HipEvent._hip is not None and self.ev:
            HipEvent._hip.hipEventDestroy(self.ev)


def time_block(block, steps, warmup, settle_s=0.5):
    """Step time over `steps` steps (HIP events on the launch stream) and the
    mean duration of the gate|up GEMM launch inside them.  Before the warm-up
    steps the GPU runs the step for settle_s seconds so that its clocks reach
    their loaded state (the first milliseconds of a burst run slower)."""
    import torch

    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(20):
            block.step()
        torch.cuda.synchronize()
    for _ in range(warmup):
        block.step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    evs = [(HipEvent(stream), HipEvent(stream)) for _ in range(steps)]
    t0, t1 = HipEvent(stream), HipEvent(stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        block.step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_ms(t1) / steps
    gemm1_ms = sum(a.elapsed_ms(b) for a, b in evs) / steps
    return ms_step, gemm1_ms, wall


def gemv_leg(dev, reps=5):
    """Batch-1 W4A16 GEMV over a 7B-decoder layer; distinct weight copies
    (>= 512 MB in total) are cycled so that the weights stream from HBM.
    Launches are replayed from a captured HIP graph: the GPU runs them back
    to back (no host gaps inside the timed region)."""
    import torch

    import bit_ptq_vla_amd as q
    from bit_ptq_vla_amd import synth

    wl = synth.CFG4
    layer = []
    for p in wl.projs:
        w = synth.weight(wl, p).to(dev)
        wq, ws = q.qlin_quantize_weights(w, bits=4, group=128)
        del w
        layer.append((p, wq, ws))
    layer_bytes = sum(p.n * p.k // 2 + p.n * (p.k // 128) * 2 for p, _, _ in layer)
    copies = max(1, -(-512 * 2 ** 20 // layer_bytes) + 1)
    layers = [layer] + [[(p, wq.clone(), ws.clone()) for p, wq, ws in layer] for _ in range(copies - 1)]
    xs = {k: synth.normal_tensor(wl.seed, f"gemv_x/{k}", (1, k), dtype="f16").to(dev) for k in (4096, 11008)}
    ys = {n: torch.empty((1, n), dtype=torch.float16, device=dev) for n in (4096, 11008)}
    for L in layers:  # warm-up (and first-use initialisation) outside capture
        for p, wq, ws in L:
            q.qlin_gemv_w4a16(xs[p.k], wq, ws, out=ys[p.n])
    torch.cuda.synchronize()

    def replay_us(launches, n_rep):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for p, wq, ws in launches:
                q.qlin_gemv_w4a16(xs[p.k], wq, ws, out=ys[p.n])
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n_rep):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n_rep

    # whole layers, every copy in turn
    all_launches = [t for L in layers for t in L]
    layer_us = replay_us(all_launches, reps) / len(layers)
    layer_gbs = (layer_bytes + sum(2 * p.k + 2 * p.n for p, _, _ in layer)) / (layer_us * 1e-6) / 1e9
    # the same layer with the projections that read one input merged along n
    # (q|k|v and gate|up stacked, as inference engines store them): 4 launches
    merged_layers = []
    for L in layers:
        by = {p.name: (p, wq, ws) for p, wq, ws in L}
        merged = []
        for names in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
            ps = [by[nm] for nm in names]
            p0 = ps[0][0]
            pm = type(p0)("|".join(names), sum(t[0].n for t in ps), p0.k, p0.scheme)
            merged.append((pm, torch.cat([t[1] for t in ps]), torch.cat([t[2] for t in ps])))
        merged_layers.append(merged)
    for n in {p.n for p, _, _ in merged_layers[0]}:
        ys.setdefault(n, torch.empty((1, n), dtype=torch.float16, device=dev))
    merged_us = replay_us([t for L in merged_layers for t in L], reps) / len(merged_layers)
    merged_gbs = (layer_bytes + sum(2 * p.k + 2 * p.n for p, _, _ in merged_layers[0])) / (merged_us * 1e-6) / 1e9
    del merged_layers
    shapes = {}
    for (n, k) in sorted({(p.n, p.k) for p, _, _ in layer}):
        launches = [(p, wq, ws) for L in layers for (p, wq, ws) in L if (p.n, p.k) == (n, k)]
        us = replay_us(launches, reps) / len(launches)
        nbytes = n * k // 2 + n * (k // 128) * 2 + 2 * k + 2 * n
        shapes[f"{n}x{k}"] = {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
    return {"workload": "decoder7b_layer_m1_w4a16_g128", "layer_MB": round(layer_bytes / 1e6, 2),
            "weight_copies": copies, "layer_us": round(layer_us, 2), "GB/s": round(layer_gbs, 1),
            "frac_hbm": round(layer_gbs / HBM_PEAK_GBS, 4), "timing": "HIP graph replay, cold weights",
            "merged_qkv_gate_up": {"launches": 4, "layer_us": round(merged_us, 2), "GB/s": round(merged_gbs, 1),
                                   "frac_hbm": round(merged_gbs / HBM_PEAK_GBS, 4)},
            "shapes": shapes}


def w4a8_leg(block, steps):
    """The W4A8 GEMM (int8 activations x int4 weights) at the gate|up shape
    816 x 32768 x 2048: X rotated and quantized to int8 with the block's fold,
    the block's int4 gate|up weights; mean launch time over `steps` launches
    between fence-free HIP events."""
    import torch

    import bit_ptq_vla_amd as q

    m, k, n = block.m, block.gu.k, block.gu.n
    xq8, xs8 = q.qlin_rotate_quant_act(block.x, fold_inv_s=block.inv1, had_block=128, bits=8)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=block.x.device)
    for _ in range(5):
        q.qlin_gemm_w4a8(xq8, xs8, block.wq1, block.ws1, k, out=y)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = HipEvent(stream), HipEvent(stream)
    e0.record()
    for _ in range(steps):
        q.qlin_gemm_w4a8(xq8, xs8, block.wq1, block.ws1, k, out=y)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_ms(e1) * 1e3 / steps
    tops = 2 * m * n * k / (us * 1e-6) / 1e12
    return {"shape": f"{m}x{n}x{k}", "us_per_launch": round(us, 3), "TOPS": round(tops, 2),
            "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4), "bound": "mfma",
            "note": "back-to-back launches of the GEMM alone (bf16 out)"}


def _time_us(fn, reps):
    """Mean time of fn() over reps calls, between fence-free HIP events."""
    import torch

    fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = HipEvent(stream), HipEvent(stream)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) * 1e3 / reps


def sweep_leg(dev, ms=(6528, 52224), reps=3):
    """One layer of the mixed-precision backbone sweep at batched-observation
    sizes (the compute-bound regime): q/k/v W4A4, o W8A8, fused gate|up GeGLU
    W4A4, down W8A8, with every activation quantization; integer GEMM ops of
    the layer / layer time."""
    import torch

    from bit_ptq_vla_amd.workload import SweepLayer

    out = {}
    for m in ms:
        layer = SweepLayer(dev, m)
        us = _time_us(layer.step, reps)
        tops = layer.ops / (us * 1e-6) / 1e12
        out[f"m{m}"] = {"us_per_layer": round(us, 1), "TOPS": round(tops, 1),
                        "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4), "layer_gop": round(layer.ops / 1e9, 1)}
        del layer
        torch.cuda.empty_cache()
    return out


def _graph_us(fn, reps):
    """Mean replay time of a HIP graph that captured fn() (no host launch
    gaps), or None when fn cannot be captured."""
    import torch

    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        g.replay()
        torch.cuda.synchronize()
    except Exception as e:  # noqa: BLE001  (capture support, not a result)
        log(f"bench: graph capture unavailable ({type(e).__name__}); eager timing used")
        return None
    return _time_us(g.replay, reps)


def action_expert_leg(dev, reps=5):
    """The action expert's projections at M = 50 over 10 denoising steps, W4A4
    (b = 64, with activation quantization), W4A4 with per-step static
    activation tables (one table and one weight copy per step), and W4A16
    g128 on the same weights; then both schemes with q, k, v reading one
    input as one stacked 3072-column projection (shared fold); weights stay
    resident in L2 / Infinity Cache across steps (warm).  The 10 steps are replayed from a captured HIP graph:
    at these sizes eager Python launches (about 10 us each) would hide the
    kernels."""
    from bit_ptq_vla_amd.workload import ActionExpert

    ae = ActionExpert(dev)
    ae.build_static()
    ae.build_merged()
    res = {"m": 50, "steps": ae.steps}
    for name, fn in (("w4a4", ae.run_w4a4), ("w4a4_static", ae.run_w4a4_static), ("w4a16", ae.run_w4a16),
                     ("w4a4_merged_qkv", ae.run_w4a4_merged), ("w4a16_merged_qkv", ae.run_w4a16_merged)):
        us = _graph_us(fn, reps)
        mode = "graph replay"
        if us is None:
            us, mode = _time_us(fn, reps), "eager launches (host-bound)"
        us /= ae.steps
        res[f"{name}_us_per_step"] = round(us, 2)
        res[f"{name}_timing"] = mode
        if name.startswith("w4a4"):
            tops = ae.ops_per_step / (us * 1e-6) / 1e12
            res[f"{name}_TOPS"] = round(tops, 2)
            res[f"{name}_frac_int8_peak"] = round(tops / INT8_PEAK_TOPS, 4)
        elif name == "w4a16":
            gbs = ae.w4a16_bytes / (us * 1e-6) / 1e9
            res["w4a16_GB/s"] = round(gbs, 1)
            res["w4a16_frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
    res["note"] = "latency-bound (six projections of at most 4096 x 1024 per step); weights warm"
    return res


def composite_leg(dev, reps=5):
    """Activation quantization with the SVD-Hadamard composite rotation and the
    zigzag permutation against the fast block Hadamard, at the action
    expert's input (50 x 1024, b = 64, fp16) and the backbone MLP's input
    (816 x 2048, b = 128, bf16; rotations from the 2048 x 2048 q projection of
    the backbone sweep); 20 calls per captured graph, us per call."""
    import torch

    import bit_ptq_vla_amd as q
    from bit_ptq_vla_amd import synth

    res = {}
    for name, wl, proj, m, b in (("m50_k1024_b64", synth.CFG3, synth.CFG3.projs[0], 50, 64),
                                 ("m816_k2048_b128", synth.CFG5, synth.CFG5.projs[0], 816, 128)):
        w = synth.weight(wl, proj).to(dev)
        x = synth.activation(wl, proj, m).to(dev)
        perm, rot = q.qlin_calibrate_composite(w, b)
        xq = torch.empty((m, proj.k // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty(m, dtype=torch.float32, device=dev)
        work = torch.empty(m * proj.k, dtype=torch.float32, device=dev)

        def had():
            for _ in range(20):
                q.qlin_rotate_quant_act(x, had_block=b, bits=4, out=(xq, xs))

        def comp():
            for _ in range(20):
                q.qlin_rotate_quant_act_composite(x, perm, rot, bits=4, out=(xq, xs), work=work)

        r = {}
        for tag, fn in (("hadamard_us", had), ("composite_us", comp)):
            fn()
            torch.cuda.synchronize()
            us = _graph_us(fn, reps)
            r[tag] = round((us if us is not None else _time_us(fn, reps)) / 20, 2)
        res[name] = r
    return res


def cpu_baseline(block, rows):
    """The oracle as it stands on a row sample of the same step (single
    thread: NumPy's int64 matmul does not use BLAS; BLAS is pinned to one
    thread for the float64 rotation)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from bit_ptq_vla_amd import synth

    with threadpool_limits(limits=1):
        s1 = block.s1.cpu().numpy()
        s2 = block.s2.cpu().numpy()
        wgu = synth.to_f64(block.wgu_cpu)
        f = block.dn.k
        if block.fused:
            wgu = oracle.interleave_gate_up(wgu[:f], wgu[f:])
        qw1, sw1, _ = oracle.quantize_weights(wgu, s1, 128, 4)
        qw2, sw2, _ = oracle.quantize_weights(synth.to_f64(block.wdn_cpu), s2, 128, 8)
        x = synth.to_f64(block.x_cpu[:rows])
        t0 = time.perf_counter()
        qx, sx, _ = oracle.rotate_quant_act(x, s1, 128, 4)
        if block.fused:
            _, _, h = oracle.gemm_geglu(qx, sx, qw1, sw1, "bf16")
            qh, sh, _ = oracle.rotate_quant_act(h, s2, 128, 8)
        else:
            _, _, y1 = oracle.gemm(qx, sx, qw1, sw1, "bf16")
            qh, sh, _ = oracle.rotate_quant_act(y1, s2, 128, 8, preop="geglu")
        oracle.gemm(qh, sh, qw2, sw2, "bf16")
        dt = time.perf_counter() - t0
    ops = 2 * rows * (block.gu.n * block.gu.k + block.dn.n * block.dn.k)
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {block.m} token rows of the M=816 MLP block step "
                      f"(weights quantized beforehand), {dt:.1f} s on 1 thread of {os.cpu_count()} host cores"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              f"(the projection path runs on a single GPU)", file=sys.stderr)
        sys.exit(2)
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("bench: preparing the MLP block (weights quantized offline)")
    block = MlpBlock(dev, fused=not args.unfused)
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps after {args.warmup} warm-up steps")
    ms_step, gemm1_ms, wall = time_block(block, args.steps, args.warmup)
    tops = block.ops / (ms_step * 1e-3) / 1e12
    gemm1_tops = block.gemm1_ops / (gemm1_ms * 1e-3) / 1e12
    out = {
        "metric": "W4A4/W8A8 qlinear TOPS + batch-1 W4A16 GEMV GB/s, % of MI355X roofline",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded normals, 1% outlier channels x30; random-init weights N(0, 0.02))",
        "config": {"workload": "backbone_mlp_m816_h2048_f16384", "m": block.m, "hidden": 2048,
                   "ffn": 16384, "gate_up": "w4a4", "down": "w8a8", "hadamard_block": 128,
                   "geglu": "gate_up GEMM epilogue" if block.fused else "int8 quantizer pre-op",
                   "out_dtype": "bf16", "step_gop": round(block.ops / 1e9, 2)},
        "roofline": {"kernel": "gate_up W4A4 GEMM 816x32768x2048" + (" + GeGLU epilogue" if block.fused else ""),
                     "bound": "mfma",
                     "achieved": round(gemm1_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(gemm1_tops / INT8_PEAK_TOPS, 4),
                     "traffic": read_traffic(TRAFFIC_SUMMARY, GATE_UP_KERNEL[block.fused]),
                     "traffic_algorithmic": block.gemm1_bytes,
                     "us_per_launch": round(gemm1_ms * 1e3, 3)},
        "frac_of_int8_peak_step": round(tops / INT8_PEAK_TOPS, 4),
        "wall_s_timed": round(wall, 3),
    }
    log("bench: W4A8 GEMM leg")
    out["w4a8"] = w4a8_leg(block, args.steps)
    if not args.no_sweep:
        log("bench: backbone sweep layer leg (M = 6528, 52224)")
        out["sweep_layer"] = sweep_leg(dev)
        log("bench: action expert leg (M = 50, 10 steps)")
        out["action_expert"] = action_expert_leg(dev)
        out["composite_rotation"] = composite_leg(dev)
    if not args.no_gemv:
        log("bench: batch-1 W4A16 GEMV leg")
        out["gemv"] = gemv_leg(dev)
    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle on {args.cpu_rows} rows")
        out["cpu_baseline"] = cpu_baseline(block, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
