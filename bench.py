#!/usr/bin/env python3
"""Throughput of the quantized linear projection on one MI355X.

A step is one pass of the whole hot path over one batch: the 18-layer
mixed-precision backbone sweep at M = 52224 tokens (64 observations x 816),
hidden 2048, MLP 16384, Hadamard block 128, bf16 outputs, distinct weights
per layer.  Per layer (8 launches):

  rotate+quantize the attention input to int4 -> q|k|v W4A4 GEMM (n = 6144)
  rotate+quantize the attention output to int8 -> o W8A8 GEMM
  rotate+quantize the MLP input to int4 -> gate|up W4A4 GEMM (n = 32768,
      gate/up rows interleaved in blocks of 32) with GeGLU in its epilogue
      -> h bf16 [M][16384]
  fold + Hadamard 128 + int8 quantization of h -> down W8A8 GEMM

Weights are quantized once before timing (offline).  Inputs are synthetic,
seeded, drawn on the device and resident in HBM before the timed region.
Before the W warm-up steps the step runs untimed for 0.5 s so that the GPU
clocks settle; the timed region (K steps) is bracketed by HIP events created
without a system-scope fence, on the launch stream.  value = integer GEMM
ops of the step (2*M*N*K summed over the 18 x 6 projections) / step time,
in TOPS.  roofline: the gate|up GEMM (the dominant kernel, 57% of the step's
ops) timed by event pairs around each of its launches inside the timed
region.

Side legs (one JSON object each): the same sweep with the W4A4 codes in FP6
E2M3 storage (the FP6 matrix-core GEMMs, bit-identical results), the sweep at
M = 6528 and 816, the
backbone MLP block at M = 816 (split-K down GEMM with its workspace), the W4A8
GEMM, the 7B-decoder projections at M = 256 W8A8 (HBM-bound), the action
expert over 10 denoising steps (W4A4, per-step static tables, W4A16; warm and
cold weights), the single W4A4 linear, the batch-1 W4A16 GEMV of a 7B-decoder
layer (cold weights), the composite rotation, a per-launch breakdown of one sweep layer, the shader
clock during the timed region, and the CPU oracle on a row sample.

Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
FP6_PEAK_TOPS = 10100.0   # MI355X dense fp6 / fp4 MFMA, 10.1 POP/s
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
# FETCH_SIZE / WRITE_SIZE summary of the sweep's kernels and the gate|up GEMM's name in it
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_sweep_m52224.txt")
# the gate|up GEMM with the GeGLU epilogue (bf16 h) at the sweep's M, in the traffic summary
GATE_UP_TAG = "gemm_i8_kernel<128,256,2,3,true,17,"


_T0 = time.perf_counter()


def log(msg: str) -> None:
    print(f"[{time.perf_counter() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--m", type=int, default=52224, help="tokens of the timed sweep (64 observations x 816)")
    ap.add_argument("--layers", type=int, default=18)
    ap.add_argument("--cpu-rows", type=int, default=64, help="token rows of the oracle's CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="the headline only")
    return ap.parse_args()


from bit_ptq_vla_amd.profile_step import read_traffic  # noqa: E402


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


def _stream():
    import torch

    return torch.cuda.current_stream().cuda_stream


class ClockSampler:
    """Samples the GPU's shader clock with amd-smi while the timed region
    runs (a thread; the readings are the driver's, not a measurement of ours)."""

    def __init__(self, period_s: float = 0.25):
        self.period = period_s
        self.samples = []
        self.raw = None
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--json"], capture_output=True, text=True,
                               timeout=5)
        except Exception as e:  # noqa: BLE001  (the tool may be missing: no reading)
            self.raw = f"amd-smi unavailable: {type(e).__name__}"
            return None
        if self.raw is None:
            self.raw = r.stdout[:600]
        try:
            data = json.loads(r.stdout)
        except Exception:  # noqa: BLE001
            return None
        found = []

        def walk(o, path):
            if isinstance(o, dict):
                for k, v in o.items():
                    walk(v, path + [str(k).lower()])
            elif isinstance(o, list):
                for v in o:
                    walk(v, path)
            else:
                p = "/".join(path)
                if "gfx" in p and "clk" in p and p.endswith("/value") and "min" not in p and "max" not in p:
                    try:
                        found.append(float(o))
                    except (TypeError, ValueError):
                        pass
        walk(data, [])
        return max(found) if found else None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        self._t.join(timeout=10)

    def summary(self):
        if not self.samples:
            return {"samples": 0, "note": self.raw}
        return {"samples": len(self.samples), "mhz_mean": round(statistics.mean(self.samples), 1),
                "mhz_min": min(self.samples), "mhz_max": max(self.samples), "source": "amd-smi metric --clock"}


def settle(fn, seconds=0.5):
    """Runs fn() back to back for `seconds` so that the clocks reach their loaded state."""
    import torch

    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        fn()
        torch.cuda.synchronize()


def _time_us(fn, reps):
    """Mean time of fn() over reps calls, between fence-free HIP events."""
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = HipEvent(_stream()), HipEvent(_stream())
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) * 1e3 / reps


def _median_us(fn, reps, trials=5):
    """Median over `trials` trials of the mean time of fn() over reps calls."""
    return statistics.median(_time_us(fn, reps) for _ in range(trials))


def _graph(fn):
    """A HIP graph that captured fn() (warmed up outside capture first)."""
    import torch

    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g


# ------------------------------------------------------------------ headline


def time_sweep(model, m, steps, warmup):
    """Step time of the whole sweep over `steps` steps and the mean duration
    of the gate|up GEMM launch inside them (event pairs on the launch stream)."""
    import torch

    settle(lambda: model.step(m))
    for _ in range(warmup):
        model.step(m)
    torch.cuda.synchronize()
    st = _stream()
    evs = [[(HipEvent(st), HipEvent(st)) for _ in range(model.layers)] for _ in range(steps)]
    marks = [HipEvent(st) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        wall0 = time.perf_counter()
        marks[0].record()
        for i in range(steps):
            model.step(m, evs[i])
            marks[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    ms_step = marks[0].elapsed_ms(marks[-1]) / steps
    per_step = [marks[i].elapsed_ms(marks[i + 1]) for i in range(steps)]
    gu = [a.elapsed_ms(b) for row in evs for a, b in row]
    return ms_step, statistics.mean(gu), per_step, wall, clk.summary()


def copy_model(read_bytes, write_bytes, reps=5):
    """The achievable time of a kernel that streams read_bytes in and
    write_bytes out once, from two measurements on fresh device buffers of
    the read size: a read-only stream (qlin_stream_read) gives the read
    time, a device-to-device copy (read and write of the same bytes) the
    added cost of writing.  Model: t = t_read(R) + (t_copy(R) - t_read(R)) * W / R."""
    import torch

    import bit_ptq_vla_amd as q

    dev = torch.device("cuda:0")
    src = torch.empty(read_bytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    t_read = _median_us(lambda: q.qlin_stream_read(src, sink=sink), reps)
    t_copy = _median_us(lambda: dst.copy_(src), reps)
    del src, dst
    torch.cuda.empty_cache()
    model = t_read + (t_copy - t_read) * write_bytes / read_bytes
    return {"read_GB/s": round(read_bytes / t_read / 1e3, 1), "copy_GB/s": round(2 * read_bytes / t_copy / 1e3, 1),
            "model_us": round(model, 2)}


def layer_breakdown(model, m, reps=3):
    """Mean duration of each of a layer's 8 launches at m tokens (events
    between consecutive launches, all layers, `reps` passes), with the
    algorithmic ops / bytes of each."""
    import torch

    st = _stream()
    names = ["quant_attn_in_int4", "gemm_qkv_w4a4", "quant_attn_out_int8", "gemm_o_w8a8", "quant_mlp_in_int4",
             "gemm_gate_up_w4a4_geglu", "quant_h_int8", "gemm_down_w8a8"]
    acc = [[] for _ in names]
    for _ in range(reps):
        for L in model.layer:
            evs = [HipEvent(st) for _ in range(9)]
            model.run_layer(L, m, evs=evs)
            torch.cuda.synchronize()
            for i in range(8):
                acc[i].append(evs[i].elapsed_ms(evs[i + 1]) * 1e3)
    hid, ffn = model.HID, model.FFN
    gemm = {"gemm_qkv_w4a4": (3 * hid, hid, 4, 4, 2 * 3 * hid), "gemm_o_w8a8": (hid, hid, 8, 8, 2 * hid),
            "gemm_gate_up_w4a4_geglu": (2 * ffn, hid, 4, 4, 2 * ffn // 2),
            "gemm_down_w8a8": (hid, ffn, 8, 8, 2 * hid)}
    quant = {"quant_attn_in_int4": (hid, 4), "quant_attn_out_int8": (hid, 8), "quant_mlp_in_int4": (hid, 4),
             "quant_h_int8": (ffn, 8)}
    out = {}
    for name, vals in zip(names, acc):
        us = statistics.median(vals)
        r = {"us": round(us, 2)}
        if name in gemm:
            n, k, ab, wb, ybytes = gemm[name]
            ops = 2 * m * n * k
            r["TOPS"] = round(ops / (us * 1e-6) / 1e12, 1)
            r["frac_int8_peak"] = round(ops / (us * 1e-6) / 1e12 / INT8_PEAK_TOPS, 4)
        else:
            k, bits = quant[name]
            nbytes = m * k * 2 + m * k * bits // 8 + 4 * m
            r["GB/s"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            r["frac_hbm"] = round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            # the achievable streaming time of the same read and write bytes on this GPU
            cm = copy_model(m * k * 2, m * k * bits // 8 + 4 * m)
            r["copy_model"] = cm
            r["frac_of_copy_model"] = round(cm["model_us"] / us, 4)
        out[name] = r
    return out


def sweep_e2m3_leg(model, m, steps=5, warmup=2):
    """The same sweep (same weights, folds, scales and int4-grid codes) with
    the W4A4 projections' codes in FP6 E2M3 storage: q|k|v and the fused
    gate|up GEMMs on the FP6 matrix cores (bit-identical results), o and down
    unchanged.  Step time over `steps` steps; the gate|up GEMM's mean launch
    time from event pairs, against both the FP6 and the int8 peak."""
    model.use_e2m3 = True
    try:
        ms_step, gu_ms, per_step, wall, clk = time_sweep(model, m, steps, warmup)
    finally:
        model.use_e2m3 = False
    tops = model.ops(m) / (ms_step * 1e-3) / 1e12
    gu_tops = 2 * m * 2 * model.FFN * model.HID / (gu_ms * 1e-3) / 1e12
    return {"ms_per_step": round(ms_step, 4), "TOPS": round(tops, 1),
            "frac_int8_peak_step": round(tops / INT8_PEAK_TOPS, 4), "steps": steps,
            "gate_up_e2m3_geglu": {"us_per_launch": round(gu_ms * 1e3, 2), "TOPS": round(gu_tops, 1),
                                   "frac_fp6_peak": round(gu_tops / FP6_PEAK_TOPS, 4),
                                   "frac_int8_peak": round(gu_tops / INT8_PEAK_TOPS, 4)},
            "sclk": clk}


def sweep_side(model, ms=(6528, 816), reps=3):
    """The sweep at smaller batches (same weights, first m tokens): median of
    5 trials of `reps` steps each."""
    out = {}
    for m in ms:
        settle(lambda: model.step(m), 0.3)
        us = _median_us(lambda: model.step(m), reps)
        tops = model.ops(m) / (us * 1e-6) / 1e12
        out[f"m{m}"] = {"ms_per_step": round(us / 1e3, 4), "TOPS": round(tops, 1),
                        "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}
    return out


def cpu_baseline_sweep(model, rows):
    """The oracle as it stands on `rows` token rows of layer 0 of the sweep:
    all six projections of the layer with their activation quantization
    (weights quantized beforehand, untimed); single thread (NumPy's int64
    matmul does not use BLAS; BLAS is pinned to one thread for the rotation)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from bit_ptq_vla_amd import synth

    hid, ffn = model.HID, model.FFN
    with threadpool_limits(limits=1):
        def w64(name, n, k):
            return synth.to_f64(model.weight(0, name, n, k).cpu())

        xa = synth.to_f64(model.x_attn[:rows].cpu())
        xo = synth.to_f64(model.x_o[:rows].cpu())
        xm = synth.to_f64(model.x_mlp[:rows].cpu())
        fold = {}
        L = model.layer[0]
        # the folds as calibrated (inputs of the oracle, computed on the full batch)
        for key in ("qkv", "o", "gu", "dn"):
            inv = L[f"inv_{key}"].cpu().numpy().astype(np.float64)
            fold[key] = (1.0 / inv).astype(np.float32)
        w_qkv = np.concatenate([w64(nm, hid, hid) for nm in ("q", "k", "v")])
        qw_qkv, sw_qkv, _ = oracle.quantize_weights(w_qkv, fold["qkv"], 128, 4)
        qw_o, sw_o, _ = oracle.quantize_weights(w64("o", hid, hid), fold["o"], 128, 8)
        w_gu = w64("gate_up", 2 * ffn, hid)
        qw_gu, sw_gu, _ = oracle.quantize_weights(oracle.interleave_gate_up(w_gu[:ffn], w_gu[ffn:]), fold["gu"], 128, 4)
        del w_gu
        qw_dn, sw_dn, _ = oracle.quantize_weights(w64("down", hid, ffn), fold["dn"], 128, 8)
        t0 = time.perf_counter()
        qx, sx, _ = oracle.rotate_quant_act(xa, fold["qkv"], 128, 4)
        oracle.gemm(qx, sx, qw_qkv, sw_qkv, "bf16")
        qx, sx, _ = oracle.rotate_quant_act(xo, fold["o"], 128, 8)
        oracle.gemm(qx, sx, qw_o, sw_o, "bf16")
        qx, sx, _ = oracle.rotate_quant_act(xm, fold["gu"], 128, 4)
        _, _, h = oracle.gemm_geglu(qx, sx, qw_gu, sw_gu, "bf16")
        qh, sh, _ = oracle.rotate_quant_act(h, fold["dn"], 128, 8)
        oracle.gemm(qh, sh, qw_dn, sw_dn, "bf16")
        dt = time.perf_counter() - t0
    ops = rows * model.ops_per_token_layer
    torch.cuda.synchronize()
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"{rows} token rows of layer 0 of the 18-layer sweep (all six projections with their "
                      f"activation quantization; weights quantized beforehand), {dt:.1f} s on 1 thread of "
                      f"{os.cpu_count()} host cores"}


# ------------------------------------------------------------------ side legs


def mlp_block_leg(dev, steps=20):
    """The backbone MLP block at M = 816: X -> int4 -> gate|up W4A4 GEMM with
    the GeGLU epilogue -> h -> int8 -> down W8A8 (split-K, caller workspace)."""
    import torch

    from bit_ptq_vla_amd.workload import MlpBlock

    block = MlpBlock(dev)
    torch.cuda.synchronize()
    settle(block.step)
    st = _stream()
    evs = [(HipEvent(st), HipEvent(st)) for _ in range(steps)]
    t0, t1 = HipEvent(st), HipEvent(st)
    for _ in range(5):
        block.step()
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        block.step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_ms(t1) / steps
    gu_us = statistics.mean(a.elapsed_ms(b) for a, b in evs) * 1e3
    tops = block.ops / (ms * 1e-3) / 1e12
    return block, {"workload": "backbone_mlp_m816_h2048_f16384", "ms_per_step": round(ms, 5),
                   "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                   "gate_up_us": round(gu_us, 2),
                   "gate_up_TOPS": round(block.gemm1_ops / (gu_us * 1e-6) / 1e12, 1)}


def w4a8_leg(block, reps=20):
    """The W4A8 GEMM (int8 activations x int4 weights) at the gate|up shape
    816 x 32768 x 2048: X rotated and quantized to int8 with the block's fold,
    the block's int4 gate|up weights; median of 5 trials."""
    import torch

    import bit_ptq_vla_amd as q

    m, k, n = block.m, block.gu.k, block.gu.n
    xq8, xs8 = q.qlin_rotate_quant_act(block.x, fold_inv_s=block.inv1, had_block=128, bits=8)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=block.x.device)
    us = _median_us(lambda: q.qlin_gemm_w4a8(xq8, xs8, block.wq1, block.ws1, k, out=y), reps)
    tops = 2 * m * n * k / (us * 1e-6) / 1e12
    return {"shape": f"{m}x{n}x{k}", "us_per_launch": round(us, 3), "TOPS": round(tops, 1),
            "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4)}


def e2m3_leg(dev, m=52224, reps=3):
    """The sweep's W4A4 GEMMs at M = 52224 with the codes in E2M3 storage (the
    int4 grid as FP6 values, on the FP6 matrix cores) beside the packed-int4
    path on the same inputs: q|k|v 52224 x 6144 x 2048 and gate|up 52224 x
    32768 x 2048 with the GeGLU epilogue; codes from the quantizers (b = 128)
    of synthetic rows.  Rates against the int8 peak and the fp6 peak."""
    import torch

    import bit_ptq_vla_amd as q
    from bit_ptq_vla_amd import synth

    k = 2048
    x = synth.device_normal(7, "e2m3/x", (m, k), dev, dtype="bf16", outliers=k // 100, outlier_scale=30.0)
    xq = {b: q.qlin_rotate_quant_act(x, had_block=128, bits=b) for b in (4, q.QLIN_BITS_E2M3)}
    del x
    res = {"m": m, "timing": "median of 5 trials"}
    for name, n, geglu in (("qkv", 6144, False), ("gate_up", 32768, True)):
        w = synth.device_normal(7, f"e2m3/w/{name}", (n, k), dev, std=0.02, dtype="f16")
        wq = {b: q.qlin_quantize_weights(w, had_block=128, bits=b) for b in (4, q.QLIN_BITS_E2M3)}
        del w
        y = torch.empty((m, n // 2 if geglu else n), dtype=torch.bfloat16, device=dev)
        r = {}
        for tag, b in (("int4", 4), ("e2m3", q.QLIN_BITS_E2M3)):
            (a, sx), (bq, sw) = xq[b], wq[b]
            scheme = q.QLIN_W4A4 if b == 4 else q.QLIN_W4A4_E2M3
            if geglu:
                fn = lambda: q.qlin_gemm_geglu(scheme, a, sx, bq, sw, k, out=y)
            elif b == 4:
                fn = lambda: q.qlin_gemm_w4a4(a, sx, bq, sw, k, out=y)
            else:
                fn = lambda: q.qlin_gemm_e2m3(a, sx, bq, sw, k, out=y)
            us = _median_us(fn, reps)
            tops = 2 * m * n * k / (us * 1e-6) / 1e12
            r[tag] = {"us": round(us, 1), "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                      "frac_fp6_peak": round(tops / FP6_PEAK_TOPS, 4)}
        res[f"{name}_{m}x{n}x{k}"] = r
        del wq, y
        torch.cuda.empty_cache()
    return res


def decoder_m256_leg(dev, reps=5):
    """The 7B-decoder projections at M = 256, W8A8 per-token / per-channel
    (no fold, no rotation): int8 quantization of X and the integer GEMM for
    q, k, v, o (4096 x 4096), gate, up (11008 x 4096) and down (4096 x 11008),
    fp16 out.  HBM-bound (I = 431..462 ops/byte < ridge 629): reported in
    GB/s of algorithmic bytes against 8 TB/s.  Weight copies (>= 512 MB in
    all) cycle so that the weights stream from HBM; graph replay."""
    import torch

    import bit_ptq_vla_amd as q
    from bit_ptq_vla_amd import synth

    wl = synth.CFG4
    m = 256
    layer = []
    for p in wl.projs:
        w = synth.weight(wl, p).to(dev)
        wq, ws = q.qlin_quantize_weights(w, bits=8)
        del w
        layer.append((p, wq, ws))
    wbytes = sum(p.n * p.k + 4 * p.n for p in layer_p(layer))
    copies = max(1, -(-512 * 2 ** 20 // wbytes) + 1)
    layers = [layer] + [[(p, wq.clone(), ws.clone()) for p, wq, ws in layer] for _ in range(copies - 1)]
    xs = {k: synth.activation(wl, wl.projs[0] if k == 4096 else wl.projs[-1], m).to(dev) for k in (4096, 11008)}
    xq = {k: (torch.empty((m, k), dtype=torch.int8, device=dev), torch.empty(m, dtype=torch.float32, device=dev))
          for k in (4096, 11008)}
    ys = {n: torch.empty((m, n), dtype=torch.float16, device=dev) for n in (4096, 11008)}
    work = {(p.n, p.k): q.gemm_workspace(q.QLIN_W8A8, m, p.n, p.k, dev) for p, _, _ in layer}

    def run(launches, with_quant):
        for p, wq, ws in launches:
            if with_quant:
                q.qlin_rotate_quant_act(xs[p.k], had_block=0, bits=8, out=xq[p.k])
            q.qlin_gemm_w8a8(xq[p.k][0], xq[p.k][1], wq, ws, p.k, out=ys[p.n], workspace=work[(p.n, p.k)])

    allp = [t for L in layers for t in L]
    for wq_quant in (True,):
        run(allp, wq_quant)
    torch.cuda.synchronize()
    res = {"m": m, "weight_copies": copies, "timing": "HIP graph replay, cold weights, median of 5"}
    g = _graph(lambda: run(allp, True))
    us_layer = _median_us(g.replay, reps) / len(layers)
    g2 = _graph(lambda: run(allp, False))
    us_gemm = _median_us(g2.replay, reps) / len(layers)
    ops = sum(2 * m * p.n * p.k for p, _, _ in layer)
    gemm_bytes = sum(m * p.k + p.n * p.k + 4 * (m + p.n) + 2 * m * p.n for p, _, _ in layer)
    res["layer_us_with_quant"] = round(us_layer, 2)
    res["layer_gemm_us"] = round(us_gemm, 2)
    res["gemm_GB/s"] = round(gemm_bytes / (us_gemm * 1e-6) / 1e9, 1)
    res["gemm_frac_hbm"] = round(gemm_bytes / (us_gemm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    res["gemm_TOPS"] = round(ops / (us_gemm * 1e-6) / 1e12, 1)
    shapes = {}
    for (n, k) in sorted({(p.n, p.k) for p, _, _ in layer}):
        launches = [(p, wq, ws) for L in layers for (p, wq, ws) in L if (p.n, p.k) == (n, k)]
        g3 = _graph(lambda: run(launches, False))
        us = _median_us(g3.replay, reps) / len(launches)
        nbytes = m * k + n * k + 4 * (m + n) + 2 * m * n
        shapes[f"{n}x{k}"] = {"us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                              "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    res["shapes"] = shapes
    return res


def layer_p(layer):
    return [p for p, _, _ in layer]


def gemv_leg(dev, reps=5):
    """Batch-1 W4A16 GEMV over a 7B-decoder layer; distinct weight copies
    (>= 512 MB in total) are cycled so that the weights stream from HBM.
    Launches are replayed from a captured HIP graph.  Beside each rate, the
    streaming-read ceiling: the plain 16-byte read reference
    (qlin_stream_read) over the same byte counts, launch for launch, cold."""
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

    def run(launches):
        for p, wq, ws in launches:
            q.qlin_gemv_w4a16(xs[p.k], wq, ws, out=ys[p.n])

    allp = [t for L in layers for t in L]
    g = _graph(lambda: run(allp))
    layer_us = _median_us(g.replay, reps) / len(layers)
    layer_gbs = (layer_bytes + sum(2 * p.k + 2 * p.n for p, _, _ in layer)) / (layer_us * 1e-6) / 1e9
    # the same layer with the projections that read one input merged along n
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
    gm = _graph(lambda: run([t for L in merged_layers for t in L]))
    merged_us = _median_us(gm.replay, reps) / len(merged_layers)
    merged_gbs = (layer_bytes + sum(2 * p.k + 2 * p.n for p, _, _ in merged_layers[0])) / (merged_us * 1e-6) / 1e9
    del merged_layers, gm
    shapes = {}
    for (n, k) in sorted({(p.n, p.k) for p, _, _ in layer}):
        launches = [(p, wq, ws) for L in layers for (p, wq, ws) in L if (p.n, p.k) == (n, k)]
        g3 = _graph(lambda: run(launches))
        us = _median_us(g3.replay, reps) / len(launches)
        nbytes = n * k // 2 + n * (k // 128) * 2 + 2 * k + 2 * n
        shapes[f"{n}x{k}"] = {"us": round(us, 3), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                              "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    # streaming-read ceiling: the same byte counts read once by the plain
    # 16-byte streaming-read reference, from cold slices of a 1 GiB buffer
    del layers
    torch.cuda.empty_cache()
    buf = torch.empty(2 ** 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(q.QLIN_STREAM_READ_SINK_WORDS, dtype=torch.int32, device=dev)

    def ceiling_gbs(sizes):
        sizes = [(b + 15) // 16 * 16 for b in sizes]
        offs, off = [], 0
        for _ in range(copies):
            for b in sizes:
                if off + b > buf.numel():
                    off = 0
                offs.append((off, b))
                off += (b + 255) // 256 * 256
        gr = _graph(lambda: [q.qlin_stream_read(buf[o:o + b], b, sink=sink) for o, b in offs])
        us = _median_us(gr.replay, reps) / copies
        return sum(sizes) / (us * 1e-6) / 1e9

    wbytes = {p.name: p.n * p.k // 2 + p.n * (p.k // 128) * 2 for p, _, _ in layer}
    layer_ceil = ceiling_gbs([wbytes[p.name] for p, _, _ in layer])
    merged_ceil = ceiling_gbs([sum(wbytes[nm] for nm in names) for names in
                               (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))])
    for key, v in shapes.items():
        n, k = (int(t) for t in key.split("x"))
        c = ceiling_gbs([n * k // 2 + n * (k // 128) * 2])
        v["read_ceiling_GB/s"] = round(c, 1)
        v["frac_of_read_ceiling"] = round(v["GB/s"] / c, 4)
    del buf
    return {"workload": "decoder7b_layer_m1_w4a16_g128", "layer_MB": round(layer_bytes / 1e6, 2),
            "weight_copies": copies, "layer_us": round(layer_us, 2), "GB/s": round(layer_gbs, 1),
            "frac_hbm": round(layer_gbs / HBM_PEAK_GBS, 4), "timing": "HIP graph replay, cold weights, median of 5",
            "read_ceiling_GB/s": round(layer_ceil, 1), "frac_of_read_ceiling": round(layer_gbs / layer_ceil, 4),
            "merged_qkv_gate_up": {"launches": 4, "layer_us": round(merged_us, 2), "GB/s": round(merged_gbs, 1),
                                   "frac_hbm": round(merged_gbs / HBM_PEAK_GBS, 4),
                                   "read_ceiling_GB/s": round(merged_ceil, 1),
                                   "frac_of_read_ceiling": round(merged_gbs / merged_ceil, 4)},
            "shapes": shapes}


def action_expert_leg(dev, reps=5):
    """The action expert's projections at M = 50 over 10 denoising steps:
    W4A4 (b = 64, with activation quantization), W4A4 with per-step static
    activation tables, W4A16 g128 on the same weights, and both schemes with
    q|k|v stacked; warm (the same weights every step: they stay in L2 /
    Infinity Cache) and cold (each step a distinct weight copy, >= 512 MB of
    copies in all).  Graph replay."""
    from bit_ptq_vla_amd.workload import ActionExpert

    ae = ActionExpert(dev)
    ae.build_static()
    ae.build_merged()
    res = {"m": 50, "steps": ae.steps, "timing": "HIP graph replay, median of 5"}
    for name, fn in (("w4a4", ae.run_w4a4), ("w4a4_static", ae.run_w4a4_static), ("w4a16", ae.run_w4a16),
                     ("w4a4_merged_qkv", ae.run_w4a4_merged), ("w4a16_merged_qkv", ae.run_w4a16_merged)):
        g = _graph(fn)
        us = _median_us(g.replay, reps) / ae.steps
        res[f"{name}_us_per_step"] = round(us, 2)
    copies = ae.build_cold_copies(512 * 2 ** 20)
    for name, fn in (("w4a4", ae.run_w4a4_cold), ("w4a16", ae.run_w4a16_cold)):
        graphs = [_graph(lambda c=c: fn(c)) for c in range(len(copies))]

        def replay_all():
            for g in graphs:
                g.replay()
        us = _median_us(replay_all, 2) / (len(graphs) * ae.steps)
        res[f"{name}_cold_us_per_step"] = round(us, 2)
    res["cold_weight_sets"] = len(copies) * ae.steps
    res["ops_per_step_gop"] = round(ae.ops_per_step / 1e9, 3)
    res["w4a16_bytes_per_step_mb"] = round(ae.w4a16_bytes / 1e6, 2)
    res["w4a16_cold_GB/s"] = round(ae.w4a16_bytes / (res["w4a16_cold_us_per_step"] * 1e-6) / 1e9, 1)
    return res


def single_linear_leg(dev, reps=5):
    """The single W4A4 linear 16 x 512 x 512 (fold, Hadamard 64): activation
    quantization and GEMM, 20 calls per captured graph; us per projection."""
    import torch

    import bit_ptq_vla_amd as q
    from bit_ptq_vla_amd import synth

    wl = synth.CFG1
    p = wl.projs[0]
    x = synth.activation(wl, p, 16).to(dev)
    w = synth.weight(wl, p).to(dev)
    s, inv = q.qlin_calibrate_fold(x, w)
    wq, ws = q.qlin_quantize_weights(w, fold_s=s, had_block=64, bits=4)
    xq = torch.empty((16, 256), dtype=torch.uint8, device=dev)
    xs = torch.empty(16, dtype=torch.float32, device=dev)
    y = torch.empty((16, 512), dtype=torch.float16, device=dev)

    def fn():
        for _ in range(20):
            q.qlin_rotate_quant_act(x, fold_inv_s=inv, had_block=64, bits=4, out=(xq, xs))
            q.qlin_gemm_w4a4(xq, xs, wq, ws, 512, out=y)

    g = _graph(fn)
    us = _median_us(g.replay, reps) / 20
    return {"workload": "single_w4a4_16x512x512", "us_per_projection": round(us, 2),
            "note": "two launches (quantize, GEMM); latency-bound (8.4 MOP)"}


def composite_leg(dev, reps=5):
    """Activation quantization with the SVD-Hadamard composite rotation and the
    zigzag permutation against the fast block Hadamard, at the action
    expert's input (50 x 1024, b = 64, fp16) and the backbone MLP's input
    (816 x 2048, b = 128, bf16); 20 calls per captured graph, us per call."""
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
            g = _graph(fn)
            r[tag] = round(_median_us(g.replay, reps) / 20, 2)
        res[name] = r
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported "
              f"(the projection path runs on a single GPU)", file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_ptq_vla_amd.workload import SweepModel

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = args.m
    log(f"bench: preparing the {args.layers}-layer sweep at M = {m} (weights quantized offline)")
    model = SweepModel(dev, m, args.layers, e2m3=not args.no_legs)
    log(f"bench: timing {args.steps} steps after {args.warmup} warm-up steps")
    ms_step, gu_ms, per_step, wall, clk = time_sweep(model, m, args.steps, args.warmup)
    tops = model.ops(m) / (ms_step * 1e-3) / 1e12
    gu_ops = 2 * m * 2 * model.FFN * model.HID
    gu_tops = gu_ops / (gu_ms * 1e-3) / 1e12
    gu_bytes = m * model.HID // 2 + 2 * model.FFN * model.HID // 2 + 4 * (m + 2 * model.FFN) + 2 * m * model.FFN
    out = {
        "metric": "W4A4/W8A8 qlinear TOPS + batch-1 W4A16 GEMV GB/s, % of MI355X roofline",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded normals drawn on the device, 1% outlier channels x30; random-init weights "
                "N(0, 0.02) per layer)",
        "config": {"workload": f"backbone_sweep_{args.layers}l_m{m}_h2048_f16384", "m": m, "layers": args.layers,
                   "hidden": model.HID, "ffn": model.FFN,
                   "schemes": {"q|k|v": "w4a4", "o": "w8a8", "gate|up": "w4a4 + GeGLU epilogue", "down": "w8a8"},
                   "hadamard_block": 128, "out_dtype": "bf16", "step_top": round(model.ops(m) / 1e12, 3)},
        "roofline": {"kernel": f"gate|up W4A4 GEMM {m}x{2 * model.FFN}x{model.HID} + GeGLU epilogue",
                     "bound": "mfma", "achieved": round(gu_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(gu_tops / INT8_PEAK_TOPS, 4),
                     "traffic": read_traffic(TRAFFIC_SUMMARY, GATE_UP_TAG),
                     "traffic_algorithmic": gu_bytes, "us_per_launch": round(gu_ms * 1e3, 2),
                     "launches_timed": args.steps * args.layers},
        "frac_of_int8_peak_step": round(tops / INT8_PEAK_TOPS, 4),
        "ms_per_step_median": round(statistics.median(per_step), 4),
        "sclk": clk,
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_legs:
        log("bench: the sweep with the W4A4 codes in E2M3 storage (FP6 matrix cores)")
        out["sweep_e2m3"] = sweep_e2m3_leg(model, m)
        log("bench: per-launch breakdown of a sweep layer")
        out["layer_breakdown_m%d" % m] = layer_breakdown(model, m)
        log("bench: sweep at M = 6528 and 816")
        out["sweep"] = sweep_side(model)
    if not args.no_cpu_baseline:
        log(f"bench: CPU oracle on {args.cpu_rows} rows")
        out["cpu_baseline"] = cpu_baseline_sweep(model, args.cpu_rows)
    del model
    torch.cuda.empty_cache()
    if not args.no_legs:
        def leg(key, fn):
            # a side leg that fails records its error instead of losing the line
            try:
                return fn()
            except Exception as e:  # noqa: BLE001
                log(f"bench: leg {key} failed: {type(e).__name__}: {e}")
                return {"error": f"{type(e).__name__}: {e}"}
            finally:
                torch.cuda.empty_cache()

        log("bench: backbone MLP block leg (M = 816)")
        block = None

        def mlp():
            nonlocal block
            block, r = mlp_block_leg(dev)
            return r
        out["mlp_block"] = leg("mlp_block", mlp)
        if block is not None:
            log("bench: W4A8 GEMM leg")
            out["w4a8"] = leg("w4a8", lambda: w4a8_leg(block))
            del block
        log("bench: E2M3 (FP6 matrix core) W4A4 GEMM leg")
        out["w4a4_e2m3"] = leg("w4a4_e2m3", lambda: e2m3_leg(dev))
        log("bench: 7B-decoder M = 256 W8A8 leg")
        out["decoder7b_m256_w8a8"] = leg("decoder7b_m256_w8a8", lambda: decoder_m256_leg(dev))
        log("bench: action expert leg (M = 50, 10 steps)")
        out["action_expert"] = leg("action_expert", lambda: action_expert_leg(dev))
        log("bench: single linear leg")
        out["single_linear"] = leg("single_linear", lambda: single_linear_leg(dev))
        log("bench: composite rotation leg")
        out["composite_rotation"] = leg("composite_rotation", lambda: composite_leg(dev))
        log("bench: batch-1 W4A16 GEMV leg")
        out["gemv"] = leg("gemv", lambda: gemv_leg(dev))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
