"""Device-resident workloads of the projection path, shared by bench.py and
the profiling program.  Nothing here computes the method itself: every step
runs through the library's entry points.
"""

from __future__ import annotations


class MlpBlock:
    """Device buffers and quantized weights of the M = 816 backbone MLP block.

    fused=True (the benchmarked chain): the gate and up weight rows are
    interleaved in blocks of 32 before quantization and the gate|up GEMM
    applies GeGLU in its epilogue, writing h [M][16384] once; h is then folded,
    rotated and quantized to int8 for the down projection.
    fused=False: the gate|up GEMM writes [M][32768] and the activation
    quantizer applies GeGLU on the way in (pre-op).
    """

    def __init__(self, dev, fused: bool = True):
        import torch

        import bit_ptq_vla_amd as q
        from bit_ptq_vla_amd import synth

        self.q = q
        self.fused = fused
        wl = synth.CFG2
        self.gu, self.dn = wl.projs
        self.m = wl.ms[0]
        f = self.dn.k
        self.x_cpu = synth.activation(wl, self.gu, self.m)
        self.wgu_cpu = synth.weight(wl, self.gu)          # gate rows, then up rows
        self.wdn_cpu = synth.weight(wl, self.dn)
        self.x = self.x_cpu.to(dev)
        wgu, wdn = self.wgu_cpu.to(dev), self.wdn_cpu.to(dev)
        if fused:
            wgu = q.interleave_gate_up(wgu[:f], wgu[f:])
        # offline: fold calibration and weight quantization
        self.s1, self.inv1 = q.qlin_calibrate_fold(self.x, wgu)
        self.wq1, self.ws1 = q.qlin_quantize_weights(wgu, fold_s=self.s1, had_block=128, bits=4)
        self.xq = torch.empty((self.m, self.gu.k // 2), dtype=torch.uint8, device=dev)
        self.xs = torch.empty(self.m, dtype=torch.float32, device=dev)
        q.qlin_rotate_quant_act(self.x, fold_inv_s=self.inv1, had_block=128, bits=4, out=(self.xq, self.xs))
        if fused:
            self.y1 = torch.empty((self.m, f), dtype=torch.bfloat16, device=dev)
            q.qlin_gemm_w4a4_geglu(self.xq, self.xs, self.wq1, self.ws1, self.gu.k, out=self.y1)
            self.s2, self.inv2 = q.qlin_calibrate_fold(self.y1, wdn)
        else:
            self.y1 = torch.empty((self.m, self.gu.n), dtype=torch.bfloat16, device=dev)
            q.qlin_gemm_w4a4(self.xq, self.xs, self.wq1, self.ws1, self.gu.k, out=self.y1)
            self.s2, self.inv2 = q.qlin_calibrate_fold(self.y1, wdn, pre=q.QLIN_PRE_GEGLU)
        self.wq2, self.ws2 = q.qlin_quantize_weights(wdn, fold_s=self.s2, had_block=128, bits=8)
        del wgu, wdn
        self.hq = torch.empty((self.m, f), dtype=torch.int8, device=dev)
        self.hs = torch.empty(self.m, dtype=torch.float32, device=dev)
        self.y2 = torch.empty((self.m, self.dn.n), dtype=torch.bfloat16, device=dev)
        self.ops = 2 * self.m * (self.gu.n * self.gu.k + self.dn.n * self.dn.k)
        self.gemm1_ops = 2 * self.m * self.gu.n * self.gu.k
        # algorithmic HBM bytes of the gate|up GEMM: packed int4 X and W once,
        # fp32 scales, its bf16 output (h [M][16384] fused, [M][32768] unfused)
        self.gemm1_bytes = (self.m * self.gu.k // 2 + self.gu.n * self.gu.k // 2 + 4 * (self.m + self.gu.n)
                            + 2 * self.y1.numel())

    def step(self, ev=None):
        q = self.q
        q.qlin_rotate_quant_act(self.x, fold_inv_s=self.inv1, had_block=128, bits=4, out=(self.xq, self.xs))
        if ev is not None:
            ev[0].record()
        if self.fused:
            q.qlin_gemm_w4a4_geglu(self.xq, self.xs, self.wq1, self.ws1, self.gu.k, out=self.y1)
        else:
            q.qlin_gemm_w4a4(self.xq, self.xs, self.wq1, self.ws1, self.gu.k, out=self.y1)
        if ev is not None:
            ev[1].record()
        if self.fused:
            q.qlin_rotate_quant_act(self.y1, fold_inv_s=self.inv2, had_block=128, bits=8, out=(self.hq, self.hs))
        else:
            q.qlin_rotate_quant_act(self.y1, k=self.dn.k, fold_inv_s=self.inv2, had_block=128, bits=8,
                                    pre=q.QLIN_PRE_GEGLU, out=(self.hq, self.hs))
        q.qlin_gemm_w8a8(self.hq, self.hs, self.wq2, self.ws2, self.dn.k, out=self.y2)


class SweepLayer:
    """One layer of the mixed-precision backbone sweep (hidden 2048, MLP 16384)
    at M tokens: q, k, v W4A4 from one int4 quantization of the attention input
    (their weights stacked along n, one 6144-column GEMM; q, k and v are column
    slices of its output), o W8A8 from the attention output, the fused gate|up
    GeGLU GEMM (W4A4) from the MLP input, then h -> int8 -> down W8A8; Hadamard
    block 128, bf16 out.
    Inputs are synthetic (one tensor each for the attention input, the
    attention output and the MLP input); weights are quantized once."""

    def __init__(self, dev, m: int):
        import torch

        import bit_ptq_vla_amd as q
        from bit_ptq_vla_amd import synth

        self.q = q
        self.m = m
        wl = synth.CFG5
        p = {pr.name: pr for pr in wl.projs}
        self.p = p
        f = p["down"].k
        bf = torch.bfloat16

        def act(name, tag):
            return synth.activation(wl, p[name], m, tag=tag).to(dev)

        def quant_w(name, x, bits, interleave=False):
            w = synth.weight(wl, p[name], tag="/L0").to(dev)
            if interleave:
                w = q.interleave_gate_up(w[:f], w[f:])
            s, inv = q.qlin_calibrate_fold(x, w)
            wq, ws = q.qlin_quantize_weights(w, fold_s=s, had_block=128, bits=bits)
            return s, inv, wq, ws

        self.x_attn = act("q", "/sweep_attn")
        self.x_o = act("o", "/sweep_o")
        self.x_mlp = act("gate_up", "/sweep_mlp")
        # q, k, v share the attention input and its fold (calibrated on q's weights)
        s_qkv, self.inv_qkv, self.wq_q, self.ws_q = quant_w("q", self.x_attn, 4)
        wk = synth.weight(wl, p["k"], tag="/L0").to(dev)
        wv = synth.weight(wl, p["v"], tag="/L0").to(dev)
        wq_k, ws_k = q.qlin_quantize_weights(wk, fold_s=s_qkv, had_block=128, bits=4)
        wq_v, ws_v = q.qlin_quantize_weights(wv, fold_s=s_qkv, had_block=128, bits=4)
        del wk, wv
        # per-row quantization: the stacked codes are the separate ones
        self.wq_qkv = torch.cat([self.wq_q, wq_k, wq_v])
        self.ws_qkv = torch.cat([self.ws_q, ws_k, ws_v])
        del self.wq_q, self.ws_q, wq_k, wq_v
        _, self.inv_o, self.wq_o, self.ws_o = quant_w("o", self.x_o, 8)
        _, self.inv_gu, self.wq_gu, self.ws_gu = quant_w("gate_up", self.x_mlp, 4, interleave=True)
        self.xq4 = torch.empty((m, 1024), dtype=torch.uint8, device=dev)
        self.xs4 = torch.empty(m, dtype=torch.float32, device=dev)
        self.xq8 = torch.empty((m, 2048), dtype=torch.int8, device=dev)
        self.xs8 = torch.empty(m, dtype=torch.float32, device=dev)
        self.h = torch.empty((m, f), dtype=bf, device=dev)
        self.hq = torch.empty((m, f), dtype=torch.int8, device=dev)
        self.hs = torch.empty(m, dtype=torch.float32, device=dev)
        self.y = {n: torch.empty((m, p[n].n), dtype=bf, device=dev) for n in ("o", "down")}
        self.y["qkv"] = torch.empty((m, p["q"].n + p["k"].n + p["v"].n), dtype=bf, device=dev)
        q.qlin_rotate_quant_act(self.x_mlp, fold_inv_s=self.inv_gu, had_block=128, bits=4, out=(self.xq4, self.xs4))
        q.qlin_gemm_w4a4_geglu(self.xq4, self.xs4, self.wq_gu, self.ws_gu, 2048, out=self.h)
        wdn = synth.weight(wl, p["down"], tag="/L0").to(dev)
        s2, self.inv_dn = q.qlin_calibrate_fold(self.h, wdn)
        self.wq_dn, self.ws_dn = q.qlin_quantize_weights(wdn, fold_s=s2, had_block=128, bits=8)
        del wdn
        self.ops = 2 * m * sum(p[n].n * p[n].k for n in ("q", "k", "v", "o", "gate_up", "down"))

    def step(self):
        q = self.q
        q.qlin_rotate_quant_act(self.x_attn, fold_inv_s=self.inv_qkv, had_block=128, bits=4,
                                out=(self.xq4, self.xs4))
        q.qlin_gemm_w4a4(self.xq4, self.xs4, self.wq_qkv, self.ws_qkv, 2048, out=self.y["qkv"])
        q.qlin_rotate_quant_act(self.x_o, fold_inv_s=self.inv_o, had_block=128, bits=8, out=(self.xq8, self.xs8))
        q.qlin_gemm_w8a8(self.xq8, self.xs8, self.wq_o, self.ws_o, 2048, out=self.y["o"])
        q.qlin_rotate_quant_act(self.x_mlp, fold_inv_s=self.inv_gu, had_block=128, bits=4, out=(self.xq4, self.xs4))
        q.qlin_gemm_w4a4_geglu(self.xq4, self.xs4, self.wq_gu, self.ws_gu, 2048, out=self.h)
        q.qlin_rotate_quant_act(self.h, fold_inv_s=self.inv_dn, had_block=128, bits=8, out=(self.hq, self.hs))
        q.qlin_gemm_w8a8(self.hq, self.hs, self.wq_dn, self.ws_dn, 16384, out=self.y["down"])


class ActionExpert:
    """The action expert's six projections at M = 50 (width 1024, MLP 4096):
    W4A4 with Hadamard block 64 (fold calibrated on the step-0 inputs) and
    W4A16 g128 on the same weights; inputs drift with the denoising step.
    build_static() adds the per-step static-table variant (W4A4, one table
    and one weight copy per step and projection)."""

    def __init__(self, dev, steps: int = 10):
        import torch

        import bit_ptq_vla_amd as q
        from bit_ptq_vla_amd import synth

        self.q = q
        wl = synth.CFG3
        self.projs = wl.projs
        self.steps = steps
        self.w4a4, self.w4a16, self.fold_s = [], [], []
        for pr in wl.projs:
            w = synth.weight(wl, pr).to(dev)
            x0 = synth.activation(wl, pr, 50, tag="/t0", std=synth.cfg3_sigma(0)).to(dev)
            s, inv = q.qlin_calibrate_fold(x0, w)
            self.fold_s.append(s)
            wq, ws = q.qlin_quantize_weights(w, fold_s=s, had_block=64, bits=4)
            wq16, ws16 = q.qlin_quantize_weights(w, bits=4, group=128)
            xs = [synth.activation(wl, pr, 50, tag=f"/t{t}", std=synth.cfg3_sigma(t)).to(dev)
                  for t in range(steps)]
            xq = torch.empty((50, pr.k // 2), dtype=torch.uint8, device=dev)
            xsc = torch.empty(50, dtype=torch.float32, device=dev)
            y = torch.empty((50, pr.n), dtype=torch.float16, device=dev)
            self.w4a4.append((pr, xs, inv, wq, ws, xq, xsc, y))
            self.w4a16.append((pr, xs, wq16, ws16, y))
        self.ops_per_step = 2 * 50 * sum(pr.n * pr.k for pr in wl.projs)
        self.w4a16_bytes = sum(pr.n * pr.k // 2 + pr.n * (pr.k // 128) * 2 + 2 * 50 * pr.k + 2 * 50 * pr.n
                               for pr in wl.projs)

    def build_static(self):
        """Per-step static activation tables (one per step and projection,
        calibrated on separate calibration tokens of that step) and the
        per-step weights with each table folded in."""
        import torch

        q = self.q
        from bit_ptq_vla_amd import synth

        wl = synth.CFG3
        dev = self.w4a4[0][3].device
        self.ones = torch.ones(50, dtype=torch.float32, device=dev)
        self.static = []
        for (pr, xs, inv, wq, ws, xq, xsc, y), s in zip(self.w4a4, self.fold_s):
            w = synth.weight(wl, pr).to(dev)
            per_step = []
            for t in range(self.steps):
                xc = synth.activation(wl, pr, 50, tag=f"/cal{t}", std=synth.cfg3_sigma(t)).to(dev)
                table = q.qlin_calibrate_step_scales(xc, fold_inv_s=inv, had_block=64, bits=4)
                wq_t, ws_t = q.qlin_quantize_weights_step(w, table, fold_s=s, had_block=64, bits=4)
                per_step.append((table, wq_t, ws_t))
            self.static.append((pr, xs, inv, per_step, xq, y))

    def build_merged(self):
        """q, k and v reading one input (the q projection's per-step tokens,
        as in a transformer block) with their weights stacked along n: one
        fold calibrated on the stacked weights, one activation quantization
        and one 3072-column projection per step instead of three of each."""
        import torch

        q = self.q
        from bit_ptq_vla_amd import synth

        wl = synth.CFG3
        names = [pr.name for pr in self.projs]
        iq = [names.index(nm) for nm in ("q", "k", "v")]
        self.rest = [i for i in range(len(self.projs)) if i not in iq]
        dev = self.w4a4[0][3].device
        w = torch.cat([synth.weight(wl, self.projs[i]).to(dev) for i in iq])
        xs = self.w4a4[iq[0]][1]
        s, inv = q.qlin_calibrate_fold(xs[0], w)
        wq, ws = q.qlin_quantize_weights(w, fold_s=s, had_block=64, bits=4)
        # group-128 rows quantize independently: the stacked codes are the separate ones
        wq16 = torch.cat([self.w4a16[i][2] for i in iq])
        ws16 = torch.cat([self.w4a16[i][3] for i in iq])
        k = self.projs[iq[0]].k
        self.merged = (xs, inv, wq, ws, wq16, ws16, k,
                       torch.empty((50, k // 2), dtype=torch.uint8, device=dev),
                       torch.empty(50, dtype=torch.float32, device=dev),
                       torch.empty((50, w.shape[0]), dtype=torch.float16, device=dev))

    def run_w4a4_merged(self):
        q = self.q
        xs, inv, wq, ws, _, _, k, xq, xsc, y = self.merged
        for t in range(self.steps):
            q.qlin_rotate_quant_act(xs[t], fold_inv_s=inv, had_block=64, bits=4, out=(xq, xsc))
            q.qlin_gemm_w4a4(xq, xsc, wq, ws, k, out=y)
            for i in self.rest:
                pr, xs_i, inv_i, wq_i, ws_i, xq_i, xsc_i, y_i = self.w4a4[i]
                q.qlin_rotate_quant_act(xs_i[t], fold_inv_s=inv_i, had_block=64, bits=4, out=(xq_i, xsc_i))
                q.qlin_gemm_w4a4(xq_i, xsc_i, wq_i, ws_i, pr.k, out=y_i)

    def run_w4a16_merged(self):
        q = self.q
        xs, _, _, _, wq16, ws16, _, _, _, y = self.merged
        for t in range(self.steps):
            q.qlin_gemv_w4a16(xs[t], wq16, ws16, out=y)
            for i in self.rest:
                pr, xs_i, wq_i, ws_i, y_i = self.w4a16[i]
                q.qlin_gemv_w4a16(xs_i[t], wq_i, ws_i, out=y_i)

    def run_w4a4_static(self):
        q = self.q
        for t in range(self.steps):
            for pr, xs, inv, per_step, xq, y in self.static:
                table, wq_t, ws_t = per_step[t]
                q.qlin_rotate_quant_act_static(xs[t], table, fold_inv_s=inv, had_block=64, bits=4, out=xq)
                q.qlin_gemm_w4a4(xq, self.ones, wq_t, ws_t, pr.k, out=y)

    def run_w4a4(self):
        q = self.q
        for t in range(self.steps):
            for pr, xs, inv, wq, ws, xq, xsc, y in self.w4a4:
                q.qlin_rotate_quant_act(xs[t], fold_inv_s=inv, had_block=64, bits=4, out=(xq, xsc))
                q.qlin_gemm_w4a4(xq, xsc, wq, ws, pr.k, out=y)

    def run_w4a16(self):
        q = self.q
        for t in range(self.steps):
            for pr, xs, wq16, ws16, y in self.w4a16:
                q.qlin_gemv_w4a16(xs[t], wq16, ws16, out=y)

