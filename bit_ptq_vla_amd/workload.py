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
        # split-K scratch of the down GEMM (its 112 output tiles under-fill the chip)
        self.ws_dn = q.gemm_workspace(q.QLIN_W8A8, self.m, self.dn.n, self.dn.k, dev)
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
        q.qlin_gemm_w8a8(self.hq, self.hs, self.wq2, self.ws2, self.dn.k, out=self.y2, workspace=self.ws_dn)


class SweepModel:
    """The 18-layer mixed-precision backbone sweep (hidden 2048, MLP 16384,
    Hadamard block 128, bf16 out) with distinct weights per layer.

    Per layer: q, k, v W4A4 from one int4 quantization of the attention input
    (their weights stacked along n with one fold calibrated on the stacked
    weights: one 6144-column GEMM whose column slices are q, k and v); o W8A8
    from the attention output; the fused gate|up GeGLU GEMM (W4A4, gate and up
    rows interleaved in blocks of 32) from the MLP input; then h -> fold,
    Hadamard, int8 -> down W8A8.  8 launches per layer.

    Inputs are synthetic, drawn on the device (synth.device_normal): one
    tensor each for the attention input, the attention output and the MLP
    input, N(0, 1) with 1% outlier channels x 30, shared by the layers (a
    layer's work does not depend on the values).  Weights N(0, 0.02) fp16 per
    layer and projection, quantized once (offline).  Buffers are sized for
    m_max tokens; step(m) runs the first m tokens (row prefixes), so the
    smaller batches of the sweep reuse the same weights and folds.
    """

    HID, FFN = 2048, 16384

    def __init__(self, dev, m_max: int, layers: int = 18, e2m3: bool = False):
        """e2m3: also keep the W4A4 weights (q|k|v, gate|up) in FP6 E2M3
        storage -- the same int4-grid codes and scales -- so that
        run_layer can take the FP6 matrix-core GEMMs (use_e2m3)."""
        import torch

        import bit_ptq_vla_amd as q
        from bit_ptq_vla_amd import synth

        self.q = q
        self.dev = dev
        self.m_max = m_max
        self.layers = layers
        wl = synth.CFG5
        self.wl = wl
        hid, ffn = self.HID, self.FFN
        nout = wl.n_outliers(hid)

        def act(tag):
            return synth.device_normal(wl.seed, f"{wl.name}/sweep/{tag}/m{m_max}", (m_max, hid), dev,
                                       dtype=wl.x_dtype, outliers=nout, outlier_scale=wl.x_outlier_scale)

        self.x_attn, self.x_o, self.x_mlp = act("attn_in"), act("attn_out"), act("mlp_in")
        bf = torch.bfloat16
        self.e2m3 = e2m3
        self.use_e2m3 = False
        self.xq4 = torch.empty((m_max, hid // 2), dtype=torch.uint8, device=dev)
        self.xq6 = torch.empty((m_max, hid * 3 // 4), dtype=torch.uint8, device=dev) if e2m3 else None
        self.xs4 = torch.empty(m_max, dtype=torch.float32, device=dev)
        self.xq8 = torch.empty((m_max, hid), dtype=torch.int8, device=dev)
        self.xs8 = torch.empty(m_max, dtype=torch.float32, device=dev)
        self.h = torch.empty((m_max, ffn), dtype=bf, device=dev)
        self.hq = torch.empty((m_max, ffn), dtype=torch.int8, device=dev)
        self.hs = torch.empty(m_max, dtype=torch.float32, device=dev)
        self.y_qkv = torch.empty((m_max, 3 * hid), dtype=bf, device=dev)
        self.y_o = torch.empty((m_max, hid), dtype=bf, device=dev)
        self.y_dn = torch.empty((m_max, hid), dtype=bf, device=dev)
        self.layer = [self._build_layer(li) for li in range(layers)]
        torch.cuda.synchronize(dev)
        # int8 ops per token of one layer: q, k, v, o, gate|up, down
        self.ops_per_token_layer = 2 * (3 * hid * hid + hid * hid + 2 * ffn * hid + hid * ffn)
        self._ws = {}

    def weight(self, li: int, name: str, n: int, k: int):
        """Float weights [n][k] of layer li's projection (fp16, on the device)."""
        from bit_ptq_vla_amd import synth

        wl = self.wl
        return synth.device_normal(wl.seed, f"{wl.name}/L{li}/{name}/w", (n, k), self.dev, std=wl.w_std,
                                   dtype=wl.w_dtype)

    def _build_layer(self, li: int) -> dict:
        import torch

        q = self.q
        hid, ffn = self.HID, self.FFN
        L = {}
        w_qkv = torch.cat([self.weight(li, nm, hid, hid) for nm in ("q", "k", "v")])
        s, L["inv_qkv"] = q.qlin_calibrate_fold(self.x_attn, w_qkv)
        L["wq_qkv"], L["ws_qkv"] = q.qlin_quantize_weights(w_qkv, fold_s=s, had_block=128, bits=4)
        if self.e2m3:
            L["wq6_qkv"], _ = q.qlin_quantize_weights(w_qkv, fold_s=s, had_block=128, bits=q.QLIN_BITS_E2M3)
        del w_qkv
        w_o = self.weight(li, "o", hid, hid)
        s, L["inv_o"] = q.qlin_calibrate_fold(self.x_o, w_o)
        L["wq_o"], L["ws_o"] = q.qlin_quantize_weights(w_o, fold_s=s, had_block=128, bits=8)
        del w_o
        w_gu = self.weight(li, "gate_up", 2 * ffn, hid)          # gate rows, then up rows
        w_gu = q.interleave_gate_up(w_gu[:ffn], w_gu[ffn:])
        s, L["inv_gu"] = q.qlin_calibrate_fold(self.x_mlp, w_gu)
        L["wq_gu"], L["ws_gu"] = q.qlin_quantize_weights(w_gu, fold_s=s, had_block=128, bits=4)
        if self.e2m3:
            L["wq6_gu"], _ = q.qlin_quantize_weights(w_gu, fold_s=s, had_block=128, bits=q.QLIN_BITS_E2M3)
        del w_gu
        # the down fold is calibrated on this layer's own h
        q.qlin_rotate_quant_act(self.x_mlp, fold_inv_s=L["inv_gu"], had_block=128, bits=4, out=(self.xq4, self.xs4))
        q.qlin_gemm_w4a4_geglu(self.xq4, self.xs4, L["wq_gu"], L["ws_gu"], hid, out=self.h)
        w_dn = self.weight(li, "down", hid, ffn)
        s, L["inv_dn"] = q.qlin_calibrate_fold(self.h, w_dn)
        L["wq_dn"], L["ws_dn"] = q.qlin_quantize_weights(w_dn, fold_s=s, had_block=128, bits=8)
        del w_dn
        return L

    def workspace(self, m: int):
        """Split-K scratch of the down and o GEMMs at m tokens (None: no split)."""
        if m not in self._ws:
            q = self.q
            a = q.gemm_workspace(q.QLIN_W8A8, m, self.HID, self.FFN, self.dev)
            b = q.gemm_workspace(q.QLIN_W8A8, m, self.HID, self.HID, self.dev)
            self._ws[m] = (a, b)
        return self._ws[m]

    def ops(self, m: int) -> int:
        return self.layers * m * self.ops_per_token_layer

    def run_layer(self, L: dict, m: int, ev=None, evs=None):
        """One layer at m tokens.  ev: (start, end) events around the gate|up
        GEMM; evs: a list of 9 events bracketing the 8 launches."""
        q = self.q
        hid, ffn = self.HID, self.FFN
        ws_dn, ws_o = self.workspace(m)

        def mark(i):
            if evs is not None:
                evs[i].record()

        xq4, xs4, xq8, xs8 = self.xq4[:m], self.xs4[:m], self.xq8[:m], self.xs8[:m]
        # the W4A4 codes packed int4, or in E2M3 storage on the FP6 matrix cores
        e6 = self.use_e2m3
        xq_w4, bits_w4 = (self.xq6[:m], q.QLIN_BITS_E2M3) if e6 else (xq4, 4)
        mark(0)
        q.qlin_rotate_quant_act(self.x_attn[:m], fold_inv_s=L["inv_qkv"], had_block=128, bits=bits_w4,
                                out=(xq_w4, xs4))
        mark(1)
        if e6:
            q.qlin_gemm_e2m3(xq_w4, xs4, L["wq6_qkv"], L["ws_qkv"], hid, out=self.y_qkv[:m])
        else:
            q.qlin_gemm_w4a4(xq4, xs4, L["wq_qkv"], L["ws_qkv"], hid, out=self.y_qkv[:m])
        mark(2)
        q.qlin_rotate_quant_act(self.x_o[:m], fold_inv_s=L["inv_o"], had_block=128, bits=8, out=(xq8, xs8))
        mark(3)
        q.qlin_gemm_w8a8(xq8, xs8, L["wq_o"], L["ws_o"], hid, out=self.y_o[:m], workspace=ws_o)
        mark(4)
        q.qlin_rotate_quant_act(self.x_mlp[:m], fold_inv_s=L["inv_gu"], had_block=128, bits=bits_w4,
                                out=(xq_w4, xs4))
        mark(5)
        if ev is not None:
            ev[0].record()
        if e6:
            q.qlin_gemm_geglu(q.QLIN_W4A4_E2M3, xq_w4, xs4, L["wq6_gu"], L["ws_gu"], hid, out=self.h[:m])
        else:
            q.qlin_gemm_w4a4_geglu(xq4, xs4, L["wq_gu"], L["ws_gu"], hid, out=self.h[:m])
        if ev is not None:
            ev[1].record()
        mark(6)
        q.qlin_rotate_quant_act(self.h[:m], fold_inv_s=L["inv_dn"], had_block=128, bits=8,
                                out=(self.hq[:m], self.hs[:m]))
        mark(7)
        q.qlin_gemm_w8a8(self.hq[:m], self.hs[:m], L["wq_dn"], L["ws_dn"], ffn, out=self.y_dn[:m], workspace=ws_dn)
        mark(8)

    def step(self, m: int, evs=None):
        """All layers at m tokens; evs: per-layer (start, end) event pairs
        around the gate|up GEMM launches."""
        for li, L in enumerate(self.layer):
            self.run_layer(L, m, ev=None if evs is None else evs[li])


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

    def build_cold_copies(self, min_bytes: int):
        """Distinct copies of the W4A4 and W4A16 weights, one per step of each
        group of `steps` steps, until the copies total at least min_bytes (so
        that a step's weights come from HBM, not from L2 / Infinity Cache).
        Returns the list of groups; group c holds `steps` weight sets."""
        per_set = sum(wq.numel() + ws.numel() * 4 for _, _, _, wq, ws, _, _, _ in self.w4a4)
        per_set += sum(wq16.numel() + ws16.numel() * 2 for _, _, wq16, ws16, _ in self.w4a16)
        groups = max(1, -(-min_bytes // (per_set * self.steps)))
        self.cold = []
        for _ in range(groups):
            sets = []
            for _t in range(self.steps):
                sets.append(([(wq.clone(), ws.clone()) for _, _, _, wq, ws, _, _, _ in self.w4a4],
                             [(wq16.clone(), ws16.clone()) for _, _, wq16, ws16, _ in self.w4a16]))
            self.cold.append(sets)
        return self.cold

    def run_w4a4_cold(self, c: int):
        """The W4A4 steps with group c of the cold weight copies (step t: set t)."""
        q = self.q
        for t in range(self.steps):
            w4, _ = self.cold[c][t]
            for (pr, xs, inv, _, _, xq, xsc, y), (wq, ws) in zip(self.w4a4, w4):
                q.qlin_rotate_quant_act(xs[t], fold_inv_s=inv, had_block=64, bits=4, out=(xq, xsc))
                q.qlin_gemm_w4a4(xq, xsc, wq, ws, pr.k, out=y)

    def run_w4a16_cold(self, c: int):
        q = self.q
        for t in range(self.steps):
            _, w16 = self.cold[c][t]
            for (pr, xs, _, _, y), (wq16, ws16) in zip(self.w4a16, w16):
                q.qlin_gemv_w4a16(xs[t], wq16, ws16, out=y)

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

