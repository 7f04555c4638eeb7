"""Device-resident workloads of the projection path, shared by bench.py and
the profiling driver.  Nothing here computes the method itself: every step
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
