"""Seeded synthetic inputs with the shapes and distributions of the workloads.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the quantization method's arithmetic.  The same bytes feed the
HIP path (as device tensors) and the CPU oracle (widened exactly to float64).

Every tensor has its own PCG64 stream: SeedSequence(entropy=config seed,
spawn_key=(crc32(tensor name),)).  Values are float32 normals scaled by the
stated standard deviation; "outlier channels" are input channels picked from
the same stream without replacement and multiplied by a factor; the result is
rounded to float16 / bfloat16 with round-half-to-even (torch's cast).
"""

from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np
import torch

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def rng_for(seed: int, name: str) -> np.random.Generator:
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(zlib.crc32(name.encode()),))
    return np.random.Generator(np.random.PCG64(ss))


def normal_tensor(seed: int, name: str, shape, std: float = 1.0, dtype: str = "f16",
                  outliers: int = 0, outlier_scale: float = 1.0) -> torch.Tensor:
    """CPU tensor of the given storage dtype; outliers scale whole columns
    (input channels, the last axis)."""
    rng = rng_for(seed, name)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if outliers:
        cols = rng.choice(shape[-1], size=outliers, replace=False)
        a[..., cols] *= np.float32(outlier_scale)
    return torch.from_numpy(a).to(_TORCH_DTYPES[dtype])


def device_normal(seed: int, name: str, shape, device, std: float = 1.0, dtype: str = "f16",
                  outliers: int = 0, outlier_scale: float = 1.0) -> torch.Tensor:
    """Device tensor of the given storage dtype drawn on the device by torch's
    Philox generator, seeded with (seed << 32) ^ crc32(name): float32 normals
    times std, `outliers` input channels (last axis, chosen without
    replacement from the same generator) times outlier_scale, rounded to the
    storage dtype with round-half-to-even.  For the multi-gigabyte inputs of
    the 18-layer sweep, which a host generator would take minutes to draw;
    the oracle gets the same bytes by copying them back."""
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 32) ^ zlib.crc32(name.encode()))
    a = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        a *= std
    if outliers:
        cols = torch.randperm(shape[-1], generator=g, device=device)[:outliers]
        a[..., cols] *= outlier_scale
    return a.to(_TORCH_DTYPES[dtype])


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU tensor to a float64 NumPy array."""
    return t.detach().cpu().to(torch.float64).numpy()


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Proj:
    """One projection: W is [n][k]; scheme is 'w4a4', 'w8a8' or 'w4a16'."""
    name: str
    n: int
    k: int
    scheme: str


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    x_dtype: str
    w_dtype: str
    out_dtype: str
    w_std: float
    had_block: int
    fold: bool
    x_outliers_frac: float = 0.0   # fraction of input channels that are outliers
    x_outliers: int = 0            # or a fixed count
    x_outlier_scale: float = 1.0
    projs: tuple = field(default_factory=tuple)
    ms: tuple = (1,)

    def n_outliers(self, k: int) -> int:
        if self.x_outliers:
            return self.x_outliers
        return int(self.x_outliers_frac * k)


# Single W4A4 linear, 16 x 512 x 512.
CFG1 = Workload("single_w4a4_16x512x512", seed=0, x_dtype="f16", w_dtype="f16", out_dtype="f16",
                w_std=0.02, had_block=64, fold=True, x_outliers=4, x_outlier_scale=20.0,
                projs=(Proj("linear", 512, 512, "w4a4"),), ms=(16,))

# Backbone-shaped MLP block: gate|up W4A4 (one N = 2 x 16384 GEMM), GeGLU,
# down W8A8, bf16 activations and outputs, Hadamard block 128, M = 816.
CFG2 = Workload("backbone_mlp_m816_h2048_f16384", seed=1, x_dtype="bf16", w_dtype="f16",
                out_dtype="bf16", w_std=0.02, had_block=128, fold=True,
                x_outliers_frac=0.01, x_outlier_scale=30.0,
                projs=(Proj("gate_up", 32768, 2048, "w4a4"), Proj("down", 2048, 16384, "w8a8")),
                ms=(816,))

# Action-expert projections over 10 denoising steps, M = 50, width 1024.
CFG3 = Workload("action_expert_m50_w1024_steps10", seed=2, x_dtype="f16", w_dtype="f16",
                out_dtype="f16", w_std=0.02, had_block=64, fold=True,
                projs=(Proj("q", 1024, 1024, "w4a4"), Proj("k", 1024, 1024, "w4a4"),
                       Proj("v", 1024, 1024, "w4a4"), Proj("o", 1024, 1024, "w4a4"),
                       Proj("up", 4096, 1024, "w4a4"), Proj("down", 1024, 4096, "w4a4")),
                ms=(50,))
CFG3_STEPS = 10


def cfg3_sigma(t: int) -> float:
    return 0.5 + 0.1 * t


# 7B-decoder-shaped projections: M = 1 W4A16 g128 and M = 256 W8A8.
CFG4 = Workload("decoder7b_h4096_f11008", seed=3, x_dtype="f16", w_dtype="f16", out_dtype="f16",
                w_std=0.015, had_block=0, fold=False,
                projs=(Proj("q", 4096, 4096, "w4a16"), Proj("k", 4096, 4096, "w4a16"),
                       Proj("v", 4096, 4096, "w4a16"), Proj("o", 4096, 4096, "w4a16"),
                       Proj("gate", 11008, 4096, "w4a16"), Proj("up", 11008, 4096, "w4a16"),
                       Proj("down", 4096, 11008, "w4a16")),
                ms=(1, 256))

# 18-layer mixed-precision backbone sweep, hidden 2048 / MLP 16384.
CFG5 = Workload("backbone_sweep_18l_h2048_f16384", seed=4, x_dtype="bf16", w_dtype="f16",
                out_dtype="bf16", w_std=0.02, had_block=128, fold=True,
                x_outliers_frac=0.01, x_outlier_scale=30.0,
                projs=(Proj("q", 2048, 2048, "w4a4"), Proj("k", 2048, 2048, "w4a4"),
                       Proj("v", 2048, 2048, "w4a4"), Proj("o", 2048, 2048, "w8a8"),
                       Proj("gate_up", 32768, 2048, "w4a4"), Proj("down", 2048, 16384, "w8a8")),
                ms=(816, 6528, 52224))
CFG5_LAYERS = 18

WORKLOADS = {w.name: w for w in (CFG1, CFG2, CFG3, CFG4, CFG5)}


def activation(wl: Workload, proj: Proj, m: int, tag: str = "", std: float = 1.0) -> torch.Tensor:
    """Input activations [m][proj.k] of a workload's projection."""
    return normal_tensor(wl.seed, f"{wl.name}/{proj.name}/x{tag}/m{m}", (m, proj.k), std=std,
                         dtype=wl.x_dtype, outliers=wl.n_outliers(proj.k),
                         outlier_scale=wl.x_outlier_scale)


def weight(wl: Workload, proj: Proj, tag: str = "") -> torch.Tensor:
    """Float weights [proj.n][proj.k] of a workload's projection."""
    return normal_tensor(wl.seed, f"{wl.name}/{proj.name}/w{tag}", (proj.n, proj.k),
                         std=wl.w_std, dtype=wl.w_dtype)


def random_codes(seed: int, name: str, rows: int, k: int, bits: int) -> torch.Tensor:
    """Uniform random operand bytes for integer-GEMM tests: int8 codes in
    [-127, 127] as int8 [rows][k], or arbitrary packed bytes (every nibble
    value, -8 included) as uint8 [rows][k/2]."""
    rng = rng_for(seed, name)
    if bits == 8:
        return torch.from_numpy(rng.integers(-127, 128, size=(rows, k), dtype=np.int8))
    return torch.from_numpy(rng.integers(0, 256, size=(rows, k // 2), dtype=np.uint8))


def random_grid_codes(seed: int, name: str, rows: int, k: int) -> np.ndarray:
    """Uniform codes of the symmetric int4 grid, -7 .. 7 (the codes the
    quantizers write), as int8 [rows][k] (numpy; storage is up to the caller)."""
    rng = rng_for(seed, name)
    return rng.integers(-7, 8, size=(rows, k), dtype=np.int8)


def random_scales(seed: int, name: str, n: int) -> torch.Tensor:
    """Positive float32 scales spread over two decades."""
    rng = rng_for(seed, name)
    return torch.from_numpy((10.0 ** rng.uniform(-3, -1, size=n)).astype(np.float32))
