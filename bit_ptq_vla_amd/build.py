"""Builds libqlin.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Run as ``python -m bit_ptq_vla_amd.build``.  The library is written next to
this file and always rebuilt from source.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlin.so")
SOURCES = ["act_quant.hip", "gemm_i8.hip", "gemv_w4a16.hip", "skinny_w4a16.hip",
           "skinny_int.hip", "composite.hip", "plan.cpp",
           "qlin_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqlin.so)")


def common_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # no packed-fp32 instructions in generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"]


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")


def build(verbose: bool = True) -> str:
    with tempfile.TemporaryDirectory(prefix="qlin_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".", "_") + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
            list(ex.map(_compile, SOURCES, objs))
        out_tmp = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
        os.replace(out_tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
