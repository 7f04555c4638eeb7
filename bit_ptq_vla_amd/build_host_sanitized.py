"""Host-only sanitizer build of the C ABI's argument validation.

Compiles qlin_api.cpp (validation, device check, dispatch) and plan.cpp (GEMM
and scratch planning) with the host compiler, AddressSanitizer and
UndefinedBehaviorSanitizer, against host_stubs.cpp in place of the kernels,
into a shared library that exports the same C entry points as libqlin.so.
The ABI tests run against it with QLIN_LIB_PATH pointing at it and the ASan
runtime preloaded into the Python process (tests/test_abi_sanitized.py).

Run as ``python -m bit_ptq_vla_amd.build_host_sanitized OUT.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["qlin_api.cpp", "plan.cpp", "host_stubs.cpp"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compiler() -> str:
    cxx = shutil.which("g++")
    if cxx is None:
        raise RuntimeError("g++ not found")
    return cxx


def runtime(name: str) -> str:
    """Path of the compiler's sanitizer runtime library (libasan.so, libubsan.so)."""
    path = subprocess.run([compiler(), f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"{name} not found next to {compiler()}")
    return path


def build(out: str) -> str:
    cmd = [compiler(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-Wall", "-Wextra", "-Werror",
           "-shared", "-fPIC"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES]
    cmd += [f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{r.stdout}{r.stderr}")
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "libqlin_host_sanitized.so")))
