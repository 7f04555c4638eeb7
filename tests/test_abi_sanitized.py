"""The C ABI's argument validation under AddressSanitizer and
UndefinedBehaviorSanitizer (host only, no GPU).

qlin_api.cpp and plan.cpp are built by the host compiler with both
sanitizers and stand-ins for the kernel launchers
(bit_ptq_vla_amd/build_host_sanitized.py); tests/test_abi_cpu.py then runs
against that library in a fresh Python process with the ASan runtime
preloaded, so every validation path it exercises (null, shape, dtype,
alignment, alias and workspace checks, the empty-call fast paths and the
device check) runs instrumented.  A sanitizer report aborts that process and
fails this test.
"""

import os
import subprocess
import sys

import pytest

from bit_ptq_vla_amd import build_host_sanitized as hs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_abi_validation_under_asan_and_ubsan(tmp_path):
    try:
        asan = hs.runtime("libasan.so")
        lib = hs.build(str(tmp_path / "libqlin_host_sanitized.so"))
    except RuntimeError as e:
        pytest.skip(f"no host sanitizer toolchain: {e}")
    env = dict(os.environ)
    env.update({
        "QLIN_LIB_PATH": lib,
        "LD_PRELOAD": asan,
        # Python and its extension modules are not instrumented: no leak report
        # at exit and no checks of their allocator pairing
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1:alloc_dealloc_mismatch=0"
                        ":detect_odr_violation=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out
