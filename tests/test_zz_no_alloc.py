"""The allocation-free GEMM entry point (qlin_gemm_static_ws) against the
workspace one (qlin_gemm_ws), through the C ABI (GPU only).

qlin_gemm_static_ws takes its split-K partials from the library's static
device scratch.  Two calls in a row, the second with a smaller input, must
each equal qlin_gemm_ws on the same inputs bit for bit (integer partial sums
and the same epilogue), and both must equal the oracle's integer GEMM on the
raw accumulators.  A shape whose partials exceed the scratch is rejected.
"""

import sys

import numpy as np
import pytest
import torch

import bit_ptq_vla_amd as q
import oracle
from bit_ptq_vla_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
SEED = 777


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def codes(scheme, tag, m, n, k):
    abits, wbits = {q.QLIN_W8A8: (8, 8), q.QLIN_W4A8: (8, 4), q.QLIN_W4A4: (4, 4)}[scheme]
    a = synth.random_codes(SEED, f"na/A/{tag}", m, k, abits)
    b = synth.random_codes(SEED, f"na/B/{tag}", n, k, wbits)
    sx = synth.random_scales(SEED, f"na/sx/{tag}", m)
    sw = synth.random_scales(SEED, f"na/sw/{tag}", n)
    return a, b, sx, sw, abits, wbits


def unpack(t, bits):
    a = t.cpu().numpy()
    return oracle.unpack_int4(a) if bits == 4 else a.astype(np.int64)


# (scheme, m, n, k): each takes split-K, so the static scratch is written and read
CALLS = [
    [(q.QLIN_W8A8, 816, 2048, 16384), (q.QLIN_W8A8, 300, 1024, 8192)],   # FFN-down at 816 tokens, then smaller
    [(q.QLIN_W4A8, 400, 2048, 8192), (q.QLIN_W4A8, 129, 512, 4096)],
]


@pytest.mark.parametrize("calls", CALLS, ids=["w8a8", "w4a8"])
def test_static_scratch_matches_workspace_twice(calls):
    for i, (scheme, m, n, k) in enumerate(calls):
        need = q.gemm_workspace_bytes(scheme, m, n, k)
        say(f"no-alloc call {i}: scheme {scheme} {m}x{n}x{k}, split-K partials {need} bytes")
        assert 0 < need <= q.QLIN_STATIC_SCRATCH_BYTES
        a, b, sx, sw, abits, wbits = codes(scheme, f"{scheme}/{m}/{n}/{k}", m, n, k)
        a, b, sx, sw = a.to(DEV), b.to(DEV), sx.to(DEV), sw.to(DEV)
        fn = {q.QLIN_W8A8: q.qlin_gemm_w8a8, q.QLIN_W4A8: q.qlin_gemm_w4a8}[scheme]
        work = q.gemm_workspace(scheme, m, n, k, DEV)
        for dt in (torch.int32, torch.bfloat16):
            got = q.qlin_gemm_static_ws(scheme, a, sx if dt != torch.int32 else None, b,
                                        sw if dt != torch.int32 else None, k, y_dtype=dt)
            ref = fn(a, sx if dt != torch.int32 else None, b, sw if dt != torch.int32 else None, k, y_dtype=dt,
                     workspace=work)
            torch.cuda.synchronize()
            bits = torch.int32 if dt == torch.int32 else torch.int16
            assert torch.equal(got.view(bits), ref.view(bits)), f"call {i} {dt}"
            if dt == torch.int32:
                rows = np.unique(np.r_[0, m - 1, np.arange(1, m, max(1, m // 16))])
                acc = oracle.int_gemm(unpack(a.cpu(), abits)[rows], unpack(b.cpu(), wbits))
                assert np.array_equal(got.cpu().numpy()[rows].astype(np.int64), acc), f"call {i} accumulators"


def test_static_scratch_rejects_oversize_and_small_m_ok():
    # W4A4 1024 x 4096 x 8192: 128 tiles of 128 x 256, four splits -> 64 MiB of partials
    m, n, k = 1024, 4096, 8192
    assert q.gemm_workspace_bytes(q.QLIN_W4A4, m, n, k) > q.QLIN_STATIC_SCRATCH_BYTES
    a = torch.zeros((m, k // 2), dtype=torch.uint8, device=DEV)
    b = torch.zeros((n, k // 2), dtype=torch.uint8, device=DEV)
    with pytest.raises(q.QlinError) as e:
        q.qlin_gemm_static_ws(q.QLIN_W4A4, a, None, b, None, k, y_dtype=torch.int32)
    assert e.value.status == q.QLIN_ERR_WORKSPACE
    # a small-M call takes no split: it runs without the scratch
    a, b, sx, sw, abits, wbits = codes(q.QLIN_W4A4, "small", 40, 256, 2048)
    got = q.qlin_gemm_static_ws(q.QLIN_W4A4, a.to(DEV), None, b.to(DEV), None, 2048, y_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.int64), oracle.int_gemm(unpack(a, 4), unpack(b, 4)))
