"""C-ABI checks that need no GPU: the library loads, exports every entry
point the header declares, and rejects invalid arguments with the documented
status before any HIP call (so fake, never-dereferenced pointers are safe).
"""

import ctypes
import os
import re

import pytest
import torch

import bit_ptq_vla_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")

P = 0x10000     # aligned fake device pointers (never dereferenced)
P2 = 0x20000000
P3 = 0x40000000
P4 = 0x60000000
BAD = 0x10001   # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.LIB_PATH):
        pytest.fail("libqlin.so is not built; run `python -m bit_ptq_vla_amd.build`")
    return q.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:qlin_status|int32_t|int64_t|const char\*)\s+(qlin_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for n in ("qlin_rotate_quant_act", "qlin_quantize_weights", "qlin_gemm_w4a4", "qlin_gemm_w8a8", "qlin_gemm_w4a8",
              "qlin_gemm_w4a4_geglu", "qlin_gemv_w4a16", "qlin_calibrate_fold", "qlin_abi_version",
              "qlin_status_string", "qlin_calibrate_step_scales", "qlin_rotate_quant_act_static",
              "qlin_quantize_weights_step", "qlin_calibrate_composite", "qlin_rotate_quant_act_composite",
              "qlin_quantize_weights_composite", "qlin_calibrate_composite_work_bytes", "qlin_gemm_ws",
              "qlin_gemm_workspace_bytes", "qlin_gemm_static_ws", "qlin_gemm_geglu", "qlin_stream_read"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in q.SIGNATURES, f"binding lacks {name}"


def test_abi_version_and_status_strings(lib):
    assert lib.qlin_abi_version() == 3
    for s in range(0, 11):
        assert lib.qlin_status_string(s).decode() not in ("", "unknown status")
    assert lib.qlin_status_string(99).decode() == "unknown status"


# ---- qlin_rotate_quant_act(x, dt, m, k, ldx, pre, inv_s, b, bits, xq, xs, stream)

def rqa(lib, x=P, dt=0, m=4, k=512, ldx=512, pre=0, inv=None, b=64, bits=4, xq=P2, xs=P3):
    return lib.qlin_rotate_quant_act(x, dt, m, k, ldx, pre, inv, b, bits, xq, xs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), q.QLIN_ERR_NULL), (dict(xq=None), q.QLIN_ERR_NULL), (dict(xs=None), q.QLIN_ERR_NULL),
    (dict(dt=3), q.QLIN_ERR_DTYPE), (dict(dt=7), q.QLIN_ERR_DTYPE),
    (dict(bits=3), q.QLIN_ERR_UNSUPPORTED), (dict(bits=16), q.QLIN_ERR_UNSUPPORTED),
    (dict(b=48), q.QLIN_ERR_UNSUPPORTED), (dict(b=512), q.QLIN_ERR_UNSUPPORTED),
    (dict(pre=2), q.QLIN_ERR_UNSUPPORTED),
    (dict(k=500, ldx=504), q.QLIN_ERR_SHAPE), (dict(k=4), q.QLIN_ERR_SHAPE),
    (dict(m=-1), q.QLIN_ERR_SHAPE), (dict(ldx=256), q.QLIN_ERR_SHAPE), (dict(ldx=513), q.QLIN_ERR_SHAPE),
    (dict(k=520, ldx=520), q.QLIN_ERR_SHAPE),        # not a multiple of the Hadamard block
    (dict(k=65536, ldx=65536, b=0), q.QLIN_ERR_SHAPE),
    (dict(pre=1, ldx=512), q.QLIN_ERR_SHAPE),         # GeGLU needs ldx >= 2k
    (dict(x=BAD), q.QLIN_ERR_ALIGN), (dict(xq=BAD), q.QLIN_ERR_ALIGN), (dict(inv=BAD), q.QLIN_ERR_ALIGN),
    (dict(xq=P + 256), q.QLIN_ERR_ALIAS), (dict(xs=P2 + 16), q.QLIN_ERR_ALIAS),
])
def test_rotate_quant_act_rejects(lib, kw, status):
    assert rqa(lib, **kw) == status


def test_rotate_quant_act_empty_is_ok(lib):
    assert rqa(lib, m=0) == q.QLIN_OK


# ---- qlin_quantize_weights(w, dt, n, k, fold_s, b, bits, group, wq, ws, stream)

def qw(lib, w=P, dt=0, n=8, k=512, s=None, b=64, bits=4, group=0, wq=P2, ws=P3):
    return lib.qlin_quantize_weights(w, dt, n, k, s, b, bits, group, wq, ws, None)


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), q.QLIN_ERR_NULL), (dict(wq=None), q.QLIN_ERR_NULL), (dict(ws=None), q.QLIN_ERR_NULL),
    (dict(dt=3), q.QLIN_ERR_DTYPE), (dict(bits=2), q.QLIN_ERR_UNSUPPORTED),
    (dict(group=64, b=0), q.QLIN_ERR_UNSUPPORTED), (dict(group=128, b=0, bits=8), q.QLIN_ERR_UNSUPPORTED),
    (dict(group=128, b=64), q.QLIN_ERR_UNSUPPORTED), (dict(group=128, b=0, s=P4), q.QLIN_ERR_UNSUPPORTED),
    (dict(n=0), q.QLIN_ERR_SHAPE), (dict(k=500), q.QLIN_ERR_SHAPE),
    (dict(group=128, b=0, k=520), q.QLIN_ERR_SHAPE), (dict(k=544), q.QLIN_ERR_SHAPE),
    (dict(w=BAD), q.QLIN_ERR_ALIGN), (dict(s=BAD), q.QLIN_ERR_ALIGN), (dict(ws=BAD), q.QLIN_ERR_ALIGN),
    (dict(wq=P + 1024), q.QLIN_ERR_ALIAS),
])
def test_quantize_weights_rejects(lib, kw, status):
    assert qw(lib, **kw) == status


# ---- qlin_gemm_*(xq, sx, wq, sw, m, n, k, y, ydt, stream)

@pytest.mark.parametrize("fn", ["qlin_gemm_w4a4", "qlin_gemm_w8a8", "qlin_gemm_w4a8"])
@pytest.mark.parametrize("kw,status", [
    (dict(xq=None), q.QLIN_ERR_NULL), (dict(wq=None), q.QLIN_ERR_NULL), (dict(y=None), q.QLIN_ERR_NULL),
    (dict(sx=None), q.QLIN_ERR_NULL), (dict(sw=None), q.QLIN_ERR_NULL),
    (dict(ydt=9), q.QLIN_ERR_DTYPE),
    (dict(k=96), q.QLIN_ERR_SHAPE), (dict(k=32), q.QLIN_ERR_SHAPE), (dict(n=0), q.QLIN_ERR_SHAPE),
    (dict(m=-2), q.QLIN_ERR_SHAPE), (dict(k=131072 + 64), q.QLIN_ERR_SHAPE), (dict(k=131072), q.QLIN_ERR_SHAPE),
    (dict(xq=BAD), q.QLIN_ERR_ALIGN), (dict(y=BAD), q.QLIN_ERR_ALIGN), (dict(sw=BAD), q.QLIN_ERR_ALIGN),
    (dict(y=P + 64), q.QLIN_ERR_ALIAS),
])
def test_gemm_rejects(lib, fn, kw, status):
    args = dict(xq=P, sx=P3, wq=P2, sw=P4, m=16, n=64, k=512, y=0x70000000, ydt=1)
    args.update(kw)
    f = getattr(lib, fn)
    assert f(args["xq"], args["sx"], args["wq"], args["sw"], args["m"], args["n"], args["k"], args["y"],
             args["ydt"], None) == status


@pytest.mark.parametrize("fn,k,status", [("qlin_gemm_w8a8", 192, q.QLIN_OK), ("qlin_gemm_w4a8", 192, q.QLIN_ERR_SHAPE),
                                         ("qlin_gemm_w4a4", 192, q.QLIN_OK), ("qlin_gemm_w4a4", 160, q.QLIN_ERR_SHAPE),
                                         ("qlin_gemm_w8a8", 160, q.QLIN_ERR_SHAPE), ("qlin_gemm_w4a8", 256, q.QLIN_OK)])
def test_gemm_k_step_per_scheme(lib, fn, k, status):
    # W8A8 and W4A4 take k in multiples of 64, W4A8 in multiples of 128 (m = 0: no device call)
    assert getattr(lib, fn)(None, None, P2, P4, 0, 64, k, 0x70000000, 1, None) == status


def test_gemm_raw_i32_needs_no_scales_and_empty_ok(lib):
    # no scales with I32 output passes validation; m == 0 then returns before any HIP call
    assert lib.qlin_gemm_w8a8(None, None, P2, None, 0, 64, 512, 0x70000000, 3, None) == q.QLIN_OK


# ---- qlin_gemm_ws(scheme, xq, sx, wq, sw, m, n, k, y, ydt, ws, ws_bytes, stream)

DOWN = dict(m=816, n=2048, k=16384)   # the FFN-down shape at 816 tokens: 112 tiles, k split in two


def test_gemm_workspace_bytes(lib):
    # 2 splits x 816 x 2048 int32 partials (planned for 256 CUs: the default without a device)
    if not torch.cuda.is_available():
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 816, 2048, 16384) == 2 * 816 * 2048 * 4
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 52224, 2048, 16384) == 0    # large grid: no split
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4, 50, 1024, 4096) == 0        # small-M kernel: no split
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4, 816, 2048, 160) == -1       # k step is 64
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4, 816, 2048, 192) >= 0
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A8, 816, 2048, 192) == -1       # W4A8 k step is 128
    assert lib.qlin_gemm_workspace_bytes(4, 816, 2048, 16384) == -1               # no such scheme
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4_E2M3, 816, 2048, 16384) == 0  # E2M3 never splits
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4_E2M3, 816, 2048, 192) == -1
    assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 0, 2048, 16384) == 0
    if not torch.cuda.is_available():   # plans for 256 CUs
        # the 7B decoder's 4096-row weights at 256 tokens: 64 x 64 tiles, no split ...
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 256, 4096, 4096) == 0
        # ... but with k past 128 stages the workspace call keeps split-K (four splits)
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 256, 4096, 11008) == 4 * 256 * 4096 * 4
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4, 816, 2048, 16448) >= 0   # W4A4 at k % 128 == 64
        # short k (at most 64 stages): up to two rounds of 64 x 64 tiles take the
        # place of split-K (o at 816 tokens: 416 tiles)
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 816, 2048, 2048) == 0
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 1000, 1800, 4096) == 0
        # one stage more: two K splits, one block per CU
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W8A8, 1000, 1800, 4160) == 2 * 1000 * 1800 * 4
        # W4A4 keeps 128 x 256 tiles when they fill the CUs with their splits
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4, 1024, 4096, 8192) == 4 * 1024 * 4096 * 4


def gemm_ws(lib, scheme=q.QLIN_W8A8, xq=P, sx=P3, wq=P2, sw=P4, m=DOWN["m"], n=DOWN["n"], k=DOWN["k"],
            y=0x70000000, ydt=1, ws=0x7C000000, wsb=64 << 20):
    return lib.qlin_gemm_ws(scheme, xq, sx, wq, sw, m, n, k, y, ydt, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(scheme=4), q.QLIN_ERR_UNSUPPORTED), (dict(scheme=-1), q.QLIN_ERR_UNSUPPORTED),
    (dict(ws=None), q.QLIN_ERR_NULL),                      # bytes > 0 with no buffer
    (dict(wsb=-16), q.QLIN_ERR_SHAPE), (dict(ws=0x7C000008), q.QLIN_ERR_ALIGN),
    (dict(wsb=1024), q.QLIN_ERR_WORKSPACE),                # smaller than the split plan needs
    (dict(ws=0x70000000 + 4096), q.QLIN_ERR_ALIAS),         # workspace overlaps y
    (dict(ws=P2 + 64), q.QLIN_ERR_ALIAS),                   # workspace overlaps the weights
    (dict(k=100), q.QLIN_ERR_SHAPE), (dict(xq=None), q.QLIN_ERR_NULL), (dict(ydt=7), q.QLIN_ERR_DTYPE),
])
def test_gemm_ws_rejects(lib, kw, status):
    assert gemm_ws(lib, **kw) == status


def test_gemm_ws_empty_and_no_workspace_ok(lib):
    assert gemm_ws(lib, m=0) == q.QLIN_OK
    assert gemm_ws(lib, m=0, ws=None, wsb=0) == q.QLIN_OK
    assert gemm_ws(lib, m=0, wsb=16) == q.QLIN_OK            # no split needed for an empty call


# ---- qlin_gemm_static_ws(scheme, xq, sx, wq, sw, m, n, k, y, ydt, stream)

def test_gemm_static_ws_rejects(lib):
    def call(scheme=q.QLIN_W8A8, m=DOWN["m"], n=DOWN["n"], k=DOWN["k"], xq=P, y=0x70000000):
        return lib.qlin_gemm_static_ws(scheme, xq, P3, P2, P4, m, n, k, y, 1, None)
    assert call(scheme=5) == q.QLIN_ERR_UNSUPPORTED
    assert call(k=100) == q.QLIN_ERR_SHAPE
    assert call(xq=None) == q.QLIN_ERR_NULL
    assert call(y=P + 64) == q.QLIN_ERR_ALIAS
    # 1024 x 4096 x 8192 W4A4: four splits of 128 x 256 tiles need 64 MiB > the 16 MiB scratch
    if not torch.cuda.is_available():
        assert lib.qlin_gemm_workspace_bytes(q.QLIN_W4A4, 1024, 4096, 8192) == 4 * 1024 * 4096 * 4
    assert call(scheme=q.QLIN_W4A4, m=1024, n=4096, k=8192, y=0x78000000) == q.QLIN_ERR_WORKSPACE
    assert call(m=0) == q.QLIN_OK


# ---- qlin_gemm_w4a4_geglu(xq, sx, wq, sw, m, n2, k, h, hdt, stream)

@pytest.mark.parametrize("kw,status", [
    (dict(xq=None), q.QLIN_ERR_NULL), (dict(wq=None), q.QLIN_ERR_NULL), (dict(h=None), q.QLIN_ERR_NULL),
    (dict(sx=None), q.QLIN_ERR_NULL), (dict(sw=None), q.QLIN_ERR_NULL),
    (dict(hdt=3), q.QLIN_ERR_DTYPE), (dict(hdt=9), q.QLIN_ERR_DTYPE),
    (dict(n2=96), q.QLIN_ERR_SHAPE), (dict(n2=32), q.QLIN_ERR_SHAPE), (dict(k=160), q.QLIN_ERR_SHAPE),
    (dict(k=32), q.QLIN_ERR_SHAPE), (dict(m=-1), q.QLIN_ERR_SHAPE), (dict(k=131072 + 128), q.QLIN_ERR_SHAPE), (dict(k=131072), q.QLIN_ERR_SHAPE),
    (dict(xq=BAD), q.QLIN_ERR_ALIGN), (dict(h=BAD), q.QLIN_ERR_ALIGN),
    (dict(h=P + 64), q.QLIN_ERR_ALIAS),
])
def test_gemm_geglu_rejects(lib, kw, status):
    a = dict(xq=P, sx=P3, wq=P2, sw=P4, m=16, n2=128, k=512, h=0x70000000, hdt=1)
    a.update(kw)
    assert lib.qlin_gemm_w4a4_geglu(a["xq"], a["sx"], a["wq"], a["sw"], a["m"], a["n2"], a["k"], a["h"],
                                    a["hdt"], None) == status


def test_gemm_geglu_empty_is_ok(lib):
    assert lib.qlin_gemm_w4a4_geglu(None, None, P2, P4, 0, 128, 512, 0x70000000, 1, None) == q.QLIN_OK


# ---- E2M3 storage of int4-grid codes (bits QLIN_BITS_E2M3, scheme QLIN_W4A4_E2M3)

def test_e2m3_quantizers_take_k_in_multiples_of_128(lib):
    e = q.QLIN_BITS_E2M3
    # k = 576: a multiple of 8 and of the Hadamard block, not of 128
    assert rqa(lib, bits=e, m=0, k=576, ldx=576) == q.QLIN_ERR_SHAPE
    assert rqa(lib, bits=e, m=0) == q.QLIN_OK
    assert qw(lib, bits=e, k=576) == q.QLIN_ERR_SHAPE
    assert qw(lib, bits=e, group=128, b=0) == q.QLIN_ERR_UNSUPPORTED
    assert lib.qlin_rotate_quant_act_static(None, 0, 0, 576, 576, None, 64, e, P3, None, None) == q.QLIN_ERR_SHAPE
    assert lib.qlin_rotate_quant_act_static(None, 0, 0, 512, 512, None, 64, e, P3, None, None) == q.QLIN_OK
    assert lib.qlin_rotate_quant_act_composite(None, 0, 0, 576, 576, None, P3, P4, 64, e, None, None, None,
                                               None) == q.QLIN_ERR_SHAPE
    assert lib.qlin_rotate_quant_act_composite(None, 0, 0, 512, 512, None, P3, P4, 64, e, None, None, None,
                                               None) == q.QLIN_OK


def test_e2m3_code_bytes_in_alias_checks(lib):
    # m = 4 rows of k = 512 codes: 4 x 384 bytes in E2M3 (4 x 256 as packed int4)
    e = q.QLIN_BITS_E2M3
    assert rqa(lib, bits=e, xq=P2, xs=P2 + 4 * 384 - 16) == q.QLIN_ERR_ALIAS
    assert rqa(lib, bits=4, xq=P2, xs=P2 + 4 * 384 - 16) != q.QLIN_ERR_ALIAS
    # weights: 8 rows x 384 bytes
    assert qw(lib, bits=e, wq=P2, ws=P2 + 8 * 384 - 16) == q.QLIN_ERR_ALIAS


def test_gemm_e2m3_validation(lib):
    e = q.QLIN_W4A4_E2M3
    assert gemm_ws(lib, scheme=e, k=192, ws=None, wsb=0) == q.QLIN_ERR_SHAPE
    assert gemm_ws(lib, scheme=e, m=0, ws=None, wsb=0) == q.QLIN_OK
    # y overlapping the last bytes of xq (m rows of 3k/4 bytes) is an alias; just past them it is not
    m, k = 16, 512
    assert gemm_ws(lib, scheme=e, m=m, k=k, y=P + m * k * 3 // 4 - 16, ws=None, wsb=0) == q.QLIN_ERR_ALIAS
    assert gemm_ws(lib, scheme=e, m=m, k=k, y=P + m * k * 3 // 4, ws=None, wsb=0) != q.QLIN_ERR_ALIAS
    assert lib.qlin_gemm_static_ws(e, P, P3, P2, P4, 0, 2048, 16384, 0x70000000, 1, None) == q.QLIN_OK


@pytest.mark.parametrize("scheme,status", [(q.QLIN_W4A4, q.QLIN_OK), (q.QLIN_W4A4_E2M3, q.QLIN_OK),
                                           (q.QLIN_W8A8, q.QLIN_ERR_UNSUPPORTED), (7, q.QLIN_ERR_UNSUPPORTED)])
def test_gemm_geglu_schemes(lib, scheme, status):
    assert lib.qlin_gemm_geglu(scheme, None, None, P2, P4, 0, 128, 512, 0x70000000, 1, None) == status


def test_gemm_geglu_e2m3_shapes(lib):
    e = q.QLIN_W4A4_E2M3
    assert lib.qlin_gemm_geglu(e, P, P3, P2, P4, 16, 96, 512, 0x70000000, 1, None) == q.QLIN_ERR_SHAPE
    assert lib.qlin_gemm_geglu(e, P, P3, P2, P4, 16, 128, 192, 0x70000000, 1, None) == q.QLIN_ERR_SHAPE
    # h overlapping the E2M3 weights (128 rows x 384 bytes)
    assert lib.qlin_gemm_geglu(e, P, P3, P2, P4, 16, 128, 512, P2 + 128 * 384 - 16, 1, None) == q.QLIN_ERR_ALIAS


# ---- qlin_gemv_w4a16(x, wq, ws, m, n, k, group, y, stream)

@pytest.mark.parametrize("kw,status", [
    (dict(x=None), q.QLIN_ERR_NULL), (dict(wq=None), q.QLIN_ERR_NULL), (dict(y=None), q.QLIN_ERR_NULL),
    (dict(group=64), q.QLIN_ERR_UNSUPPORTED), (dict(m=65), q.QLIN_ERR_SHAPE), (dict(k=200), q.QLIN_ERR_SHAPE),
    (dict(n=0), q.QLIN_ERR_SHAPE), (dict(k=32768 + 128), q.QLIN_ERR_SHAPE), (dict(x=BAD), q.QLIN_ERR_ALIGN),
    (dict(y=P2 + 16), q.QLIN_ERR_ALIAS),
])
def test_gemv_rejects(lib, kw, status):
    a = dict(x=P, wq=P2, ws=P3, m=1, n=256, k=4096, group=128, y=P4)
    a.update(kw)
    assert lib.qlin_gemv_w4a16(a["x"], a["wq"], a["ws"], a["m"], a["n"], a["k"], a["group"], a["y"],
                               None) == status


# ---- qlin_calibrate_fold(x, xdt, m, k, ldx, pre, w, wdt, n, s, inv_s, stream)

@pytest.mark.parametrize("kw,status", [
    (dict(x=None), q.QLIN_ERR_NULL), (dict(s=None), q.QLIN_ERR_NULL), (dict(xdt=3), q.QLIN_ERR_DTYPE),
    (dict(pre=5), q.QLIN_ERR_UNSUPPORTED), (dict(m=0), q.QLIN_ERR_SHAPE), (dict(k=12, ldx=16), q.QLIN_ERR_SHAPE),
    (dict(pre=1), q.QLIN_ERR_SHAPE), (dict(inv=BAD), q.QLIN_ERR_ALIGN), (dict(inv=P3 + 32), q.QLIN_ERR_ALIAS),
])
def test_calibrate_fold_rejects(lib, kw, status):
    a = dict(x=P, xdt=1, m=8, k=512, ldx=512, pre=0, w=P2, wdt=0, n=16, s=P3, inv=P4)
    a.update(kw)
    assert lib.qlin_calibrate_fold(a["x"], a["xdt"], a["m"], a["k"], a["ldx"], a["pre"], a["w"], a["wdt"],
                                   a["n"], a["s"], a["inv"], None) == status


# ---- per-step table entry points

# qlin_calibrate_step_scales(x, dt, m, k, ldx, inv_s, b, bits, table, stream)
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), q.QLIN_ERR_NULL), (dict(t=None), q.QLIN_ERR_NULL), (dict(dt=3), q.QLIN_ERR_DTYPE),
    (dict(bits=5), q.QLIN_ERR_UNSUPPORTED), (dict(b=96), q.QLIN_ERR_UNSUPPORTED),
    (dict(m=0), q.QLIN_ERR_SHAPE), (dict(k=500, ldx=504), q.QLIN_ERR_SHAPE), (dict(ldx=256), q.QLIN_ERR_SHAPE),
    (dict(k=65536, ldx=65536, b=0), q.QLIN_ERR_SHAPE), (dict(t=BAD), q.QLIN_ERR_ALIGN),
    (dict(inv=BAD), q.QLIN_ERR_ALIGN), (dict(t=P + 64), q.QLIN_ERR_ALIAS),
])
def test_calibrate_step_scales_rejects(lib, kw, status):
    a = dict(x=P, dt=0, m=8, k=512, ldx=512, inv=P4, b=64, bits=4, t=P3)
    a.update(kw)
    assert lib.qlin_calibrate_step_scales(a["x"], a["dt"], a["m"], a["k"], a["ldx"], a["inv"], a["b"], a["bits"],
                                          a["t"], None) == status


# qlin_rotate_quant_act_static(x, dt, m, k, ldx, inv_s, b, bits, table, xq, stream)
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), q.QLIN_ERR_NULL), (dict(t=None), q.QLIN_ERR_NULL), (dict(xq=None), q.QLIN_ERR_NULL),
    (dict(dt=3), q.QLIN_ERR_DTYPE), (dict(bits=2), q.QLIN_ERR_UNSUPPORTED), (dict(b=3), q.QLIN_ERR_UNSUPPORTED),
    (dict(m=-1), q.QLIN_ERR_SHAPE), (dict(k=520, ldx=520), q.QLIN_ERR_SHAPE), (dict(ldx=513), q.QLIN_ERR_SHAPE),
    (dict(xq=BAD), q.QLIN_ERR_ALIGN), (dict(t=BAD), q.QLIN_ERR_ALIGN),
    (dict(xq=P + 128), q.QLIN_ERR_ALIAS), (dict(xq=P3), q.QLIN_ERR_ALIAS),
])
def test_rotate_quant_act_static_rejects(lib, kw, status):
    a = dict(x=P, dt=1, m=4, k=512, ldx=512, inv=None, b=64, bits=4, t=P3, xq=P2)
    a.update(kw)
    assert lib.qlin_rotate_quant_act_static(a["x"], a["dt"], a["m"], a["k"], a["ldx"], a["inv"], a["b"], a["bits"],
                                            a["t"], a["xq"], None) == status


def test_rotate_quant_act_static_empty_is_ok(lib):
    assert lib.qlin_rotate_quant_act_static(None, 0, 0, 512, 512, None, 64, 4, P3, None, None) == q.QLIN_OK


# qlin_quantize_weights_step(w, dt, n, k, fold_s, b, bits, table, wq, ws, stream)
@pytest.mark.parametrize("kw,status", [
    (dict(w=None), q.QLIN_ERR_NULL), (dict(t=None), q.QLIN_ERR_NULL), (dict(wq=None), q.QLIN_ERR_NULL),
    (dict(ws=None), q.QLIN_ERR_NULL), (dict(dt=4), q.QLIN_ERR_DTYPE), (dict(bits=16), q.QLIN_ERR_UNSUPPORTED),
    (dict(n=0), q.QLIN_ERR_SHAPE), (dict(k=544), q.QLIN_ERR_SHAPE), (dict(ws=BAD), q.QLIN_ERR_ALIGN),
    (dict(s=BAD), q.QLIN_ERR_ALIGN), (dict(wq=P + 1024), q.QLIN_ERR_ALIAS), (dict(ws=P3 + 16), q.QLIN_ERR_ALIAS),
])
def test_quantize_weights_step_rejects(lib, kw, status):
    a = dict(w=P, dt=0, n=8, k=512, s=None, b=64, bits=4, t=P3, wq=P2, ws=P4)
    a.update(kw)
    assert lib.qlin_quantize_weights_step(a["w"], a["dt"], a["n"], a["k"], a["s"], a["b"], a["bits"], a["t"],
                                          a["wq"], a["ws"], None) == status


# ---- composite rotation entry points

# qlin_calibrate_composite(w, dt, n, k, fold_s, b, perm, rot, work, work_bytes, stream)
@pytest.mark.parametrize("kw,status", [
    (dict(w=None), q.QLIN_ERR_NULL), (dict(perm=None), q.QLIN_ERR_NULL), (dict(rot=None), q.QLIN_ERR_NULL),
    (dict(work=None), q.QLIN_ERR_NULL), (dict(work=BAD), q.QLIN_ERR_ALIGN), (dict(wb=64), q.QLIN_ERR_WORKSPACE),
    (dict(work=P + 256), q.QLIN_ERR_ALIAS),
    (dict(dt=3), q.QLIN_ERR_DTYPE), (dict(b=8), q.QLIN_ERR_UNSUPPORTED), (dict(b=256), q.QLIN_ERR_UNSUPPORTED),
    (dict(b=48), q.QLIN_ERR_UNSUPPORTED), (dict(n=0), q.QLIN_ERR_SHAPE), (dict(k=520), q.QLIN_ERR_SHAPE),
    (dict(k=65536), q.QLIN_ERR_SHAPE), (dict(rot=BAD), q.QLIN_ERR_ALIGN), (dict(s=BAD), q.QLIN_ERR_ALIGN),
    (dict(perm=P + 64), q.QLIN_ERR_ALIAS), (dict(rot=P3 + 512), q.QLIN_ERR_ALIAS),
])
def test_calibrate_composite_rejects(lib, kw, status):
    a = dict(w=P, dt=0, n=16, k=512, s=None, b=64, perm=P3, rot=P4, work=0x50000000, wb=1 << 20)
    a.update(kw)
    assert lib.qlin_calibrate_composite(a["w"], a["dt"], a["n"], a["k"], a["s"], a["b"], a["perm"], a["rot"],
                                        a["work"], a["wb"], None) == status


def test_calibrate_composite_work_bytes(lib):
    nb = lib.qlin_calibrate_composite_work_bytes(16, 512, 64)
    assert 8 * 512 * 64 <= nb <= 1 << 20
    assert lib.qlin_calibrate_composite_work_bytes(16, 512, 48) == -1
    assert lib.qlin_calibrate_composite_work_bytes(0, 512, 64) == -1
    assert lib.qlin_calibrate_composite_work_bytes(16, 520, 64) == -1


# qlin_rotate_quant_act_composite(x, dt, m, k, ldx, inv_s, perm, rot, b, bits, xq, xs, work, stream)
@pytest.mark.parametrize("kw,status", [
    (dict(work=None), q.QLIN_ERR_NULL),
    (dict(work=BAD), q.QLIN_ERR_ALIGN), (dict(work=P2 + 512), q.QLIN_ERR_ALIAS), (dict(work=P + 1024), q.QLIN_ERR_ALIAS),
    (dict(x=None), q.QLIN_ERR_NULL), (dict(perm=None), q.QLIN_ERR_NULL), (dict(xq=None), q.QLIN_ERR_NULL),
    (dict(xs=None), q.QLIN_ERR_NULL), (dict(dt=5), q.QLIN_ERR_DTYPE), (dict(b=4), q.QLIN_ERR_UNSUPPORTED),
    (dict(bits=2), q.QLIN_ERR_UNSUPPORTED), (dict(m=-1), q.QLIN_ERR_SHAPE), (dict(ldx=256), q.QLIN_ERR_SHAPE),
    (dict(k=65536, ldx=65536, b=128), q.QLIN_ERR_SHAPE), (dict(xq=BAD), q.QLIN_ERR_ALIGN),
    (dict(perm=BAD), q.QLIN_ERR_ALIGN), (dict(xq=P + 32), q.QLIN_ERR_ALIAS), (dict(xs=P4 + 16), q.QLIN_ERR_ALIAS),
])
def test_rotate_quant_act_composite_rejects(lib, kw, status):
    a = dict(x=P, dt=1, m=4, k=512, ldx=512, inv=None, perm=P3, rot=P4, b=64, bits=4, xq=P2, xs=0x70000000,
             work=0x50000000)
    a.update(kw)
    assert lib.qlin_rotate_quant_act_composite(a["x"], a["dt"], a["m"], a["k"], a["ldx"], a["inv"], a["perm"],
                                               a["rot"], a["b"], a["bits"], a["xq"], a["xs"], a["work"],
                                               None) == status


def test_rotate_quant_act_composite_empty_is_ok(lib):
    assert lib.qlin_rotate_quant_act_composite(None, 0, 0, 512, 512, None, P3, P4, 64, 4, None, None, None,
                                               None) == q.QLIN_OK


# qlin_quantize_weights_composite(w, dt, n, k, fold_s, perm, rot, b, bits, wq, ws, work, stream)
@pytest.mark.parametrize("kw,status", [
    (dict(w=None), q.QLIN_ERR_NULL), (dict(rot=None), q.QLIN_ERR_NULL), (dict(ws=None), q.QLIN_ERR_NULL),
    (dict(work=None), q.QLIN_ERR_NULL), (dict(work=BAD), q.QLIN_ERR_ALIGN), (dict(work=0x70000000), q.QLIN_ERR_ALIAS),
    (dict(b=512), q.QLIN_ERR_UNSUPPORTED), (dict(bits=3), q.QLIN_ERR_UNSUPPORTED), (dict(n=0), q.QLIN_ERR_SHAPE),
    (dict(k=96), q.QLIN_ERR_SHAPE), (dict(wq=BAD), q.QLIN_ERR_ALIGN), (dict(wq=P + 128), q.QLIN_ERR_ALIAS),
])
def test_quantize_weights_composite_rejects(lib, kw, status):
    a = dict(w=P, dt=0, n=8, k=512, s=None, perm=P3, rot=P4, b=64, bits=4, wq=P2, ws=0x70000000, work=0x50000000)
    a.update(kw)
    assert lib.qlin_quantize_weights_composite(a["w"], a["dt"], a["n"], a["k"], a["s"], a["perm"], a["rot"],
                                               a["b"], a["bits"], a["wq"], a["ws"], a["work"], None) == status


def test_binding_raises_qlin_error(lib):
    err = q.QlinError(q.QLIN_ERR_SHAPE, "where")
    assert "invalid shape" in str(err) and err.status == q.QLIN_ERR_SHAPE


@pytest.mark.skipif(torch.cuda.is_available(), reason="only meaningful where no GPU is visible")
def test_valid_call_without_device_reports_device_error(lib):
    # arguments pass validation; the device check then fails cleanly (no GPU here)
    assert rqa(lib) == q.QLIN_ERR_DEVICE


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), q.QLIN_ERR_NULL), (dict(sink=None), q.QLIN_ERR_NULL),
    (dict(nbytes=0), q.QLIN_ERR_SHAPE), (dict(nbytes=4100), q.QLIN_ERR_SHAPE), (dict(nbytes=-16), q.QLIN_ERR_SHAPE),
    (dict(src=BAD), q.QLIN_ERR_ALIGN), (dict(sink=BAD), q.QLIN_ERR_ALIGN),
    (dict(sink=P + 1024), q.QLIN_ERR_ALIAS),
])
def test_stream_read_rejects(lib, kw, status):
    a = dict(src=P, nbytes=4096, sink=P2)
    a.update(kw)
    assert lib.qlin_stream_read(a["src"], a["nbytes"], a["sink"], None) == status

