"""Python binding of the qlin C ABI (libqlin.so, HIP kernels for gfx950).

Argument marshalling only: device tensors are passed as raw pointers together
with torch's current HIP stream, output tensors are allocated with torch, and
every computation runs in the library's kernels.  The function names mirror
the C entry points declared in include/qlin.h; a non-zero status raises
QlinError.  Importing works without a GPU; calling a compute entry point
without the built library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QLIN_LIB_PATH selects another build of the library with the same entry
# points (the host-only sanitizer build of the argument validation is tested
# this way); by default the in-tree libqlin.so.
LIB_PATH = os.environ.get("QLIN_LIB_PATH") or os.path.join(_HERE, "libqlin.so")

QLIN_OK = 0
QLIN_ERR_NULL = 1
QLIN_ERR_SHAPE = 2
QLIN_ERR_DTYPE = 3
QLIN_ERR_ALIGN = 4
QLIN_ERR_UNSUPPORTED = 5
QLIN_ERR_DEVICE = 6
QLIN_ERR_LAUNCH = 7
QLIN_ERR_ALIAS = 8
QLIN_ERR_CAPTURE = 9
QLIN_ERR_WORKSPACE = 10

QLIN_F16, QLIN_BF16, QLIN_F32, QLIN_I32 = 0, 1, 2, 3
QLIN_PRE_NONE, QLIN_PRE_GEGLU = 0, 1
QLIN_W4A4, QLIN_W8A8, QLIN_W4A8, QLIN_W4A4_E2M3 = 0, 1, 2, 3
QLIN_BITS_E2M3 = 6
_SCHEME = {"qlin_gemm_w4a4": QLIN_W4A4, "qlin_gemm_w8a8": QLIN_W8A8, "qlin_gemm_w4a8": QLIN_W4A8}

_TORCH_TO_QLIN = {torch.float16: QLIN_F16, torch.bfloat16: QLIN_BF16,
                  torch.float32: QLIN_F32, torch.int32: QLIN_I32}

# (name, argtypes) of every exported entry point; restype is int32 unless noted.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
SIGNATURES = {
    "qlin_abi_version": [],
    "qlin_status_string": [_I32],
    "qlin_calibrate_fold": [_P, _I32, _I64, _I64, _I64, _I32, _P, _I32, _I64, _P, _P, _P],
    "qlin_quantize_weights": [_P, _I32, _I64, _I64, _P, _I32, _I32, _I32, _P, _P, _P],
    "qlin_rotate_quant_act": [_P, _I32, _I64, _I64, _I64, _I32, _P, _I32, _I32, _P, _P, _P],
    "qlin_gemm_w4a4": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P],
    "qlin_gemm_w8a8": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P],
    "qlin_gemm_w4a8": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P],
    "qlin_gemm_ws": [_I32, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P, _I64, _P],
    "qlin_gemm_workspace_bytes": [_I32, _I64, _I64, _I64],
    "qlin_gemm_static_ws": [_I32, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P],
    "qlin_gemm_w4a4_geglu": [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P],
    "qlin_gemm_geglu": [_I32, _P, _P, _P, _P, _I64, _I64, _I64, _P, _I32, _P],
    "qlin_gemv_w4a16": [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _P],
    "qlin_stream_read": [_P, _I64, _P, _P],
    "qlin_calibrate_step_scales": [_P, _I32, _I64, _I64, _I64, _P, _I32, _I32, _P, _P],
    "qlin_rotate_quant_act_static": [_P, _I32, _I64, _I64, _I64, _P, _I32, _I32, _P, _P, _P],
    "qlin_quantize_weights_step": [_P, _I32, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _P],
    "qlin_calibrate_composite_work_bytes": [_I64, _I64, _I32],
    "qlin_calibrate_composite": [_P, _I32, _I64, _I64, _P, _I32, _P, _P, _P, _I64, _P],
    "qlin_rotate_quant_act_composite": [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _I32, _I32, _P, _P, _P, _P],
    "qlin_quantize_weights_composite": [_P, _I32, _I64, _I64, _P, _P, _P, _I32, _I32, _P, _P, _P, _P],
}

_lib = None


class QlinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Loads libqlin.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_ptq_vla_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = (ctypes.c_char_p if name == "qlin_status_string"
                      else ctypes.c_int64 if name.endswith("_bytes") else ctypes.c_int32)
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().qlin_status_string(status).decode()


def abi_version() -> int:
    return load().qlin_abi_version()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int, where: str) -> None:
    if status != QLIN_OK:
        raise QlinError(status, where)


def _dev_tensor(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _need(t, nbytes: int, name: str) -> None:
    """A buffer handed to the library: a contiguous device tensor of at least
    nbytes (the library sees only its pointer)."""
    if t is None:
        return
    _dev_tensor(t, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the call needs {nbytes}")


def code_row_bytes(k: int, bits: int) -> int:
    """Bytes of one row of k codes: int8 (bits 8), packed int4 (bits 4) or
    int4-grid codes in E2M3 storage (bits 6, three bytes per four codes)."""
    return {8: k, 4: k // 2, QLIN_BITS_E2M3: k // 4 * 3}[bits]


def _codes(rows: int, k: int, bits: int, device) -> torch.Tensor:
    """An uninitialised code tensor: int8 [rows][k], or uint8 [rows][row bytes]."""
    return torch.empty((rows, code_row_bytes(k, bits)), dtype=torch.int8 if bits == 8 else torch.uint8,
                       device=device)


def _operand_bytes(scheme: int, k: int) -> Tuple[int, int]:
    """Row bytes of the activation and weight codes of a GEMM scheme."""
    return {QLIN_W4A4: (k // 2, k // 2), QLIN_W8A8: (k, k), QLIN_W4A8: (k, k // 2),
            QLIN_W4A4_E2M3: (k // 4 * 3, k // 4 * 3)}[scheme]


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------


def qlin_calibrate_fold(x: torch.Tensor, w: torch.Tensor, pre: int = QLIN_PRE_NONE
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fold vector s[k] and 1/s[k] from activations x [m][k] (or [m][2k] =
    gate|up with pre=GEGLU) and weights w [n][k]."""
    lib = load()
    _dev_tensor(x, "x"); _dev_tensor(w, "w")
    n, k = w.shape
    s = torch.empty(k, dtype=torch.float32, device=x.device)
    inv_s = torch.empty_like(s)
    st = lib.qlin_calibrate_fold(x.data_ptr(), _TORCH_TO_QLIN[x.dtype], x.shape[0], k, x.stride(0), pre,
                                 w.data_ptr(), _TORCH_TO_QLIN[w.dtype], n, s.data_ptr(), inv_s.data_ptr(),
                                 _stream(x.device))
    _check(st, "qlin_calibrate_fold")
    return s, inv_s


def qlin_quantize_weights(w: torch.Tensor, fold_s: Optional[torch.Tensor] = None, had_block: int = 0,
                          bits: int = 4, group: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Codes (int8 [n][k], packed uint8 [n][k/2], or E2M3 uint8 [n][3k/4] for
    bits 6) and scales (float32 [n], or fp16 [n][k/group] for group
    quantization) of weights w [n][k]."""
    lib = load()
    _dev_tensor(w, "w")
    n, k = w.shape
    wq = _codes(n, k, bits, w.device)
    ws = (torch.empty((n, k // group), dtype=torch.float16, device=w.device) if group
          else torch.empty(n, dtype=torch.float32, device=w.device))
    st = lib.qlin_quantize_weights(w.data_ptr(), _TORCH_TO_QLIN[w.dtype], n, k, _ptr(fold_s), had_block,
                                   bits, group, wq.data_ptr(), ws.data_ptr(), _stream(w.device))
    _check(st, "qlin_quantize_weights")
    return wq, ws


def qlin_rotate_quant_act(x: torch.Tensor, k: Optional[int] = None, fold_inv_s: Optional[torch.Tensor] = None,
                          had_block: int = 0, bits: int = 4, pre: int = QLIN_PRE_NONE,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Activation codes and per-token scales of x [m][ldx] (k inputs, or
    gate|up of width 2k with pre=GEGLU)."""
    lib = load()
    _dev_tensor(x, "x")
    m = x.shape[0]
    if k is None:
        k = x.shape[1] // 2 if pre == QLIN_PRE_GEGLU else x.shape[1]
    if x.dim() != 2 or x.stride(1) != 1 or (2 * k if pre == QLIN_PRE_GEGLU else k) > x.shape[1]:
        raise ValueError("x must be a row-major [m][>= k] tensor ([m][>= 2k] with the GeGLU pre-op)")
    if out is None:
        xq = _codes(m, k, bits, x.device)
        xs = torch.empty(m, dtype=torch.float32, device=x.device)
    else:
        xq, xs = out
    _need(xq, m * code_row_bytes(k, bits), "xq")
    _need(xs, m * 4, "x_scale")
    st = lib.qlin_rotate_quant_act(x.data_ptr(), _TORCH_TO_QLIN[x.dtype], m, k, x.stride(0), pre,
                                   _ptr(fold_inv_s), had_block, bits, xq.data_ptr(), xs.data_ptr(),
                                   _stream(x.device))
    _check(st, "qlin_rotate_quant_act")
    return xq, xs


def _rows_arg(x: torch.Tensor, k: Optional[int]) -> int:
    _dev_tensor(x, "x")
    if k is None:
        k = x.shape[1]
    if x.dim() != 2 or x.stride(1) != 1 or k > x.shape[1]:
        raise ValueError("x must be a row-major [m][>= k] tensor")
    return k


def qlin_calibrate_step_scales(x: torch.Tensor, k: Optional[int] = None,
                               fold_inv_s: Optional[torch.Tensor] = None, had_block: int = 0,
                               bits: int = 4, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One row of the per-step static scale table (float32 [k]) from the
    calibration tokens x [m][ldx] of one denoising step."""
    lib = load()
    k = _rows_arg(x, k)
    table = out if out is not None else torch.empty(k, dtype=torch.float32, device=x.device)
    _need(table, k * 4, "table")
    _need(fold_inv_s, k * 4, "fold_inv_s")
    st = lib.qlin_calibrate_step_scales(x.data_ptr(), _TORCH_TO_QLIN[x.dtype], x.shape[0], k, x.stride(0),
                                        _ptr(fold_inv_s), had_block, bits, table.data_ptr(), _stream(x.device))
    _check(st, "qlin_calibrate_step_scales")
    return table


def qlin_rotate_quant_act_static(x: torch.Tensor, table: torch.Tensor, k: Optional[int] = None,
                                 fold_inv_s: Optional[torch.Tensor] = None, had_block: int = 0,
                                 bits: int = 4, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Activation codes of x [m][ldx] with one step's static per-channel
    scales (no per-row scale: the GEMM takes x_scale = 1)."""
    lib = load()
    k = _rows_arg(x, k)
    m = x.shape[0]
    xq = out if out is not None else _codes(m, k, bits, x.device)
    _need(xq, m * code_row_bytes(k, bits), "xq")
    _need(table, k * 4, "table")
    _need(fold_inv_s, k * 4, "fold_inv_s")
    st = lib.qlin_rotate_quant_act_static(x.data_ptr(), _TORCH_TO_QLIN[x.dtype], m, k, x.stride(0),
                                          _ptr(fold_inv_s), had_block, bits, table.data_ptr(), xq.data_ptr(),
                                          _stream(x.device))
    _check(st, "qlin_rotate_quant_act_static")
    return xq


def qlin_quantize_weights_step(w: torch.Tensor, table: torch.Tensor, fold_s: Optional[torch.Tensor] = None,
                               had_block: int = 0, bits: int = 4) -> Tuple[torch.Tensor, torch.Tensor]:
    """One step's weights w [n][k] with that step's table folded in: codes
    and float32 [n] scales."""
    lib = load()
    _dev_tensor(w, "w")
    n, k = w.shape
    _need(w, n * k * w.element_size(), "w")
    _need(table, k * 4, "table")
    _need(fold_s, k * 4, "fold_s")
    wq = _codes(n, k, bits, w.device)
    ws = torch.empty(n, dtype=torch.float32, device=w.device)
    st = lib.qlin_quantize_weights_step(w.data_ptr(), _TORCH_TO_QLIN[w.dtype], n, k, _ptr(fold_s), had_block,
                                        bits, table.data_ptr(), wq.data_ptr(), ws.data_ptr(), _stream(w.device))
    _check(st, "qlin_quantize_weights_step")
    return wq, ws


def qlin_calibrate_composite(w: torch.Tensor, had_block: int, fold_s: Optional[torch.Tensor] = None
                             ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Zigzag channel permutation (int32 [k]) and per-block composite
    rotations (float32 [k/b][b][b]) from the weights w [n][k] (times fold_s)."""
    lib = load()
    _dev_tensor(w, "w")
    n, k = w.shape
    _need(w, n * k * w.element_size(), "w")
    _need(fold_s, k * 4, "fold_s")
    perm = torch.empty(k, dtype=torch.int32, device=w.device)
    rot = torch.empty((k // had_block, had_block, had_block), dtype=torch.float32, device=w.device)
    nbytes = lib.qlin_calibrate_composite_work_bytes(n, k, had_block)
    if nbytes < 0:
        raise QlinError(QLIN_ERR_SHAPE, "qlin_calibrate_composite_work_bytes")
    work = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=w.device)
    st = lib.qlin_calibrate_composite(w.data_ptr(), _TORCH_TO_QLIN[w.dtype], n, k, _ptr(fold_s), had_block,
                                      perm.data_ptr(), rot.data_ptr(), work.data_ptr(), work.numel(),
                                      _stream(w.device))
    _check(st, "qlin_calibrate_composite")
    return perm, rot


def qlin_rotate_quant_act_composite(x: torch.Tensor, perm: torch.Tensor, rot: torch.Tensor,
                                    fold_inv_s: Optional[torch.Tensor] = None, bits: int = 4,
                                    k: Optional[int] = None,
                                    out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                                    work: Optional[torch.Tensor] = None
                                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Activation codes and per-token scales with the composite rotation
    (work: float32 scratch of m * k elements; allocated here when None)."""
    lib = load()
    k = _rows_arg(x, k)
    m, b = x.shape[0], rot.shape[-1]
    if out is None:
        xq = _codes(m, k, bits, x.device)
        xs = torch.empty(m, dtype=torch.float32, device=x.device)
    else:
        xq, xs = out
    _need(xq, m * code_row_bytes(k, bits), "xq")
    _need(xs, m * 4, "x_scale")
    _need(perm, k * 4, "perm")
    _need(rot, k * b * 4, "rot")
    _need(fold_inv_s, k * 4, "fold_inv_s")
    if work is None:
        work = torch.empty(max(m, 1) * k, dtype=torch.float32, device=x.device)
    _need(work, m * k * 4, "work")
    st = lib.qlin_rotate_quant_act_composite(x.data_ptr(), _TORCH_TO_QLIN[x.dtype], m, k, x.stride(0),
                                             _ptr(fold_inv_s), perm.data_ptr(), rot.data_ptr(), b, bits,
                                             xq.data_ptr(), xs.data_ptr(), work.data_ptr(), _stream(x.device))
    _check(st, "qlin_rotate_quant_act_composite")
    return xq, xs


def qlin_quantize_weights_composite(w: torch.Tensor, perm: torch.Tensor, rot: torch.Tensor,
                                    fold_s: Optional[torch.Tensor] = None, bits: int = 4,
                                    work: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Weight codes and per-row scales with the composite rotation (work:
    float32 scratch of n * k elements; allocated here when None)."""
    lib = load()
    _dev_tensor(w, "w")
    n, k = w.shape
    b = rot.shape[-1]
    _need(w, n * k * w.element_size(), "w")
    _need(perm, k * 4, "perm")
    _need(rot, k * b * 4, "rot")
    _need(fold_s, k * 4, "fold_s")
    wq = _codes(n, k, bits, w.device)
    ws = torch.empty(n, dtype=torch.float32, device=w.device)
    if work is None:
        work = torch.empty(n * k, dtype=torch.float32, device=w.device)
    _need(work, n * k * 4, "work")
    st = lib.qlin_quantize_weights_composite(w.data_ptr(), _TORCH_TO_QLIN[w.dtype], n, k, _ptr(fold_s),
                                             perm.data_ptr(), rot.data_ptr(), b, bits, wq.data_ptr(),
                                             ws.data_ptr(), work.data_ptr(), _stream(w.device))
    _check(st, "qlin_quantize_weights_composite")
    return wq, ws


def gemm_workspace_bytes(scheme: int, m: int, n: int, k: int) -> int:
    """Bytes of split-K workspace a qlin_gemm_ws call of this shape takes (0: none)."""
    nbytes = load().qlin_gemm_workspace_bytes(scheme, m, n, k)
    if nbytes < 0:
        raise QlinError(QLIN_ERR_SHAPE, "qlin_gemm_workspace_bytes")
    return nbytes


def gemm_workspace(scheme: int, m: int, n: int, k: int, device) -> Optional[torch.Tensor]:
    """A device buffer for qlin_gemm_ws's split-K partials (None when the
    shape takes no split)."""
    nbytes = gemm_workspace_bytes(scheme, m, n, k)
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def _gemm(fn_name: str, xq, x_scale, wq, w_scale, k: int, y_dtype, out, workspace=None):
    lib = load()
    _dev_tensor(wq, "wq")
    m, n = xq.shape[0], wq.shape[0]
    ka, kb = _operand_bytes(_SCHEME[fn_name], k)
    _need(xq, m * ka, "xq")
    _need(wq, n * kb, "wq")
    _need(x_scale, m * 4, "x_scale")
    _need(w_scale, n * 4, "w_scale")
    y = out if out is not None else torch.empty((m, n), dtype=y_dtype, device=wq.device)
    _need(y, m * n * y.element_size(), "y")
    if workspace is None:
        st = getattr(lib, fn_name)(xq.data_ptr(), _ptr(x_scale), wq.data_ptr(), _ptr(w_scale), m, n, k,
                                   y.data_ptr(), _TORCH_TO_QLIN[y.dtype], _stream(wq.device))
        _check(st, fn_name)
    else:
        _need(workspace, 0, "workspace")
        st = lib.qlin_gemm_ws(_SCHEME[fn_name], xq.data_ptr(), _ptr(x_scale), wq.data_ptr(), _ptr(w_scale), m, n, k,
                              y.data_ptr(), _TORCH_TO_QLIN[y.dtype], workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _stream(wq.device))
        _check(st, "qlin_gemm_ws")
    return y


QLIN_STATIC_SCRATCH_BYTES = 16 << 20


def qlin_gemm_static_ws(scheme: int, xq, x_scale, wq, w_scale, k: int, y_dtype=torch.bfloat16,
                        out=None) -> torch.Tensor:
    """The integer GEMM of `scheme` with split-K partials in the library's
    static device scratch (no workspace argument, nothing allocated by the
    library; calls overlapping on one GPU race)."""
    lib = load()
    _dev_tensor(wq, "wq")
    m, n = xq.shape[0], wq.shape[0]
    ka, kb = _operand_bytes(scheme, k)
    _need(xq, m * ka, "xq")
    _need(wq, n * kb, "wq")
    _need(x_scale, m * 4, "x_scale")
    _need(w_scale, n * 4, "w_scale")
    y = out if out is not None else torch.empty((m, n), dtype=y_dtype, device=wq.device)
    _need(y, m * n * y.element_size(), "y")
    st = lib.qlin_gemm_static_ws(scheme, xq.data_ptr(), _ptr(x_scale), wq.data_ptr(), _ptr(w_scale), m, n, k,
                                 y.data_ptr(), _TORCH_TO_QLIN[y.dtype], _stream(wq.device))
    _check(st, "qlin_gemm_static_ws")
    return y


def qlin_gemm_w4a4(xq, x_scale, wq, w_scale, k: int, y_dtype=torch.bfloat16, out=None,
                   workspace=None) -> torch.Tensor:
    """y [m][n] from packed int4 codes xq [m][k/2], wq [n][k/2] (workspace:
    split-K scratch from gemm_workspace, through qlin_gemm_ws)."""
    return _gemm("qlin_gemm_w4a4", xq, x_scale, wq, w_scale, k, y_dtype, out, workspace)


def qlin_gemm_w8a8(xq, x_scale, wq, w_scale, k: int, y_dtype=torch.bfloat16, out=None,
                   workspace=None) -> torch.Tensor:
    """y [m][n] from int8 codes xq [m][k], wq [n][k]."""
    return _gemm("qlin_gemm_w8a8", xq, x_scale, wq, w_scale, k, y_dtype, out, workspace)


def qlin_gemm_w4a8(xq, x_scale, wq, w_scale, k: int, y_dtype=torch.bfloat16, out=None,
                   workspace=None) -> torch.Tensor:
    """y [m][n] from int8 activation codes xq [m][k] and packed int4 weight codes wq [n][k/2]."""
    return _gemm("qlin_gemm_w4a8", xq, x_scale, wq, w_scale, k, y_dtype, out, workspace)


def qlin_gemm_e2m3(xq, x_scale, wq, w_scale, k: int, y_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """y [m][n] from int4-grid codes in E2M3 storage, xq [m][3k/4] and wq
    [n][3k/4] (qlin_gemm_ws with scheme QLIN_W4A4_E2M3, which takes no
    workspace): the results of qlin_gemm_w4a4 on the same codes."""
    lib = load()
    _dev_tensor(wq, "wq")
    m, n = xq.shape[0], wq.shape[0]
    ka, kb = _operand_bytes(QLIN_W4A4_E2M3, k)
    _need(xq, m * ka, "xq")
    _need(wq, n * kb, "wq")
    _need(x_scale, m * 4, "x_scale")
    _need(w_scale, n * 4, "w_scale")
    y = out if out is not None else torch.empty((m, n), dtype=y_dtype, device=wq.device)
    _need(y, m * n * y.element_size(), "y")
    st = lib.qlin_gemm_ws(QLIN_W4A4_E2M3, xq.data_ptr(), _ptr(x_scale), wq.data_ptr(), _ptr(w_scale), m, n, k,
                          y.data_ptr(), _TORCH_TO_QLIN[y.dtype], None, 0, _stream(wq.device))
    _check(st, "qlin_gemm_ws")
    return y


def qlin_gemm_geglu(scheme: int, xq, x_scale, wq, w_scale, k: int, h_dtype=torch.bfloat16,
                    out=None) -> torch.Tensor:
    """h [m][n2/2] = gelu(gate) * up from activation codes xq and the gate|up
    weight codes wq [n2] with rows interleaved in blocks of 32, both packed
    int4 (QLIN_W4A4) or both in E2M3 storage (QLIN_W4A4_E2M3)."""
    lib = load()
    _dev_tensor(wq, "wq")
    m, n2 = xq.shape[0], wq.shape[0]
    ka, kb = _operand_bytes(scheme, k)
    _need(xq, m * ka, "xq")
    _need(wq, n2 * kb, "wq")
    _need(x_scale, m * 4, "x_scale")
    _need(w_scale, n2 * 4, "w_scale")
    h = out if out is not None else torch.empty((m, n2 // 2), dtype=h_dtype, device=wq.device)
    _need(h, m * (n2 // 2) * h.element_size(), "h")
    st = lib.qlin_gemm_geglu(scheme, xq.data_ptr(), _ptr(x_scale), wq.data_ptr(), _ptr(w_scale), m, n2, k,
                             h.data_ptr(), _TORCH_TO_QLIN[h.dtype], _stream(wq.device))
    _check(st, "qlin_gemm_geglu")
    return h


def qlin_gemm_w4a4_geglu(xq, x_scale, wq, w_scale, k: int, h_dtype=torch.bfloat16, out=None) -> torch.Tensor:
    """h [m][n2/2] = gelu(gate) * up from packed int4 codes xq [m][k/2] and the
    gate|up weight codes wq [n2][k/2] with rows interleaved in blocks of 32."""
    lib = load()
    _dev_tensor(wq, "wq")
    m, n2 = xq.shape[0], wq.shape[0]
    _need(xq, m * (k // 2), "xq")
    _need(wq, n2 * (k // 2), "wq")
    _need(x_scale, m * 4, "x_scale")
    _need(w_scale, n2 * 4, "w_scale")
    h = out if out is not None else torch.empty((m, n2 // 2), dtype=h_dtype, device=wq.device)
    _need(h, m * (n2 // 2) * h.element_size(), "h")
    st = lib.qlin_gemm_w4a4_geglu(xq.data_ptr(), _ptr(x_scale), wq.data_ptr(), _ptr(w_scale), m, n2, k,
                                  h.data_ptr(), _TORCH_TO_QLIN[h.dtype], _stream(wq.device))
    _check(st, "qlin_gemm_w4a4_geglu")
    return h


def interleave_gate_up(gate: torch.Tensor, up: torch.Tensor, block: int = 32) -> torch.Tensor:
    """Rows of the fused gate|up weight (layout of qlin_gemm_w4a4_geglu): blocks
    of `block` gate rows, each followed by the same rows of up.  Pure data
    movement (torch ops), for preparing weights before quantization."""
    f = gate.shape[0]
    if up.shape[0] != f or f % block:
        raise ValueError("gate and up need the same row count, a multiple of the block")
    tail = tuple(gate.shape[1:])
    return torch.cat([gate.reshape((f // block, block) + tail), up.reshape((f // block, block) + tail)],
                     dim=1).reshape((2 * f,) + tail)


def qlin_gemv_w4a16(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor, group: int = 128,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [m][n] fp16 from fp16 x [m][k] and packed int4 weights with fp16 group scales."""
    lib = load()
    _dev_tensor(x, "x")
    m, k = x.shape
    n = wq.shape[0]
    _need(x, m * k * 2, "x")
    _need(wq, n * (k // 2), "wq")
    _need(w_scale, n * (k // group) * 2 if group > 0 else 0, "w_scale")
    y = out if out is not None else torch.empty((m, n), dtype=torch.float16, device=x.device)
    _need(y, m * n * 2, "y")
    st = lib.qlin_gemv_w4a16(x.data_ptr(), wq.data_ptr(), w_scale.data_ptr(), m, n, k, group, y.data_ptr(),
                             _stream(x.device))
    _check(st, "qlin_gemv_w4a16")
    return y


QLIN_STREAM_READ_SINK_WORDS = 4096


def qlin_stream_read(src: torch.Tensor, nbytes: Optional[int] = None, sink: Optional[torch.Tensor] = None
                     ) -> torch.Tensor:
    """Streaming read of the first nbytes (default: all) of the contiguous
    device tensor src (measurement aid); returns the sink words."""
    lib = load()
    _dev_tensor(src, "src")
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    _need(src, nbytes, "src")
    if sink is None:
        sink = torch.empty(QLIN_STREAM_READ_SINK_WORDS, dtype=torch.int32, device=src.device)
    _need(sink, QLIN_STREAM_READ_SINK_WORDS * 4, "sink")
    _check(lib.qlin_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(src.device)), "qlin_stream_read")
    return sink

