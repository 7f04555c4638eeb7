"""Agreement rules between the HIP path and the oracle.

TEST INFRASTRUCTURE ONLY.

  codes    equal, or off by exactly one where the oracle's pre-rounding value
           lies within 1e-5 * max(1, |r|) of a rounding boundary (a
           half-integer), for at most floor(1e-4 * count) elements;
  scales   relative difference <= 1e-6 (zero only against zero);
  outputs  max|y - y_ref| / max|y_ref| <= 1e-2 and
           ||y - y_ref||_2 / ||y_ref||_2 <= 1e-3, where y_ref is the oracle's
           float32 result rounded to the output dtype.
  integers (accumulators, packed bytes) are compared for equality directly.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class CompareResult:
    ok: bool
    detail: str
    stats: dict = field(default_factory=dict)

    def __bool__(self) -> bool:  # pragma: no cover - convenience
        return self.ok


def compare_codes(q_gpu, q_ref, r_ref, window: float = 1e-5,
                  max_frac: float = 1e-4) -> CompareResult:
    q_gpu = np.asarray(q_gpu, dtype=np.int64)
    q_ref = np.asarray(q_ref, dtype=np.int64)
    r_ref = np.asarray(r_ref, dtype=np.float64)
    if q_gpu.shape != q_ref.shape:
        return CompareResult(False, f"shape {q_gpu.shape} != {q_ref.shape}")
    d = q_gpu - q_ref
    n_diff = int(np.count_nonzero(d))
    if n_diff == 0:
        return CompareResult(True, "identical", {"flips": 0, "count": q_ref.size})
    if np.max(np.abs(d)) > 1:
        idx = np.unravel_index(np.argmax(np.abs(d)), d.shape)
        return CompareResult(False, f"code differs by {int(d[idx])} at {idx}: "
                             f"gpu {int(q_gpu[idx])} ref {int(q_ref[idx])} r {r_ref[idx]!r}")
    mask = d != 0
    r = r_ref[mask]
    dist = np.abs(np.abs(r - np.floor(r)) - 0.5)  # distance to nearest half-integer
    near = dist <= window * np.maximum(1.0, np.abs(r))
    if not np.all(near):
        bad = np.argwhere(mask)[~near][0]
        bad = tuple(int(i) for i in bad)
        return CompareResult(False, f"flip away from a rounding boundary at {bad}: "
                             f"gpu {int(q_gpu[bad])} ref {int(q_ref[bad])} r {r_ref[bad]!r}")
    limit = int(np.floor(max_frac * q_ref.size))
    if n_diff > limit:
        return CompareResult(False, f"{n_diff} boundary flips > limit {limit}",
                             {"flips": n_diff, "count": q_ref.size})
    return CompareResult(True, f"{n_diff} boundary flips (limit {limit})",
                         {"flips": n_diff, "count": q_ref.size})


def compare_scales(s_gpu, s_ref, rtol: float = 1e-6) -> CompareResult:
    s_gpu = np.asarray(s_gpu, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    if s_gpu.shape != s_ref.shape:
        return CompareResult(False, f"shape {s_gpu.shape} != {s_ref.shape}")
    zero = s_ref == 0
    if np.any(s_gpu[zero] != 0):
        return CompareResult(False, "nonzero scale where the oracle's is zero")
    rel = np.abs(s_gpu[~zero] - s_ref[~zero]) / np.abs(s_ref[~zero])
    worst = float(rel.max()) if rel.size else 0.0
    return CompareResult(worst <= rtol, f"max rel {worst:.3g} (tol {rtol})", {"max_rel": worst})


def compare_outputs(y, y_ref, max_rel: float = 1e-2, rms_rel: float = 1e-3) -> CompareResult:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        return CompareResult(False, f"shape {y.shape} != {y_ref.shape}")
    if not np.all(np.isfinite(y)):
        return CompareResult(False, "non-finite output")
    denom_max = float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    denom_rms = float(np.linalg.norm(y_ref))
    err = y - y_ref
    if denom_max == 0.0:
        ok = not np.any(err)
        return CompareResult(ok, "reference is all zeros", {})
    mrel = float(np.max(np.abs(err))) / denom_max
    rrel = float(np.linalg.norm(err)) / denom_rms
    ok = mrel <= max_rel and rrel <= rms_rel
    return CompareResult(ok, f"max rel {mrel:.3g} (tol {max_rel}), rms rel {rrel:.3g} (tol {rms_rel})",
                         {"max_rel": mrel, "rms_rel": rrel})
