"""Static per-tensor activation scales, the saturation monitor and delayed scaling.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* Per-tensor FP8 scaling x_fp8 = clamp(x / s, -448, 448), with s chosen so that
  max|x| / s is about 448: [P-FP8INT8] §5, "FP8 in practice" (Scaling).
* Static activation scales are calibrated once; traffic beyond the calibrated maximum
  saturates, and the monitor is the fraction of saturated values per layer on live
  traffic: [P-FP8FP4] "Recipe" (static vs dynamic scales) and "Failure modes and how to
  detect them".
* Delayed scaling sets the scale from a history of recent amax values, so that no
  synchronization is needed: [P-FP8INT8] §5, "FP8 in practice".

Readings (listed in the design notes):
* The quotient is one IEEE fp32 division, as in the dynamic quantizers.
* "Saturated" means the clamp changed the value: |x / s| > 448 for E4M3FN, and
  |rne(x / s)| > 127 for INT8. NaN elements are not counted; they encode as in the dynamic
  quantizers (E4M3FN NaN code, INT8 zero).
* The tensor amax ignores NaN (IEEE maxNum), like the dynamic quantizers.
* Delayed scaling: the amax of step t goes to slot t mod H of an H-long history, and the
  scale for the next step is fp32(max(max(history), 1e-8)) / qmax, the per-tensor form of
  the dynamic rule.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, e4m3_encode

E4M3_MAX = 448.0
INT8_QMAX = 127.0


def _tensor_f32(x_bits):
    return bf16_to_f32(np.asarray(x_bits, dtype=np.uint16))


def tensor_amax(x_bits) -> np.float32:
    x = _tensor_f32(x_bits)
    if x.size == 0:
        return np.float32(0.0)
    with np.errstate(invalid="ignore"):
        m = np.nanmax(np.abs(x)) if not np.all(np.isnan(x)) else np.float32(0.0)
    return np.float32(m)


def quantize_static_fp8(x_bits, s):
    """-> (E4M3FN codes, number of saturated elements, tensor amax)."""
    x = _tensor_f32(x_bits)
    with np.errstate(all="ignore"):
        v = (x / np.float32(s)).astype(np.float32)          # IEEE fp32 division
        sat = int(np.count_nonzero(np.abs(v) > np.float32(E4M3_MAX)))
        v = np.clip(v, -E4M3_MAX, E4M3_MAX)                  # NaN passes through
    return e4m3_encode(v.astype(np.float64)), sat, tensor_amax(x_bits)


def quantize_static_int8(x_bits, s):
    """-> (int8 codes, number of saturated elements, tensor amax)."""
    x = _tensor_f32(x_bits)
    with np.errstate(all="ignore"):
        r = np.rint((x / np.float32(s)).astype(np.float32))
        sat = int(np.count_nonzero(np.abs(r) > INT8_QMAX))
        q = np.nan_to_num(np.clip(r, -INT8_QMAX, INT8_QMAX), nan=0.0)
    return q.astype(np.int8), sat, tensor_amax(x_bits)


def delayed_scale_update(history, amax, step: int, fmt: str):
    """-> (updated history, next scale): history[step mod H] = amax, then
    scale = fp32(max(max(history), 1e-8)) / qmax."""
    h = np.array(history, dtype=np.float32, copy=True)
    h[step % len(h)] = np.float32(amax)
    m = np.float32(max(float(np.max(h)), float(np.float32(1e-8))))
    qmax = np.float32(E4M3_MAX if fmt == "e4m3fn" else INT8_QMAX)
    return h, np.float32(m / qmax)
