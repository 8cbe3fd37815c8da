"""SmoothQuant offline preparation for the INT8 W8A8 variant.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* Identity Y = X W^T = (X diag(s)^-1)(W diag(s))^T for any positive per-input-channel
  vector s, and the choice s_j = max|X_:j|^alpha / max|W_:j|^(1-alpha), with
  alpha = 0.5 equalising the two per-channel ranges: [P-FP8FP4] "SmoothQuant: move the
  outliers into the weights"; [P-LOWBIT] §4.2 (formulation, migration strength table).
* Clamping both maxima below at 1e-5 before the powers: ``smooth`` in [P-FP8FP4]
  "Implementation sketch".
* Applied offline, before quantization: [P-LOWBIT] §4.3.

W is stored [N, K] (output rows), so max|W_:j| over output channels is the maximum over
rows of column j, as ``W.abs().amax(0)`` is in the pages' emulation.

Readings (the pages leave the precision open):
* Channel maxima are exact (a max of bf16 magnitudes).
* s is evaluated in fp32. For alpha = 1/2 the two powers are correctly rounded fp32
  square roots and the quotient is one IEEE fp32 division, so the result is a single
  well-defined fp32 value. alpha = 0 and alpha = 1 reduce to 1/w and a (one division or
  none). Other alpha values use fp64 powers rounded once to fp32 and are compared within
  a relative tolerance, since no library computes fp32 powers correctly rounded.
* Smoothed inputs are rounded to bfloat16 (round to nearest even) from the fp32 quotient
  x / s_j (activations) or product w * s_j (weights): they are the bf16 tensors the INT8
  quantizer then reads.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, f64_to_bf16_rne

_FLOOR = np.float32(1e-5)


def channel_absmax(x_bits: np.ndarray) -> np.ndarray:
    """max_r |x[r, j]| for each column j of a [R, K] bf16 matrix -> fp32 [K]."""
    x = bf16_to_f32(np.asarray(x_bits, np.uint16))
    if x.shape[0] == 0:
        return np.zeros(x.shape[1], np.float32)
    return np.nanmax(np.abs(x), axis=0).astype(np.float32)


def smooth_scales(act_max, w_max, alpha: float = 0.5) -> np.ndarray:
    """s_j = max(a_j, 1e-5)^alpha / max(w_j, 1e-5)^(1 - alpha), fp32 [K]."""
    a = np.maximum(np.asarray(act_max, np.float32), _FLOOR).astype(np.float32)
    w = np.maximum(np.asarray(w_max, np.float32), _FLOOR).astype(np.float32)
    if alpha == 0.5:
        return (np.sqrt(a) / np.sqrt(w)).astype(np.float32)
    if alpha == 0.0:
        return (np.float32(1.0) / w).astype(np.float32)
    if alpha == 1.0:
        return a.copy()
    s = np.power(a.astype(np.float64), alpha) / np.power(w.astype(np.float64), 1.0 - alpha)
    return s.astype(np.float32)


def smooth_activations(x_bits, s) -> np.ndarray:
    """Xhat = bf16(x[:, j] / s_j) with one fp32 division per element; bf16 bits out."""
    x = bf16_to_f32(np.asarray(x_bits, np.uint16))
    with np.errstate(all="ignore"):
        v = (x / np.asarray(s, np.float32)[None, :]).astype(np.float32)
    return f64_to_bf16_rne(v.astype(np.float64))


def smooth_weights(w_bits, s) -> np.ndarray:
    """What = bf16(w[:, j] * s_j) with one fp32 product per element; bf16 bits out."""
    w = bf16_to_f32(np.asarray(w_bits, np.uint16))
    with np.errstate(all="ignore"):
        v = (w * np.asarray(s, np.float32)[None, :]).astype(np.float32)
    return f64_to_bf16_rne(v.astype(np.float64))
