"""Extended GEMM epilogue: bias, activation and FP8 requantized output.

Test infrastructure only (see ``oracle/__init__.py``).

Source: [P-FP8INT8] §6-9, the FP8 GEMM epilogue written out under "Under the hood". After
the FP32 accumulation the epilogue (1) dequantizes by the product of the two scales, (2)
adds the bias, (3) applies the activation, and (4) when the next layer consumes FP8,
divides by a static output scale, clamps to +-448 and stores E4M3; otherwise it stores
BF16. The same section's INT8 schematic writes the INT8 form as
diag(S_x) (X_int8 W_int8) diag(S_w) + bias.

Readings where the pages are silent (each listed in the design notes):
* The bias is a bf16 vector over the N output channels, widened exactly.
* Activations: none, ReLU max(v, 0), and SiLU v * sigmoid(v) (the pages use SiLU for the
  MLP's gate; they name no other).
* FP8 operands: the reference is the exact value up to fp64 rounding,
  y = s_x[m] s_w[n] acc + b[n], the activation in fp64, then y / s_out clamped to +-448
  and encoded E4M3 round-half-even. Outputs are compared within a tolerance because the
  GPU's accumulation order is free.
* INT8 operands: one fixed fp32 order, so that the result is bit-exact for no activation
  and ReLU: v = fp32(fp32(fp32(acc) s_x) s_w), then fp32(v + b), then ReLU; the FP8
  output divides in IEEE fp32 and clamps before encoding. SiLU is evaluated in fp64 from
  the fp32 value and compared within a tolerance (the exponential is not fixed by the
  pages).
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, e4m3_encode, f64_to_bf16_rne
from .gemm import gemm_fp8_ref, gemm_int8_acc

ACTIVATIONS = ("none", "relu", "silu")
FP8_MAX = 448.0


def silu64(v) -> np.ndarray:
    """v * sigmoid(v) = v / (1 + exp(-v)) in fp64, written so that exp never overflows."""
    v = np.asarray(v, np.float64)
    e = np.exp(-np.abs(v))                      # in (0, 1]
    sig = np.where(v >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return v * sig


def _activate(v, act: str):
    if act == "none":
        return v
    if act == "relu":
        return np.maximum(v, 0)
    if act == "silu":
        return silu64(v)
    raise ValueError(f"unknown activation {act!r}")


def fp8_path_ref(xq, sx, wq, sw, bias_bits=None, act: str = "none", s_out=None):
    """FP8 operands. Returns the fp64 value the epilogue stores before the final rounding:
    act(s_x s_w acc + b) for a bf16 output, or clamp(act(...) / s_out, +-448) for an FP8
    output (whose E4M3 code is ``e4m3_encode`` of it)."""
    y = gemm_fp8_ref(xq, sx, wq, sw)
    if bias_bits is not None:
        y = y + bf16_to_f64(bias_bits)[None, :]
    y = _activate(y, act)
    if s_out is None:
        return y
    return np.clip(y / float(s_out), -FP8_MAX, FP8_MAX)


def int8_path_values(xq, sx, wq, sw, bias_bits=None, act: str = "none") -> np.ndarray:
    """INT8 operands: the fp32 value after dequantization, bias and activation, in the
    fixed order above (float32 array; SiLU's value is rounded from fp64)."""
    acc = gemm_int8_acc(xq, wq)
    v = (np.asarray(acc).astype(np.float32) * np.asarray(sx, np.float32)[:, None]).astype(np.float32)
    v = (v * np.asarray(sw, np.float32)[None, :]).astype(np.float32)
    if bias_bits is not None:
        b = bf16_to_f64(bias_bits).astype(np.float32)
        v = (v + b[None, :]).astype(np.float32)
    if act == "silu":
        return silu64(v.astype(np.float64)).astype(np.float32)
    return _activate(v, act).astype(np.float32)


def int8_path_ref(xq, sx, wq, sw, bias_bits=None, act: str = "none", s_out=None) -> np.ndarray:
    """INT8 operands: bf16 bit patterns (s_out None) or E4M3FN codes of the output."""
    v = int8_path_values(xq, sx, wq, sw, bias_bits, act)
    if s_out is None:
        return f64_to_bf16_rne(v.astype(np.float64))
    q = (v / np.float32(s_out)).astype(np.float32)           # IEEE fp32 division
    q = np.clip(q, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return e4m3_encode(q.astype(np.float64))


def e4m3_spacing(v) -> np.ndarray:
    """Distance between adjacent E4M3 values around |v| (2^(e-3) in the binade of v,
    2^-9 among the subnormals): one unit of the final rounding."""
    a = np.abs(np.asarray(v, np.float64))
    _, e = np.frexp(np.maximum(a, 2.0 ** -9))
    return np.exp2(np.maximum(e - 1, -6) - 3)
