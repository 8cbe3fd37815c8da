"""W4A16: symmetric INT4 weights with one fp16 scale per group of 128 along K, bf16
activations, and the weight-only GEMM over them.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* Symmetric INT4: q in [-7, 7], S = max|x| / 7, no zero point; groups of 32, 64 or 128
  values share one scale: [P-LOWBIT] §2.3 (INT4 table).
* Scale metadata of 2 bytes per group (262,144 bytes, 3.125%, for a 4096 x 4096 matrix at
  G = 128) and the weight-only path: unpack, dequantize S * q, multiply with 16-bit
  activations: [P-LOWBIT] §2.3 (metadata overhead) and §3.3 (weight-only execution path).
* Group size 128 and 0.5 bytes per parameter plus scales (about 3.88x less weight traffic
  than fp16): [P-LOWBIT] §3.3 and §5.1; [P-FP8FP4] "Why low precision helps".

Readings where the pages leave a step open:
* The 2-byte scale is an IEEE fp16 value: S = fp16_rne(fp32(amax / 7)). Codes are computed
  against that stored scale, q = clamp(rint_half_even(fp32(x) / S), -7, 7) with an IEEE
  fp32 quotient, so that S * q is the value the stored pair represents.
* A group whose amax is 0 gets S = 1 (the [P-FP8FP4] emulation's rule for a zero scale);
  its codes are 0. A scale above the largest fp16 (amax > 7 * 65504) saturates to 65504.
* Codes are 4-bit two's complement, two per byte, element 2i in the low nibble (the
  packing used for E2M1 here).
* The GEMM is y[m, n] = sum_g S[n, g] sum_{k in g} x[m, k] q[n, k], exact in fp64, compared
  within the floating-point tolerance. The pages' pipeline rounds S * q to fp16 before a
  16-bit matrix product; keeping S outside the group sum is the exact form of the same
  contraction, and both fall within that tolerance.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32

GROUP = 128
INT4_QMAX = 7
_F16_MAX = np.float32(65504.0)


def _f16_rne(v: np.ndarray) -> np.ndarray:
    """fp32 -> nearest fp16 (ties to even), saturating at +-65504; returns float16."""
    v = np.asarray(v, np.float32)
    with np.errstate(over="ignore"):
        h = v.astype(np.float16)                       # IEEE round to nearest even
    return np.where(np.isinf(h) & np.isfinite(v), np.float16(65504.0) * np.sign(v), h).astype(np.float16)


def quantize_int4_groups(w_bits: np.ndarray, group: int = GROUP):
    """bf16 [N, K] (K % group == 0) -> (packed uint8 [N, K/2], fp16 scales [N, K/group])."""
    w = bf16_to_f32(np.asarray(w_bits, np.uint16))
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(N, K // group, group)
    amax = np.max(np.abs(wg), axis=-1).astype(np.float32)
    s = _f16_rne((amax / np.float32(INT4_QMAX)).astype(np.float32))
    s = np.where(s == 0, np.float16(1.0), s).astype(np.float16)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (wg / s.astype(np.float32)[..., None]).astype(np.float32)
    q = np.clip(np.rint(v), -INT4_QMAX, INT4_QMAX).astype(np.int64).reshape(N, K)
    nib = (q & 15).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8), s


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Packed nibbles -> int64 codes in [-8, 7] (two's complement)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int64)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return np.where(out >= 8, out - 16, out)


def dequantize_int4(packed: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """fp64 S[n, g] * q[n, k]."""
    q = unpack_int4(packed).astype(np.float64)
    return q * np.repeat(np.asarray(scales, np.float16).astype(np.float64), group, axis=1)


def gemm_w4a16_ref(x_bits: np.ndarray, packed: np.ndarray, scales: np.ndarray,
                   group: int = GROUP) -> np.ndarray:
    """y[m, n] = sum_g S[n, g] sum_{k in g} x[m, k] q[n, k], in fp64 (every product and
    partial sum of bf16 x and integer q is exact in fp64 at these sizes)."""
    x = bf16_to_f32(np.asarray(x_bits, np.uint16)).astype(np.float64)
    return x @ dequantize_int4(packed, scales, group).T
