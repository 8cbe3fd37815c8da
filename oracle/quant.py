"""Quantizers: per-token / per-channel FP8 and INT8, 1x128 / 128x128 block FP8, MXFP4.

Test infrastructure only (see ``oracle/__init__.py``).

All inputs are bfloat16 bit patterns (``uint16`` arrays, row-major ``[rows, K]``); they
widen to fp32 exactly.

Sources:
* Scale rule s = max(amax, 1e-8) / 448 and q = e4m3(x / s), one scale per row:
  ``fp8_per_token`` in [P-FP8FP4] "Implementation sketch"; per-token activations and
  per-output-channel weights in [P-FP8FP4] "Scale granularity" and [P-FP8INT8] §5
  ("FP8 in practice", "INT8 in practice").
* Symmetric INT8, S = max|x| / 127: [P-LOWBIT] §2.1; per-token dynamic activations and
  per-channel static weights: [P-FP8INT8] §5 "INT8 in practice".
* 1x128 activation groups and 128x128 weight blocks: [P-FP8FP4] "Scale granularity";
  [P-FP8INT8] §5 "What DeepSeek did" and "The blockwise/fine-grained trend".
* MXFP4 (E2M1 elements, one E8M0 power-of-two scale per 32 elements): [P-LOWBIT] §2.4;
  [P-FP8FP4] "Where it came from" and the measured-model section.

Readings where the pages leave a step open:
* The scale and the quotient x/s are each one IEEE fp32 division (round to nearest
  even), in that order; the pages' emulation runs in fp32 and divides by s.
* The 1e-8 floor of the FP8 emulation is used for every amax-based scale (INT8 and
  block scales too), so an all-zero row or block gets s = fp32(1e-8)/qmax.
* INT8 codes are round-half-even(x/s) clamped to [-127, 127]; -128 is never produced.
* MXFP4 scale exponent (OCP MX rule, the spec the pages cite for MX formats):
  e = floor(log2(amax)) - 2, where 2 is E2M1's largest binade exponent, clamped to
  [-127, 127]; scale code e + 127; elements x / 2^e are encoded with saturation to +-6.
  A block whose amax is 0 gets code 127 (scale 1), following the emulation's rule that a
  zero scale becomes 1 ([P-FP8FP4] ``nvfp4``).
* A 32-element MX block that holds an infinity or a NaN (the pages do not say): the
  E8M0 scale code 255, the format's one special value (NaN), and element codes 0 (E2M1
  has no special values). Such a block decodes to NaN, so a non-finite input stays
  non-finite through the GEMM.
"""

from __future__ import annotations

import numpy as np

from .formats import (
    bf16_to_f32, e4m3_encode, e2m1_encode, pack_e2m1, INT8_QMAX, E4M3_MAX,
)

_EPS = np.float32(1e-8)


def _rows_f32(x_bits: np.ndarray) -> np.ndarray:
    x = np.asarray(x_bits, dtype=np.uint16)
    if x.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array of bf16 bits")
    return bf16_to_f32(x)


def _absmax_last(x: np.ndarray) -> np.ndarray:
    # NaN is ignored (IEEE maxNum), so one NaN element does not poison its row's scale.
    return np.nanmax(np.abs(x), axis=-1) if x.shape[-1] else np.zeros(x.shape[:-1], np.float32)


def fp8_scale(amax: np.ndarray) -> np.ndarray:
    """s = fp32(max(amax, 1e-8)) / 448, one IEEE fp32 division."""
    a = np.asarray(amax, dtype=np.float32)
    a = np.where(np.isnan(a), a, np.maximum(a, _EPS)).astype(np.float32)
    return (a / np.float32(E4M3_MAX)).astype(np.float32)


def quantize_rows_fp8(x_bits: np.ndarray):
    """Per-row dynamic E4M3FN quantization -> (codes uint8 [R,K], scales fp32 [R]).

    Used both per token (rows of X) and per output channel (rows of W [N,K]).
    """
    x = _rows_f32(x_bits)
    with np.errstate(all="ignore"):
        s = fp8_scale(_absmax_last(x))
        v = (x / s[:, None]).astype(np.float32)      # IEEE fp32 division per element
    return e4m3_encode(v), s


def quantize_per_token_fp8(x_bits):
    """Activations X [M,K] -> per-token E4M3FN codes and fp32 scales [M]."""
    return quantize_rows_fp8(x_bits)


def quantize_weight_per_channel_fp8(w_bits):
    """Weights W [N,K] -> per-output-channel E4M3FN codes and fp32 scales [N]."""
    return quantize_rows_fp8(w_bits)


def quantize_rows_int8(x_bits: np.ndarray):
    """Per-row symmetric INT8: s = fp32(max(amax,1e-8))/127, q = clamp(rne(x/s), +-127)."""
    x = _rows_f32(x_bits)
    with np.errstate(all="ignore"):
        a = _absmax_last(x).astype(np.float32)
        a = np.where(np.isnan(a), a, np.maximum(a, _EPS)).astype(np.float32)
        s = (a / np.float32(INT8_QMAX)).astype(np.float32)
        v = (x / s[:, None]).astype(np.float32)
        q = np.clip(np.rint(v), -INT8_QMAX, INT8_QMAX)
    q = np.nan_to_num(q, nan=0.0)
    return q.astype(np.int8), s


def quantize_per_token_int8(x_bits):
    return quantize_rows_int8(x_bits)


def quantize_weight_per_channel_int8(w_bits):
    return quantize_rows_int8(w_bits)


def quantize_per_token_group_fp8(x_bits: np.ndarray, group: int = 128):
    """1 x group activation scales: codes [M,K], scales fp32 [M, K/group].

    Each contiguous run of ``group`` elements along K is quantized like a row of
    ``quantize_rows_fp8``.
    """
    x = _rows_f32(x_bits)
    M, K = x.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    xg = x.reshape(M, K // group, group)
    with np.errstate(all="ignore"):
        s = fp8_scale(_absmax_last(xg))
        v = (xg / s[..., None]).astype(np.float32)
    return e4m3_encode(v).reshape(M, K), s


def quantize_weight_block_fp8(w_bits: np.ndarray, block: int = 128):
    """block x block weight scales: codes [N,K], scales fp32 [ceil(N/block), K/block].

    One amax per (block of output rows, block of K); a partial last row block (N not a
    multiple of ``block``) covers the remaining rows.
    """
    w = _rows_f32(w_bits)
    N, K = w.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    nb, kb = -(-N // block), K // block
    s = np.empty((nb, kb), dtype=np.float32)
    q = np.empty((N, K), dtype=np.uint8)
    for b in range(nb):
        rows = w[b * block:(b + 1) * block].reshape(-1, kb, block)   # [r, kb, block]
        with np.errstate(all="ignore"):
            amax = np.nanmax(np.abs(rows), axis=(0, 2))
            sb = fp8_scale(amax)
            v = (rows / sb[None, :, None]).astype(np.float32)
        s[b] = sb
        q[b * block:(b + 1) * block] = e4m3_encode(v).reshape(-1, K)
    return q, s


def mx_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """OCP MX shared exponent for E2M1: floor(log2 amax) - 2, clamped to [-127, 127].

    Exact via frexp. amax == 0 maps to 0 (scale code 127).
    """
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)
    e = np.clip(ex - 1 - 2, -127, 127)
    return np.where(a == 0, 0, e).astype(np.int64)


def quantize_mxfp4(x_bits: np.ndarray):
    """MXFP4 rows: packed E2M1 [R, K/2] (element 2i in the low nibble) + E8M0 [R, K/32]."""
    x = _rows_f32(x_bits).astype(np.float64)
    R, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(R, K // 32, 32)
    bad = ~np.all(np.isfinite(xb), axis=-1)        # blocks with an infinity or a NaN
    xb = np.where(bad[..., None], 0.0, xb)
    amax = np.max(np.abs(xb), axis=-1)
    e = mx_scale_exponent(amax)
    scaled = xb / np.ldexp(1.0, e)[..., None]      # exact: division by a power of two
    codes = e2m1_encode(scaled).reshape(R, K)
    sc = np.where(bad, 255, e + 127).astype(np.uint8)
    return pack_e2m1(codes), sc
