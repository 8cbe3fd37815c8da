"""Element and scale formats: OCP FP8 E4M3FN, FP4 E2M1, E8M0, INT8 and bfloat16.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* E4M3FN layout, bias 7, max 448 = 1.75 * 2^8 at 0x7E/0xFE, min normal 2^-6, ULP(1) = 2^-3,
  signed zeros, NaN only at S.1111.111, saturating conversion: [P-LOWBIT] §2.2 (FP8 format
  comparison table and E4M3FN details) and Try-it 05.
* Value formula (-1)^S 2^(E-bias) (1 + M/2^m) with subnormals, relative error bound
  2^-(m+1): [P-FP8FP4] "The number formats".
* Rounding: the emulation ``fp_round(x, mbits, emin, maxv)`` of [P-FP8FP4]
  "Implementation sketch": pick the binade of |x| (clamped below at emin), round to the
  2^mbits-step grid of that binade half-to-even, then clamp to +-maxv. E4M3 is
  (3, -6, 448), E2M1 is (1, 0, 6).
* E2M1 elements and E8M0 (8-bit pure exponent, bias 127) scales: [P-LOWBIT] §2.4 table.

Reading (the pages' emulation picks the binade with a float log2, which can misplace
values just below a power of two): the binade is taken exactly, from ``frexp``.
NaN encodes to 0x7F. A code is produced from the rounded value, so a value that rounds
up into the next binade gets that binade's code.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL_EXP = -6
E4M3_MBITS = 3
E2M1_MAX = 6.0


# ----------------------------------------------------------------------------- E4M3FN
def e4m3_decode(codes) -> np.ndarray:
    """Decode E4M3FN byte codes to float64 ([P-LOWBIT] §2.2).

    S = bit 7, E = bits 6..3, M = bits 2..0; E == 15 and M == 7 is NaN; E == 0 is the
    subnormal range 2^-6 * M/8; otherwise 2^(E-7) * (1 + M/8).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def fp_round(x, mbits: int, emin: int, maxv: float) -> np.ndarray:
    """Round to a low-precision float grid, as the [P-FP8FP4] emulation does.

    Steps: binade exponent e = max(floor(log2|x|), emin) (exact, via frexp); grid step
    2^(e - mbits); round |x|/step half-to-even; multiply back; clamp to maxv. Returns the
    rounded magnitude with the sign of x (NaN stays NaN). All steps are exact in fp64 for
    fp32 or fp64 inputs, since they only scale by powers of two.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1)
        e = np.maximum(ex - 1, emin)
        step = np.ldexp(1.0, e - mbits)
        r = np.rint(a / step)
        val = np.minimum(r * step, maxv)
    val = np.where(np.isinf(a), maxv, val)
    return np.copysign(val, x)


def e4m3_encode(x) -> np.ndarray:
    """Encode to E4M3FN codes: round half-to-even with saturation to +-448.

    [P-LOWBIT] §2.2 (saturation mode) and the e4m3 instance of ``fp_round`` in
    [P-FP8FP4] "Implementation sketch". Signed zeros keep their sign; NaN -> 0x7F.
    """
    with np.errstate(invalid="ignore"):
        x = np.asarray(x, dtype=np.float64)
    v = fp_round(x, E4M3_MBITS, E4M3_MIN_NORMAL_EXP, E4M3_MAX)
    a = np.abs(v)
    with np.errstate(invalid="ignore", divide="ignore"):
        _, ex = np.frexp(a)
        eb = ex - 1                                   # binade of the rounded value
        normal = a >= 2.0 ** -6
        mant = np.where(normal, np.ldexp(a, -np.where(normal, eb, 0)) - 1.0, 0.0) * 8.0
        code_n = (eb + 7) * 8 + mant
        code_s = a * 512.0                            # subnormal grid step 2^-9
        code = np.where(normal, code_n, code_s)
    code = np.nan_to_num(code, nan=0.0).astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------------------- E2M1 / E8M0
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (low 4 bits of each value) to float64 ([P-LOWBIT] §2.4).

    1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2,
    3, 4, 6 (the grid of fp_round(x, 1, 0, 6.0) in [P-FP8FP4]).
    """
    c = np.asarray(codes).astype(np.int64) & 15
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(x) -> np.ndarray:
    """Encode to E2M1 4-bit codes (uint8 in 0..15): RNE, saturate to +-6, keep zero sign."""
    x = np.asarray(x, dtype=np.float64)
    v = fp_round(x, 1, 0, E2M1_MAX)
    a = np.abs(v)
    with np.errstate(invalid="ignore", divide="ignore"):
        _, ex = np.frexp(a)
        eb = ex - 1
        normal = a >= 1.0
        mant = np.where(normal, np.ldexp(a, -np.where(normal, eb, 0)) - 1.0, 0.0) * 2.0
        code = np.where(normal, (eb + 1) * 2 + mant, a * 2.0)
    code = np.nan_to_num(code, nan=0.0).astype(np.int64)
    code = np.where(np.signbit(v), code | 8, code)
    return code.astype(np.uint8)


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale: 2^(c - 127); 0xFF is NaN ([P-LOWBIT] §2.4: pure exponent, bias 127)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    """Pack pairs of 4-bit codes along the last axis: element 2i low nibble, 2i+1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 15) | ((c[..., 1::2] & 15) << 4)


def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


# ----------------------------------------------------------------------------- bfloat16
def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 (exact): the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f64_to_bf16_rne(x) -> np.ndarray:
    """Round float values to the nearest bfloat16, ties to even; return uint16 bits.

    Written from the definition: bf16 keeps 8 significant bits and fp32's exponent range
    (min normal 2^-126, subnormal step 2^-133). Values whose rounding exceeds the largest
    finite bf16 become infinity; NaN becomes a quiet NaN (0x7FC0 with the input's sign).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, ex = np.frexp(a)
        e = np.maximum(ex - 1, -126)
        step = np.ldexp(1.0, e - 7)
        r = np.rint(a / step) * step
    maxbf = float(np.ldexp(255.0, 120))  # (2 - 2^-7) * 2^127
    r = np.where((r > maxbf) | np.isinf(a), np.inf, r)
    r = np.copysign(r, x)
    bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nan_bits = np.where(np.signbit(x), 0xFFC0, 0x7FC0).astype(np.uint16)
    return np.where(np.isnan(x), nan_bits, bits)


# ----------------------------------------------------------------------------- INT8
INT8_QMAX = 127
