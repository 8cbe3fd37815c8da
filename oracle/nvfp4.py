"""NVFP4: E2M1 elements, one E4M3 scale per 16 elements, one fp32 scale per tensor.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* Two-level scaling as the ``nvfp4`` emulation of [P-FP8FP4] "Implementation sketch"
  computes it: a tensor scale g from the whole tensor's amax, an E4M3 scale per block of
  16 consecutive values, E2M1 elements. The measured-model section of [P-FP8FP4] describes
  the same format (an E4M3 scale per 16 values and an fp32 tensor scale).
* Block of 16, E4M3 scale, 0.5 bits of scale per element, 4.5 bits per element in all:
  [P-LOWBIT] §2.4 (the MXFP4 / NVFP4 table).

Steps, in the emulation's order, each an IEEE fp32 operation (the emulation runs on fp32
tensors):
1. g = amax(|x| over the tensor) / 2688, where 2688 = 448 * 6 (largest E4M3 times largest
   E2M1 magnitude).
2. For each block b of 16 values along a row: t_b = (amax_b / 6) / g, two divisions in
   that order; the block's scale code is e4m3(t_b) (round half to even, saturating at 448).
3. s_b = dec(code_b) * g; a block whose s_b is 0 uses s_b = 1 instead.
4. Each element: code = e2m1(x / s_b) (round half to even, saturating at 6).
The dequantized value of an element is dec4(code) * s_b.

Readings where the pages leave a step open:
* An all-zero tensor makes step 1 give g = 0 and step 2 divide 0 by 0. The emulation's own
  rule for a zero scale (use 1) is applied to g as well: g = 1, and every code is then 0.
* The stored form is the packed E2M1 codes [R, K/2] (element 2i in the low nibble, as for
  MXFP4), the E4M3 scale codes [R, K/16] and g; step 3 recomputes s_b from them, so the
  stored form fixes every dequantized value.
* A caller may supply g instead of computing it from the tensor (a calibrated or offline
  tensor scale); steps 2-4 are the same. Values beyond 6 * 448 * g then saturate.
* Non-finite inputs are outside the contract, as for the other quantizers.
"""

from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, e4m3_decode, e4m3_encode, e2m1_decode, e2m1_encode, pack_e2m1, unpack_e2m1

BLOCK = 16
_TENSOR_DIV = np.float32(448.0 * 6.0)
_SIX = np.float32(6.0)


def tensor_scale(x_bits: np.ndarray) -> np.float32:
    """Step 1: g = fp32(amax / 2688), or 1 for an all-zero tensor."""
    x = bf16_to_f32(np.asarray(x_bits, np.uint16))
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / _TENSOR_DIV)


def block_scales(codes: np.ndarray, g) -> np.ndarray:
    """Step 3: fp32 s_b = dec(code_b) * g, with 1 where that product is 0."""
    g = np.float32(g)
    s = (e4m3_decode(codes).astype(np.float32) * g).astype(np.float32)
    return np.where(s == 0, np.float32(1.0), s).astype(np.float32)


def quantize_nvfp4(x_bits: np.ndarray, g=None):
    """Rows of a bf16 [R, K] tensor (K % 16 == 0) to NVFP4.

    Returns (packed E2M1 uint8 [R, K/2], E4M3 scale codes uint8 [R, K/16], g fp32).
    With g None the tensor scale comes from this tensor (step 1); otherwise g is used.
    """
    x = bf16_to_f32(np.asarray(x_bits, np.uint16))
    R, K = x.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 16")
    g = tensor_scale(x_bits) if g is None else np.float32(g)
    xb = x.reshape(R, K // BLOCK, BLOCK)
    amax_b = np.max(np.abs(xb), axis=-1).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = ((amax_b / _SIX).astype(np.float32) / g).astype(np.float32)
    scodes = e4m3_encode(t)
    s = block_scales(scodes, g)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        v = (xb / s[..., None]).astype(np.float32)
    codes = e2m1_encode(v).reshape(R, K)
    return pack_e2m1(codes), scodes, np.float32(g)


def dequantize_nvfp4(packed: np.ndarray, scodes: np.ndarray, g) -> np.ndarray:
    """fp64 values dec4(code) * s_b of a stored NVFP4 tensor."""
    q = e2m1_decode(unpack_e2m1(packed))
    s = np.repeat(block_scales(scodes, g).astype(np.float64), BLOCK, axis=1)
    return q * s


def gemm_nvfp4_ref(xq, xs, gx, wq, ws, gw) -> np.ndarray:
    """y[m,n] = sum_b s_x[m,b] s_w[n,b] sum_{k in b} dec4(xq[m,k]) dec4(wq[n,k]), in fp64.

    The scaled operands are formed first (each product dec4 * s_b is exact in fp64), then
    one fp64 matrix product.
    """
    return dequantize_nvfp4(xq, xs, gx) @ dequantize_nvfp4(wq, ws, gw).T
