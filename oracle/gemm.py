"""Reference contractions with their scale epilogues.

Test infrastructure only (see ``oracle/__init__.py``).

Shapes: activations codes ``xq [M,K]``, weight codes ``wq [N,K]`` (output-channel rows,
K contiguous), output ``[M,N] = X W^T``.

Sources:
* Scale-factoring identity Xhat What^T = diag(s_X) (X_q W_q^T) diag(s_W), which makes the
  scales an epilogue after the low-precision reduction: [P-FP8FP4] "Scale granularity";
  [P-LOWBIT] §3.4 (W8A8 execution path) and §4.3 (runtime GEMM, equation with
  diag(Delta_X) and diag(Delta_W)).
* FP8 operands with FP32 accumulation; INT8 operands with INT32 accumulation and the
  dequantization Y = Y_int32 x s_x[token] x s_w[channel]: [P-FP8INT8] §5 ("FP8 in
  practice", "INT8 in practice") and §6-9 (GEMM epilogue).
* Block-scaled FP8 with the fp32 partial of each 128-wide K group multiplied by its two
  scales before it joins the running sum: [P-FP8INT8] §5 "What DeepSeek did".
* MXFP4: [P-LOWBIT] §2.4.

The FP8, block-scaled and MXFP4 references return fp64 results: the exact value of the
sum up to fp64 rounding (the GPU's accumulation order is free, so its outputs are
compared within a tolerance). The INT8 reference is bit-exact: its accumulation is an
exact integer and its epilogue order is fixed (reading: two separately rounded fp32
products, left to right as written on [P-FP8INT8], then round-to-nearest-even bf16).
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, e2m1_decode, e8m0_decode, unpack_e2m1, f64_to_bf16_rne


def gemm_fp8_ref(xq, sx, wq, sw) -> np.ndarray:
    """y[m,n] = s_x[m] * s_w[n] * sum_k dec(xq[m,k]) * dec(wq[n,k]), in fp64.

    The contraction over decoded codes is one fp64 matrix product (each product of two
    E4M3 values is exact in fp64); the scales are applied after it.
    """
    a = e4m3_decode(xq)
    b = e4m3_decode(wq)
    acc = a @ b.T
    return acc * np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]


def gemm_fp8_bruteforce(xq, sx, wq, sw) -> np.ndarray:
    """Same as ``gemm_fp8_ref`` with explicit loops (for tiny shapes only)."""
    xq = np.asarray(xq); wq = np.asarray(wq)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(e4m3_decode(xq[m, k])) * float(e4m3_decode(wq[n, k]))
            y[m, n] = float(sx[m]) * float(sw[n]) * acc
    return y


def gemm_int8_acc(xq, wq) -> np.ndarray:
    """Exact INT32 accumulator acc[m,n] = sum_k xq[m,k] * wq[n,k].

    Computed as an fp64 matrix product of the integer codes: every product and every
    partial sum is an integer of magnitude at most K * 127^2, below 2^53 for any K under
    5e11, so the fp64 sums are exact in any order and the result converts back exactly.
    """
    xq = np.asarray(xq)
    wq = np.asarray(wq)
    if xq.shape[-1] * 127 * 127 >= 2 ** 53:
        raise ValueError("K too large for an exact fp64 integer product")
    return (xq.astype(np.float64) @ wq.astype(np.float64).T).astype(np.int64)


def gemm_int8_acc_bruteforce(xq, wq) -> np.ndarray:
    """Same accumulator with int64 arithmetic only (slow; for pins on small shapes)."""
    return np.asarray(xq, np.int64) @ np.asarray(wq, np.int64).T


def int8_epilogue_bf16(acc, sx, sw) -> np.ndarray:
    """bf16 bits of fp32(fp32(fp32(acc) * s_x[m]) * s_w[n]) rounded half-to-even."""
    a32 = np.asarray(acc).astype(np.float32)
    t = (a32 * np.asarray(sx, np.float32)[:, None]).astype(np.float32)
    y = (t * np.asarray(sw, np.float32)[None, :]).astype(np.float32)
    return f64_to_bf16_rne(y.astype(np.float64))


def gemm_int8_ref(xq, sx, wq, sw) -> np.ndarray:
    """INT8 W8A8 output as bf16 bit patterns [M,N] (bit-exact contract)."""
    return int8_epilogue_bf16(gemm_int8_acc(xq, wq), sx, sw)


def gemm_blockscaled_ref(xq, sx, wq, sw, group: int = 128) -> np.ndarray:
    """y = sum_g s_x[m,g] * s_w[n // group, g] * (sum_{k in g} dec * dec), in fp64.

    sx: [M, K/group]; sw: [ceil(N/group), K/group].
    """
    a = e4m3_decode(xq)
    b = e4m3_decode(wq)
    M, K = a.shape
    N = b.shape[0]
    G = K // group
    sx = np.asarray(sx, np.float64)
    sw = np.asarray(sw, np.float64)
    y = np.zeros((M, N))
    sw_rows = sw[np.arange(N) // group]                  # [N, G]
    for g in range(G):
        part = a[:, g * group:(g + 1) * group] @ b[:, g * group:(g + 1) * group].T
        y += part * sx[:, g][:, None] * sw_rows[:, g][None, :]
    return y


def gemm_mxfp4_ref(xq_packed, sx_e8m0, wq_packed, sw_e8m0) -> np.ndarray:
    """y = sum_blk 2^(e_x) 2^(e_w) sum_{k in blk} dec4 * dec4, in fp64.

    Every term is exact in fp64; the sum is exact while the terms' binades span fewer
    than 53 bits, which holds for the synthetic MXFP4 workloads.
    """
    a = e2m1_decode(unpack_e2m1(xq_packed))
    b = e2m1_decode(unpack_e2m1(wq_packed))
    M, K = a.shape
    sa = np.repeat(e8m0_decode(sx_e8m0), 32, axis=1)     # [M, K]
    sb = np.repeat(e8m0_decode(sw_e8m0), 32, axis=1)     # [N, K]
    return (a * sa) @ (b * sb).T


def within_tolerance(y, y_ref, rel: float = 1e-2):
    """Element-wise |y - y_ref| <= rel * (|y_ref| + rms(y_ref)); rms over the whole matrix.

    Returns (ok, worst_ratio) where worst_ratio is max |y - y_ref| / bound.
    """
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    bound = rel * (np.abs(y_ref) + rms)
    err = np.abs(y - y_ref)
    if y.size == 0:
        return True, 0.0
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    worst = float(np.max(ratio))
    return bool(worst <= 1.0), worst
