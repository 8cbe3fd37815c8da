"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the bench.

This module holds input generation only: random draws and their rounding to bfloat16.
None of the quantization or GEMM arithmetic lives here, and it imports neither the
oracle nor the HIP library.

Workloads (the pages quote an 8B model and a DeepSeek-V3-style block-scaled recipe but
ship no data; these draws stand in for them):

* ``tiny``      X 16x256 ~ N(0,1) with 4 outlier channels x100, W 128x256 ~ N(0, 0.02^2).
* ``prefill``   8B-style prefill linears at M=2048 tokens:
                (K,N) in {(4096,6144) QKV, (4096,4096) O, (4096,28672) gate+up,
                (14336,4096) down}; X ~ N(0,1) with round(0.001 K) outlier channels, each
                scaled by a log-uniform factor in [50, 500] for every token (outliers are
                systematic per channel); W ~ N(0, 0.02^2).
* ``decode``    M in {1,8,32,128,512} (the first M rows of one 512-row draw of the
                prefill X generator), K=4096, N in {4096, 14336}; a separate 512-token
                calibration draw with the same outlier channels feeds SmoothQuant.
* ``blockscaled`` M=4096, K=7168, N=18432; X i.i.d. Student-t (nu = 3); W ~ N(0, 0.02^2).
* ``mxfp4``     M=N=K=8192; X ~ N(0,1) times 2^u per (row, 32-element block),
                u ~ U(-8, 8); W ~ N(0, 0.02^2).
* ``random_bytes`` raw uniform bytes (seeded like the rest, workload index 9), shaped into
                operand codes by the tests at the library's largest operand size.

Seeds: workload index c (tiny 1, prefill 2, decode 3, blockscaled 4, mxfp4 5, largest
operands 9) and shape index i give base = 1000 c + 100 i; X uses base+1, W base+2,
outlier channels base+3, the calibration draw base+4. Draws are fp64 from
``numpy.random.default_rng`` (PCG64), rounded to fp32 and then to bfloat16 with
round-to-nearest-even.
"""

from __future__ import annotations

import numpy as np

PREFILL_SHAPES = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 28672), ("down", 14336, 4096)]
PREFILL_M = 2048
DECODE_MS = [1, 8, 32, 128, 512]
DECODE_NS = [4096, 14336]
DECODE_K = 4096
BLOCKSCALED_SHAPE = (4096, 7168, 18432)   # M, K, N
MXFP4_SHAPE = (8192, 8192, 8192)          # M, K, N


def seed(workload: int, shape_index: int, role: int) -> int:
    return 1000 * workload + 100 * shape_index + role


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bfloat16 bits (uint16), round to nearest even; NaN kept quiet."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(K: int, count: int, s: int) -> tuple[np.ndarray, np.ndarray]:
    """`count` distinct channels and their log-uniform factors in [50, 500]."""
    rng = np.random.default_rng(s)
    ch = rng.choice(K, size=count, replace=False)
    fac = np.exp(rng.uniform(np.log(50.0), np.log(500.0), size=count))
    return ch, fac


def gaussian_weights(N: int, K: int, s: int, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(s)
    return to_bf16_bits(rng.standard_normal((N, K)) * std)


def activations_with_outliers(M: int, K: int, s_x: int, s_out: int) -> np.ndarray:
    rng = np.random.default_rng(s_x)
    x = rng.standard_normal((M, K))
    ch, fac = outlier_channels(K, max(1, int(round(0.001 * K))), s_out)
    x[:, ch] *= fac[None, :]
    return to_bf16_bits(x)


# ----------------------------------------------------------------------------- workloads
def tiny():
    """(X [16,256], W [128,256]) bf16 bits."""
    rng = np.random.default_rng(seed(1, 0, 1))
    x = rng.standard_normal((16, 256))
    ch = np.random.default_rng(seed(1, 0, 3)).choice(256, size=4, replace=False)
    x[:, ch] *= 100.0
    return to_bf16_bits(x), gaussian_weights(128, 256, seed(1, 0, 2))


def prefill(i: int, M: int = PREFILL_M, n_limit: int | None = None):
    """Shape i of the 8B prefill set -> (name, X [M,K], W [N,K]); n_limit trims N."""
    name, K, N = PREFILL_SHAPES[i]
    x = activations_with_outliers(M, K, seed(2, i, 1), seed(2, i, 3))
    n = N if n_limit is None else min(N, n_limit)
    w = gaussian_weights(n, K, seed(2, i, 2))
    return name, x, w


def decode_x(K: int = DECODE_K) -> np.ndarray:
    """512-row draw; decode size M uses its first M rows."""
    return activations_with_outliers(512, K, seed(3, 0, 1), seed(3, 0, 3))


def decode_calibration(K: int = DECODE_K) -> np.ndarray:
    """Separate 512-token draw with the same outlier channels (for SmoothQuant maxima)."""
    return activations_with_outliers(512, K, seed(3, 0, 4), seed(3, 0, 3))


def decode_w(N: int, K: int = DECODE_K) -> np.ndarray:
    return gaussian_weights(N, K, seed(3, DECODE_NS.index(N) if N in DECODE_NS else 9, 2))


def blockscaled(M: int = BLOCKSCALED_SHAPE[0], K: int = BLOCKSCALED_SHAPE[1],
                N: int = BLOCKSCALED_SHAPE[2]):
    rng = np.random.default_rng(seed(4, 0, 1))
    x = to_bf16_bits(rng.standard_t(3.0, size=(M, K)))
    return x, gaussian_weights(N, K, seed(4, 0, 2))


def mxfp4_x(M: int, K: int) -> np.ndarray:
    rng = np.random.default_rng(seed(5, 0, 1))
    x = rng.standard_normal((M, K))
    u = rng.uniform(-8.0, 8.0, size=(M, K // 32))
    x *= np.repeat(np.exp2(u), 32, axis=1)
    return to_bf16_bits(x)


def mxfp4(M: int = MXFP4_SHAPE[0], K: int = MXFP4_SHAPE[1], N: int = MXFP4_SHAPE[2]):
    return mxfp4_x(M, K), gaussian_weights(N, K, seed(5, 0, 2))


def random_bf16(shape, s: int, scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) bf16 draw for edge-case tests."""
    return to_bf16_bits(np.random.default_rng(s).standard_normal(shape) * scale)


def random_bytes(n: int, s: int) -> np.ndarray:
    """n uniform random bytes (writable uint8), for operand codes too large to build by
    quantizing a bf16 draw (the largest operand the library accepts is 2^31 bytes)."""
    return np.random.default_rng(s).integers(0, 256, size=n, dtype=np.uint8)
