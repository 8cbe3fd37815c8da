"""Roofline arithmetic for a linear layer, as the pages model it.

Test infrastructure only (see ``oracle/__init__.py``).

Sources:
* A layer with P weights serving B tokens does 2PB FLOPs and reads at least P*b_w/8
  bytes of weights; with bandwidth beta and peak pi the step time is bounded below by the
  larger of the two times: [P-FP8FP4] "The bottleneck". The page's displayed formula is
  lost; this reading reproduces all five bounds the page prints for an 8B model.
* Weight-traffic-only decode model, operational intensity I = 2PB / bytes, ridge
  I_ridge = peak / bandwidth, crossover B* = pi_16 / (2 beta): [P-LOWBIT] §5.1-5.4.
* Metadata overheads of per-channel INT8 and grouped INT4 scales: [P-LOWBIT] §2.3 and
  Try-it 03.
"""

from __future__ import annotations


def step_time_lower_bound(P: float, B: float, bits_w: float, beta: float, pi: float) -> float:
    """max(P * bits_w / 8 / beta, 2 * P * B / pi) in seconds."""
    return max(P * bits_w / 8.0 / beta, 2.0 * P * B / pi)


def ridge_point(pi: float, beta: float) -> float:
    """FLOP per byte where a kernel stops being bandwidth-bound."""
    return pi / beta


def intensity_w8a8(B: float) -> float:
    """I = 2PB / (1.0 P) bytes of 8-bit weights."""
    return 2.0 * B


def intensity_w4a16(B: float, eta: float) -> float:
    """I = 2PB / (0.5 P (1 + eta))."""
    return 4.0 * B / (1.0 + eta)


def crossover_batch(pi16: float, beta: float) -> float:
    """Batch where bandwidth-bound 8-bit weights reach the 16-bit compute ceiling."""
    return pi16 / (2.0 * beta)


def scale_overhead_bytes(rows: int, cols: int, group: int | None, scale_bytes: int) -> int:
    """Bytes of scales: one per row (group None) or one per `group` elements."""
    if group is None:
        return rows * scale_bytes
    return rows * cols // group * scale_bytes


def gemm_flops(M: int, N: int, K: int) -> float:
    return 2.0 * M * N * K
