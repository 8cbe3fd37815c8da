"""Helpers for the GPU parity tests: numpy <-> torch device transfers of raw bit patterns."""

import numpy as np
import torch


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> contiguous bf16 tensor on cuda:0."""
    b = np.ascontiguousarray(np.asarray(bits, np.uint16))
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t if dtype is None else t.view(dtype)


def bits_u8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def bits_i8(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int8).cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    idx = np.argwhere(a != b)
    if len(idx) == 0:
        return "none"
    i = tuple(idx[0])
    return f"{len(idx)} mismatches, first at {i}: got {a[i]!r} expected {b[i]!r}"
