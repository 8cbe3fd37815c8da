"""GPU parity: W4A16 (symmetric INT4, one fp16 scale per 128 along K) quantization bit for
bit, and the weight-only GEMM within |y - y_ref| <= 1e-2 (|y_ref| + rms(y_ref)), against the
oracle."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import gemm as G
from oracle import w4a16 as W
from tests.gpu_util import bf16_to_f64, bits_u8, first_mismatch, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def _f16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_quant(wb, q, s, what):
    oq, os_ = W.quantize_int4_groups(wb)
    assert np.array_equal(_f16_bits(s), os_.view(np.uint16)), f"{what}: scales {first_mismatch(_f16_bits(s), os_.view(np.uint16))}"
    assert np.array_equal(bits_u8(q), oq), f"{what}: codes {first_mismatch(bits_u8(q), oq)}"


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (300, 1024), (4096, 4096)])
def test_quantize_int4(N, K):
    need_gpu()
    rng = np.random.default_rng(N + K)
    wb = _bf16(rng.standard_normal((N, K)) * 0.02 * np.exp2(rng.uniform(-6, 6, (N, 1))))
    q, s = w8.quantize_int4(to_dev_bf16(wb))
    torch.cuda.synchronize()
    _check_quant(wb, q, s, f"{N}x{K}")


def test_quantize_int4_special_groups():
    need_gpu()
    v = np.zeros((3, 512))
    v[0, 128:256] = 1e6                      # fp16 scale saturates at 65504
    v[1, :128] = [7.0, -3.5, 1.75, 0.5, -0.75, 2.5, -7.0] + [0.0] * 121
    v[1, 128:256] = 1e-30                    # scale underflows fp16 -> 0 -> 1
    v[2] = np.random.default_rng(2).standard_normal(512) * 3e4
    v[2, 300] = -0.0
    wb = _bf16(v)
    q, s = w8.quantize_int4(to_dev_bf16(wb))
    torch.cuda.synchronize()
    _check_quant(wb, q, s, "special groups")


def _gemm_compare(xb, wb, what):
    q, s = w8.quantize_int4(to_dev_bf16(wb))
    y = w8.gemm_w4a16(to_dev_bf16(xb), q, s)
    torch.cuda.synchronize()
    oq, os_ = W.quantize_int4_groups(wb)
    assert np.array_equal(bits_u8(q), oq) and np.array_equal(_f16_bits(s), os_.view(np.uint16))
    ok, worst = G.within_tolerance(bf16_to_f64(y), W.gemm_w4a16_ref(xb, oq, os_), TOL)
    assert ok, f"{what}: worst error / bound = {worst:.3f}"


# every 16-row subtile edge, M above 128 (slices), N not a multiple of 4 or 16, one group;
# K a multiple of 1024 above 32 tokens (16 above 8192 outputs) takes the LDS-staged kernel:
# each of its launch shapes (32, 64 or 128 token rows x 16, 32 or 64 weight rows), one to
# three rows of workgroups, ragged M and N
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (5, 7, 256), (16, 130, 384), (17, 64, 1024),
                                   (33, 300, 512), (64, 4099, 256), (100, 96, 2048), (128, 257, 640),
                                   (129, 33, 256), (300, 200, 384), (2, 9000, 1152),
                                   (100, 1001, 2048), (129, 77, 1024), (300, 4100, 1024),
                                   (48, 20000, 1024), (200, 3001, 1024), (1, 4096, 1024),
                                   (16, 4096, 2048), (257, 9000, 3072), (17, 20000, 1024),
                                   (17, 9000, 1024), (33, 4100, 1024), (33, 9000, 1024),
                                   (65, 7000, 1024), (32, 4096, 1024)])
def test_gemm_w4a16_ragged(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M * 13 + N * 3 + K)
    xb = _bf16(rng.standard_normal((M, K)))
    wb = _bf16(rng.standard_normal((N, K)) * 0.02)
    _gemm_compare(xb, wb, f"{M}x{N}x{K}")


# one token with K a multiple of 2048 up to 16384 takes the whole-row GEMV: one to eight
# kilobyte loads per row, N below, at and above one row per wave of the grid (1024
# workgroups of 4 waves), N = 1; two tokens and K = 18432 take the tile kernel beside it
@pytest.mark.parametrize("M,N,K", [(1, 1, 2048), (1, 4099, 4096), (1, 5, 6144), (1, 1001, 10240),
                                   (1, 257, 16384), (1, 9000, 8192), (1, 4096, 14336), (2, 300, 4096),
                                   (1, 130, 18432), (1, 12000, 2048)])
def test_gemm_w4a16_gemv(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M * 7 + N * 5 + K)
    xb = _bf16(rng.standard_normal((M, K)))
    wb = _bf16(rng.standard_normal((N, K)) * 0.02)
    _gemm_compare(xb, wb, f"gemv {M}x{N}x{K}")


# 2-128 tokens with K a multiple of 512 take the narrow-tile kernel where one round of tiles
# covers the output: 16 x 32 tiles (2-16 tokens above 8192 outputs, with 8 staged rows of X up
# to 8 tokens; 17-32 up to 8192; 33-64 up to 4096), 16 x 16 tiles (2-16 tokens on 4097-8192
# outputs, 8 staged rows of X up to 8 tokens; 17-32 tokens up to 4096 outputs; groups split
# over 4 waves) and 32 x 64 tiles (17-32 tokens up to 16384; 65-128 up to
# 4096); ragged M and N, one stage (K = 512, fewer stages than the ring holds) up to many
@pytest.mark.parametrize("M,N,K", [(2, 8193, 512), (5, 9000, 1536), (8, 14336, 4096), (7, 16000, 2048),
                                   (9, 8200, 512), (12, 9001, 2048), (16, 16384, 1536), (17, 100, 512),
                                   (20, 4099, 1536), (32, 4096, 4096), (24, 6144, 1024), (31, 8191, 512),
                                   (25, 9000, 1536), (32, 14336, 2048), (33, 4096, 512), (64, 4090, 1536),
                                   (50, 300, 4096), (65, 4096, 1024), (128, 4100, 512), (100, 2000, 2048),
                                   (2, 4097, 512), (5, 6144, 1536), (8, 8192, 4096), (12, 8000, 1024), (16, 5000, 2048)])
def test_gemm_w4a16_narrow(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M * 11 + N * 7 + K)
    xb = _bf16(rng.standard_normal((M, K)))
    wb = _bf16(rng.standard_normal((N, K)) * 0.02)
    _gemm_compare(xb, wb, f"narrow {M}x{N}x{K}")


@pytest.mark.parametrize("N", synthetic.DECODE_NS)
def test_gemm_w4a16_decode_sweep(N):
    """The decode sweep's shapes (M in 1, 8, 32, 128; K = 4096) on its activations."""
    need_gpu()
    x_all = synthetic.decode_x()
    wb = synthetic.decode_w(N)
    q, s = w8.quantize_int4(to_dev_bf16(wb))
    oq, os_ = W.quantize_int4_groups(wb)
    torch.cuda.synchronize()
    assert np.array_equal(bits_u8(q), oq) and np.array_equal(_f16_bits(s), os_.view(np.uint16))
    for M in (1, 8, 32, 128):
        xb = x_all[:M]
        y = w8.gemm_w4a16(to_dev_bf16(xb), q, s)
        torch.cuda.synchronize()
        ok, worst = G.within_tolerance(bf16_to_f64(y), W.gemm_w4a16_ref(xb, oq, os_), TOL)
        assert ok, f"M={M} N={N}: worst error / bound = {worst:.3f}"
