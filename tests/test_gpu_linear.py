"""GPU parity of w8a8_linear (per-token quantization and the scaled GEMM in one call; one
fused kernel for one token with K a multiple of 1024 up to 16384, the quantizer and the GEMM
otherwise): the codes and scales it writes bit for bit against the oracle's quantizer, the
output against the oracle's contraction (FP8 within |y - y_ref| <= 1e-2 (|y_ref| + rms(y_ref)),
INT8 bit for bit), and the output bit-identical to the library's quantize + gemm on the same
inputs."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import gemm as G
from oracle import quant as Q
from tests.gpu_util import bf16_bits, bf16_to_f64, bits_i8, bits_u8, f32, first_mismatch, need_gpu, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _xw(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    ch = rng.choice(K, size=max(1, K // 1000), replace=False)
    x[:, ch] *= rng.uniform(50, 500, size=len(ch))
    w = rng.standard_normal((N, K)) * 0.02
    return synthetic.to_bf16_bits(x), synthetic.to_bf16_bits(w)


# one token on the fused kernel (one to sixteen kilobytes of K, ragged N, N above one row per
# wave of the grid), and the two-kernel path: one token with K outside the fused kernel's
# range (not a multiple of 1024, above 16384), and 2-33 tokens on the narrow 16 x 16 and 16 x 32
# tiles and wider (ragged N, K from 1152 to 14336)
CASES = [(1, 4096, 4096), (1, 4100, 1024), (1, 77, 14336), (1, 20000, 16384), (1, 300, 640),
         (1, 5, 17408), (5, 4096, 4096), (2, 4096, 2048), (16, 4096, 4096), (8, 14336, 4096),
         (3, 4100, 4096), (16, 300, 2048), (9, 10000, 2048), (8, 4096, 1536), (4, 1000, 14336),
         (2, 20000, 4096), (33, 700, 1152)]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", CASES)
def test_linear(M, N, K, fmt):
    need_gpu()
    xb, wb = _xw(M, N, K, 5 * M + 3 * N + K)
    if fmt == "int8":
        oxq, osx = Q.quantize_per_token_int8(xb)
        owq, osw = Q.quantize_weight_per_channel_int8(wb)
        dt = torch.int8
    else:
        oxq, osx = Q.quantize_per_token_fp8(xb)
        owq, osw = Q.quantize_weight_per_channel_fp8(wb)
        dt = torch.float8_e4m3fn
    wq, sw = to_dev(owq, dt), to_dev(osw)
    y, xq, sx = w8.linear(to_dev_bf16(xb), wq, sw, return_codes=True)
    torch.cuda.synchronize()
    got = bits_i8(xq) if fmt == "int8" else bits_u8(xq)
    assert np.array_equal(got, oxq), first_mismatch(got, oxq)
    assert np.array_equal(f32(sx).view(np.uint32), osx.view(np.uint32))
    what = f"{fmt} {M}x{N}x{K}"
    if fmt == "int8":
        exp = np.asarray(G.gemm_int8_ref(oxq, osx, owq, osw), np.uint16)
        assert np.array_equal(bf16_bits(y), exp), what
    else:
        ok, worst = G.within_tolerance(bf16_to_f64(y), G.gemm_fp8_ref(oxq, osx, owq, osw), TOL)
        assert ok, f"{what}: worst error / bound = {worst:.3f}"
    y2 = w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), what


def test_linear_one_token_non_finite():
    """The fused kernel quantizes a row holding NaN and infinity as the quantizer does (same
    codes, infinite scale), and its output equals the GEMM's on those codes bit for bit."""
    need_gpu()
    xb, wb = _xw(1, 600, 4096, 11)
    x = synthetic.bf16_bits_to_f32(xb).astype(np.float64)
    x[0, 17] = np.nan
    x[0, 900] = np.inf
    xb = synthetic.to_bf16_bits(x)
    owq, osw = Q.quantize_weight_per_channel_fp8(wb)
    wq, sw = to_dev(owq, torch.float8_e4m3fn), to_dev(osw)
    xd = to_dev_bf16(xb)
    y, xq, sx = w8.linear(xd, wq, sw, return_codes=True)
    q2, s2 = w8.quantize_per_token(xd)
    y2 = w8.gemm(q2, s2, wq, sw)
    torch.cuda.synchronize()
    assert np.array_equal(bits_u8(xq), bits_u8(q2))
    assert np.array_equal(f32(sx).view(np.uint32), f32(s2).view(np.uint32)) and np.isinf(f32(sx)[0])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_linear_few_tokens_non_finite():
    """A few tokens with NaN and infinity: the same codes and scales as the quantizer (an
    infinite scale on the row holding the infinity), and the GEMM's output on those codes."""
    need_gpu()
    xb, wb = _xw(6, 5000, 4096, 13)
    x = synthetic.bf16_bits_to_f32(xb).astype(np.float64)
    x[1, 33] = np.nan
    x[4, 2000] = -np.inf
    xb = synthetic.to_bf16_bits(x)
    for fmt, dt in (("e4m3fn", torch.float8_e4m3fn), ("int8", torch.int8)):
        if fmt == "int8":
            owq, osw = Q.quantize_weight_per_channel_int8(wb)
        else:
            owq, osw = Q.quantize_weight_per_channel_fp8(wb)
        wq, sw = to_dev(owq, dt), to_dev(osw)
        xd = to_dev_bf16(xb)
        y, xq, sx = w8.linear(xd, wq, sw, return_codes=True)
        q2, s2 = w8.quantize_per_token(xd, fmt)
        y2 = w8.gemm(q2, s2, wq, sw)
        torch.cuda.synchronize()
        bits = bits_i8 if fmt == "int8" else bits_u8
        assert np.array_equal(bits(xq), bits(q2)), fmt
        assert np.array_equal(f32(sx).view(np.uint32), f32(s2).view(np.uint32)), fmt
        assert np.isinf(f32(sx)[4]) and np.isfinite(f32(sx)[0]), fmt
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), fmt


def test_linear_repeat_identical_and_empty():
    need_gpu()
    xb, wb = _xw(1, 14336, 4096, 3)
    owq, osw = Q.quantize_weight_per_channel_fp8(wb)
    wq, sw = to_dev(owq, torch.float8_e4m3fn), to_dev(osw)
    xd = to_dev_bf16(xb)
    y0 = w8.linear(xd, wq, sw)
    torch.cuda.synchronize()
    ref = y0.clone()
    for r in range(6):
        w8.linear(xd, wq, sw, out=y0)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), ref.view(torch.int16)), f"run {r + 1} differs"
    e = w8.linear(torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda:0"), wq, sw)
    assert e.shape == (0, 14336)
