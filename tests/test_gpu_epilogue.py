"""GPU parity of the extended epilogue (w8a8_gemm_ex): bias, ReLU / SiLU, bf16 or FP8 output.

INT8 operands with no activation or ReLU: bf16 bits and E4M3FN codes bit for bit.
FP8 operands, and SiLU: within |y - y_ref| <= 1e-2 (|y_ref| + rms(y_ref)) of the oracle's
exact value; an FP8 output code additionally may sit one E4M3 spacing from the exact
quotient (the rounding of a value that is itself within the tolerance).
"""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import epilogue as E
from oracle import quant as Q
from oracle.formats import bf16_to_f64, e4m3_decode
from tests.gpu_util import bf16_bits, bits_u8, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

TOL = 1e-2

# the prefill kernels (ragged and 16-aligned N), every narrow tile (16 x 16 with K split over
# 4 waves, 16 x 32, 16 x 64, 32 x 64, and the 8-wave 64-, 96- and 128-row tiles above 64 tokens,
# one and several row tiles) and the one-token vector kernel (its epilogue runs in one lane
# per output)
SHAPES = [(1100, 4100, 256), (2048, 4096, 128), (600, 549, 256), (256, 512, 384), (5, 130, 1152), (64, 10000, 256), (100, 262, 512),
          (128, 9001, 256), (200, 9001, 384), (300, 549, 256), (448, 2050, 256),
          (300, 6100, 384), (100, 20001, 256), (48, 40000, 128), (40, 4100, 256),
          (16, 6144, 512), (300, 4096, 384), (1, 4100, 2048), (1, 77, 14336)]


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    ch = rng.choice(K, size=max(1, K // 1000), replace=False)
    x[:, ch] *= rng.uniform(50, 500, size=len(ch))
    w = rng.standard_normal((N, K)) * 0.02
    return synthetic.to_bf16_bits(x), synthetic.to_bf16_bits(w)


def _rms(v):
    return float(np.sqrt(np.mean(np.square(v))))


def _check_values(y, ref, what):
    bound = TOL * (np.abs(ref) + _rms(ref))
    err = np.abs(y - ref)
    assert np.all(err <= bound), f"{what}: worst error / bound = {np.max(err / bound):.3f}"


def _check_fp8_codes(codes, z_ref, what):
    dec = e4m3_decode(codes)
    assert not np.any(np.isnan(dec)), f"{what}: NaN code"
    tol = TOL * (np.abs(z_ref) + _rms(z_ref))
    bound = E.e4m3_spacing(np.minimum(np.abs(z_ref) * (1 + TOL) + tol, 448.0)) + tol
    err = np.abs(dec - z_ref)
    assert np.all(err <= bound), f"{what}: worst error / bound = {np.max(err / bound):.3f}"


def _setup(fmt, M, N, K, seed):
    xb, wb = _inputs(M, N, K, seed)
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    xq, sx = w8.quantize_per_token(x, fmt)
    wq, sw = w8.quantize_weight_per_channel(w, fmt)
    torch.cuda.synchronize()
    if fmt == "int8":
        oxq, osx = Q.quantize_per_token_int8(xb)
        owq, osw = Q.quantize_weight_per_channel_int8(wb)
        assert np.array_equal(xq.view(torch.uint8).cpu().numpy().view(np.int8), oxq)
    else:
        oxq, osx = Q.quantize_per_token_fp8(xb)
        owq, osw = Q.quantize_weight_per_channel_fp8(wb)
        assert np.array_equal(bits_u8(xq), oxq)
    return (xq, sx, wq, sw), (oxq, osx, owq, osw)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
def test_bias_activation_bf16_out(M, N, K, fmt):
    need_gpu()
    dev, ora = _setup(fmt, M, N, K, M + 3 * N + 7 * K)
    plain = (E.int8_path_values(*ora) if fmt == "int8" else E.fp8_path_ref(*ora)).astype(np.float64)
    bias_bits = synthetic.to_bf16_bits(np.random.default_rng(N).standard_normal(N) * _rms(plain))
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).to(dev[0].device)
    for use_bias in (False, True):
        for act in ("none", "relu", "silu"):
            b = bias if use_bias else None
            bb = bias_bits if use_bias else None
            y = w8.gemm_ex(*dev, bias=b, act=act)
            torch.cuda.synchronize()
            what = f"{fmt} {M}x{N}x{K} bias={use_bias} act={act}"
            if fmt == "int8" and act != "silu":
                ref = E.int8_path_ref(*ora, bias_bits=bb, act=act)
                assert np.array_equal(bf16_bits(y), ref), what
            elif fmt == "int8":
                ref = E.int8_path_values(*ora, bias_bits=bb, act=act).astype(np.float64)
                _check_values(bf16_to_f64(bf16_bits(y)), ref, what)
            else:
                ref = E.fp8_path_ref(*ora, bias_bits=bb, act=act)
                _check_values(bf16_to_f64(bf16_bits(y)), ref, what)


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
def test_fp8_requantized_out(M, N, K, fmt):
    need_gpu()
    dev, ora = _setup(fmt, M, N, K, 2 * M + N + K)
    plain = (E.int8_path_values(*ora) if fmt == "int8" else E.fp8_path_ref(*ora)).astype(np.float64)
    amax = float(np.max(np.abs(plain)))
    bias_bits = synthetic.to_bf16_bits(np.random.default_rng(M).standard_normal(N) * _rms(plain))
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).to(dev[0].device)
    # a scale that fits the range, and one that saturates the largest outputs
    for s_out in (np.float32(amax / 300.0), np.float32(amax / 2000.0)):
        for act in ("none", "relu", "silu"):
            y = w8.gemm_ex(*dev, bias=bias, act=act, out_scale=float(s_out))
            torch.cuda.synchronize()
            codes = bits_u8(y)
            what = f"{fmt} {M}x{N}x{K} s_out={s_out:.3g} act={act}"
            if fmt == "int8" and act != "silu":
                ref = E.int8_path_ref(*ora, bias_bits=bias_bits, act=act, s_out=s_out)
                assert np.array_equal(codes, ref), what
            elif fmt == "int8":
                v = E.int8_path_values(*ora, bias_bits=bias_bits, act=act).astype(np.float64)
                _check_fp8_codes(codes, np.clip(v / float(s_out), -448, 448), what)
            else:
                z = E.fp8_path_ref(*ora, bias_bits=bias_bits, act=act, s_out=float(s_out))
                _check_fp8_codes(codes, z, what)


# The 224-wide tile, which the dispatcher picks for 2048-token layers of about 28672
# outputs (gate+up): ragged rows and columns, the plain GEMM, bias with SiLU, and FP8
# outputs, compared on sampled rows that include the first, last and tile-edge rows.
WIDE_SHAPES = [(1999, 28001, 256), (2048, 28016, 128)]


@pytest.mark.parametrize("M,N,K", WIDE_SHAPES)
def test_wide_tile_sampled(M, N, K):
    need_gpu()
    dev, ora = _setup("e4m3fn", M, N, K, M + N + K)
    rng = np.random.default_rng(M * N)
    rows = np.unique(np.r_[0, 1, 255, 256, 257, 1023, 1024, M - 257, M - 256, M - 1,
                           rng.choice(M, 22, replace=False)])
    ors = (ora[0][rows], ora[1][rows], ora[2], ora[3])
    plain = E.fp8_path_ref(*ors).astype(np.float64)
    bias_bits = synthetic.to_bf16_bits(rng.standard_normal(N) * _rms(plain))
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).to(dev[0].device)
    y = w8.gemm(*dev)
    torch.cuda.synchronize()
    _check_values(bf16_to_f64(bf16_bits(y)[rows]), plain, f"{M}x{N}x{K} plain")
    y = w8.gemm_ex(*dev, bias=bias, act="silu")
    torch.cuda.synchronize()
    _check_values(bf16_to_f64(bf16_bits(y)[rows]), E.fp8_path_ref(*ors, bias_bits=bias_bits, act="silu"),
                  f"{M}x{N}x{K} bias silu")
    s_out = float(np.float32(np.max(np.abs(plain)) / 300.0))
    for act, b, bb in (("none", None, None), ("relu", bias, bias_bits)):
        y = w8.gemm_ex(*dev, bias=b, act=act, out_scale=s_out)
        torch.cuda.synchronize()
        _check_fp8_codes(bits_u8(y)[rows], E.fp8_path_ref(*ors, bias_bits=bb, act=act, s_out=s_out),
                         f"{M}x{N}x{K} fp8 out act={act}")


# INT8 layers of about 6000 outputs at 2048 tokens take 192-wide tiles (one wave of 256
# workgroups instead of 1.5): bias and ReLU with bf16 and FP8 outputs bit for bit, SiLU
# within the tolerance, on sampled rows including the first, last and tile-edge rows.
@pytest.mark.parametrize("M,N,K", [(1999, 6001, 384), (2048, 6144, 256)])
def test_int8_wide_tile_sampled(M, N, K):
    need_gpu()
    dev, ora = _setup("int8", M, N, K, 3 * M + N + K)
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.r_[0, 1, 255, 256, 257, 1023, 1024, M - 257, M - 256, M - 1,
                           rng.choice(M, 22, replace=False)])
    ors = (ora[0][rows], ora[1][rows], ora[2], ora[3])
    plain = E.int8_path_values(*ors).astype(np.float64)
    bias_bits = synthetic.to_bf16_bits(rng.standard_normal(N) * _rms(plain))
    bias = torch.from_numpy(bias_bits.view(np.int16)).view(torch.bfloat16).to(dev[0].device)
    y = w8.gemm_ex(*dev, bias=bias, act="relu")
    torch.cuda.synchronize()
    ref = E.int8_path_ref(*ors, bias_bits=bias_bits, act="relu")
    assert np.array_equal(bf16_bits(y)[rows], ref), f"int8 {M}x{N}x{K} bias relu"
    y = w8.gemm_ex(*dev, bias=bias, act="silu")
    torch.cuda.synchronize()
    _check_values(bf16_to_f64(bf16_bits(y)[rows]),
                  E.int8_path_values(*ors, bias_bits=bias_bits, act="silu").astype(np.float64),
                  f"int8 {M}x{N}x{K} bias silu")
    s_out = np.float32(np.max(np.abs(plain)) / 300.0)
    y = w8.gemm_ex(*dev, bias=bias, act="none", out_scale=float(s_out))
    torch.cuda.synchronize()
    ref = E.int8_path_ref(*ors, bias_bits=bias_bits, act="none", s_out=s_out)
    assert np.array_equal(bits_u8(y)[rows], ref), f"int8 {M}x{N}x{K} fp8 out"


def test_gemm_ex_options_off_equal_gemm():
    need_gpu()
    for fmt in ("e4m3fn", "int8"):
        for M, N, K in SHAPES:
            dev, _ = _setup(fmt, M, N, K, 5 * M + N)
            y0 = w8.gemm(*dev)
            y1 = w8.gemm_ex(*dev)
            torch.cuda.synchronize()
            assert np.array_equal(bf16_bits(y0), bf16_bits(y1)), f"{fmt} {M}x{N}x{K}"
