"""GPU parity of the narrow-tile GEMM (the kernel w8a8_gemm uses for two or more tokens wherever
one round of its tiles covers the output) against
the oracle: FP8 outputs within |y - y_ref| <= 1e-2 (|y_ref| + rms(y_ref)) of the oracle's fp64
contraction over the same codes, INT8 outputs bit for bit, repeated launches bit-identical;
and the shader-clock probe used by the measurements."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import gemm as G
from oracle import quant as Q
from tests.gpu_util import bf16_bits, bf16_to_f64, need_gpu, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _xw(M, N, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    ch = rng.choice(K, size=max(1, K // 1000), replace=False)
    x[:, ch] *= rng.uniform(50, 500, size=len(ch))
    w = rng.standard_normal((N, K)) * 0.02
    return synthetic.to_bf16_bits(x), synthetic.to_bf16_bits(w)


def _codes(xb, wb, fmt):
    if fmt == "int8":
        oxq, osx = Q.quantize_per_token_int8(xb)
        owq, osw = Q.quantize_weight_per_channel_int8(wb)
        dt = torch.int8
    else:
        oxq, osx = Q.quantize_per_token_fp8(xb)
        owq, osw = Q.quantize_weight_per_channel_fp8(wb)
        dt = torch.float8_e4m3fn
    return (oxq, osx, owq, osw), (to_dev(oxq, dt), to_dev(osx), to_dev(owq, dt), to_dev(osw))


def _check(y, o, fmt, what):
    if fmt == "int8":
        got, exp = bf16_bits(y), np.asarray(G.gemm_int8_ref(*o), np.uint16)
        assert np.array_equal(got, exp), f"{what}: {np.count_nonzero(got != exp)} outputs differ"
    else:
        ok, worst = G.within_tolerance(bf16_to_f64(y), G.gemm_fp8_ref(*o), TOL)
        assert ok, f"{what}: worst error / bound = {worst:.3f}"


# Every tile the kernel has: 16 x 16 (4-way K split over the waves), 16 x 32 (2-way),
# 16 x 64 and 32 x 64 on 256- and 512-byte stages, the 128-byte-step tiles (16 / 32 token
# rows x 64 / 128 weight rows), and the 8-wave 64 x 64, 64 x 128, 96 x 64, 128 x 64 and
# 128 x 128 tiles (above 128 tokens the smallest that fits one round of the CUs, at any token
# count: up to 4100 tokens on 200 outputs); ragged M and N (N not a multiple of 4 or 16);
# K a whole number of stages, and K ending in a partial stage (fewer K steps than a stage
# holds: one, or fewer than the waves splitting it), including K shorter than one stage;
# step counts below and above the ring depth; several row tiles (257-512 tokens); K = 14336.
CASES = [(1, 6144, 4096), (5, 4096, 4096), (16, 1000, 640), (9, 3000, 896), (12, 2048, 384),
         (16, 4100, 128), (7, 14336, 640), (3, 28672, 256), (17, 5000, 1152), (24, 4096, 896),
         (32, 14336, 384), (32, 20000, 256), (33, 6144, 512), (40, 4096, 4096), (64, 3000, 640),
         (48, 4096, 1408), (64, 4099, 2048), (50, 28672, 256), (100, 4096, 1152), (65, 8200, 640),
         (128, 14336, 1024), (100, 20000, 256), (128, 28672, 128), (256, 4096, 384), (300, 4101, 256),
         (512, 4096, 1152), (257, 6144, 128), (384, 4096, 14336), (16, 4096, 14336), (128, 4096, 14336),
         (100, 6144, 896), (80, 8192, 4096), (129, 4100, 640), (200, 6144, 1152), (255, 9000, 512),
         (384, 6144, 640), (511, 8190, 256), (250, 4000, 1408), (192, 2048, 4096),
         (300, 4096, 1152), (350, 3000, 896),
         (700, 1000, 640), (1030, 3000, 512), (2048, 1024, 256), (4100, 200, 384)]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("M,N,K", CASES)
def test_narrow_parity(M, N, K, fmt):
    need_gpu()
    xb, wb = _xw(M, N, K, 3 * M + 7 * N + K)
    o, d = _codes(xb, wb, fmt)
    y = w8.gemm(*d)
    torch.cuda.synchronize()
    _check(y, o, fmt, f"{fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (8, 4096, 4096), (32, 4096, 896), (64, 28672, 512),
                                   (128, 14336, 1024), (128, 4096, 4096), (512, 4096, 1024)])
def test_narrow_repeat_identical(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, M + N + K)
    o, d = _codes(xb, wb, "fp8")
    y0 = w8.gemm(*d)
    torch.cuda.synchronize()
    ref = y0.clone()
    for r in range(8):
        w8.gemm(*d, out=y0)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), ref.view(torch.int16)), f"{M}x{N}x{K}: run {r + 1} differs"
    _check(ref, o, "fp8", f"{M}x{N}x{K}")


@pytest.mark.parametrize("N", synthetic.DECODE_NS)
def test_decode_sweep_full_size(N):
    """The decode sweep's shapes in the bench's configuration (the first M rows of one
    512-token draw, K = 4096), whichever kernel takes them: FP8 within tolerance on every
    output, INT8 bit for bit on every output."""
    need_gpu()
    xall = synthetic.decode_x()
    wb = synthetic.decode_w(N)
    owq8, osw8 = Q.quantize_weight_per_channel_fp8(wb)
    owqi, oswi = Q.quantize_weight_per_channel_int8(wb)
    dw8 = (to_dev(owq8, torch.float8_e4m3fn), to_dev(osw8))
    dwi = (to_dev(owqi, torch.int8), to_dev(oswi))
    for M in synthetic.DECODE_MS:
        xb = xall[:M]
        oxq, osx = Q.quantize_per_token_fp8(xb)
        y = w8.gemm(to_dev(oxq, torch.float8_e4m3fn), to_dev(osx), *dw8)
        torch.cuda.synchronize()
        _check(y, (oxq, osx, owq8, osw8), "fp8", f"fp8 {M}x{N}")
        oxi, osi = Q.quantize_per_token_int8(xb)
        y = w8.gemm(to_dev(oxi, torch.int8), to_dev(osi), *dwi)
        torch.cuda.synchronize()
        _check(y, (oxi, osi, owqi, oswi), "int8", f"int8 {M}x{N}")


def test_sclk_probe_reads_a_plausible_clock():
    """The measurement helper: one-wave workgroups over a 2 ms window report about 2 ms of
    real-time ticks and a shader clock between 0.1 and 2.5 GHz."""
    need_gpu()
    out = torch.zeros((16,), dtype=torch.int64, device="cuda:0")
    st = w8.lib().w8a8_sclk_probe(out.data_ptr(), 8, 200000, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(8, 2).astype(np.float64)
    assert np.all(o[:, 0] >= 200000) and np.all(o[:, 0] < 400000), o
    ghz = o[:, 1] / o[:, 0] * 0.1
    assert np.all(ghz > 0.1) and np.all(ghz < 2.5), ghz


def test_stream_probe_writes_the_high_bytes():
    """The same-split stream kernel the quantizer is measured against: output byte i is the
    high byte of bf16 element i, over a ragged count of 16-byte chunks."""
    need_gpu()
    rng = np.random.default_rng(3)
    n = 8 * 12345
    bits = rng.integers(0, 65536, size=n, dtype=np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).to("cuda:0")
    y = torch.zeros((n,), dtype=torch.uint8, device="cuda:0")
    assert w8.lib().w8a8_stream_probe(x.data_ptr(), n, y.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), (bits >> 8).astype(np.uint8))
