"""GPU parity: the HIP GEMMs (FP8, INT8 + SmoothQuant, block-scaled FP8, MXFP4) against the
oracle. Codes, scales and INT8 outputs bit for bit; FP8 / FP4 outputs within
|y - y_ref| <= 1e-2 (|y_ref| + rms(y_ref)) of the oracle's fp64 contraction."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import gemm as G
from oracle import quant as Q
from oracle import smoothquant as S
from tests.gpu_util import (bf16_bits, bf16_to_f64, bits_i8, bits_u8, f32, first_mismatch,
                            need_gpu, to_dev_bf16)

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def _assert_tol(y_gpu, y_ref, what):
    ok, worst = G.within_tolerance(y_gpu, y_ref, TOL)
    assert ok, f"{what}: worst error / bound = {worst:.3f}"


def _xw(M, N, K, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    if outliers:
        ch = rng.choice(K, size=max(1, K // 1000), replace=False)
        x[:, ch] *= rng.uniform(50, 500, size=len(ch))
    w = rng.standard_normal((N, K)) * 0.02
    return _bf16(x), _bf16(w)


# ----------------------------------------------------------------------------- FP8
def _fp8_full_compare(xb, wb, what):
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    xq, sx = w8.quantize_per_token(x)
    wq, sw = w8.quantize_weight_per_channel(w)
    y = w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    oxq, osx = Q.quantize_per_token_fp8(xb)
    owq, osw = Q.quantize_weight_per_channel_fp8(wb)
    assert np.array_equal(bits_u8(xq), oxq) and np.array_equal(f32(sx), osx)
    assert np.array_equal(bits_u8(wq), owq) and np.array_equal(f32(sw), osw)
    _assert_tol(bf16_to_f64(y), G.gemm_fp8_ref(oxq, osx, owq, osw), what)


def test_fp8_tiny_config():
    need_gpu()
    x, w = synthetic.tiny()
    _fp8_full_compare(x, w, "tiny 16x128x256")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (17, 130, 384), (300, 549, 256), (3, 1000, 4096),
                                   (256, 256, 128), (513, 129, 1024), (260, 4100, 256), (1100, 4100, 512)])
def test_fp8_ragged(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, M * 31 + N * 7 + K)
    _fp8_full_compare(xb, wb, f"{M}x{N}x{K}")


# Few-token and mid-size paths (the narrow-tile kernel): every tile and several row tiles,
# every 16-row bucket edge, N not a multiple of 4 or 16, one K step and K ending in a partial
# stage, step counts below and above the ring depth, wide layers with a ragged last tile (up
# to 128 weight rows per tile), 513 tokens on 1000 outputs, and the prefill kernels where
# narrow tiles would take more than one round of the CUs (200 tokens on 20000 outputs, 400 on
# 7000, 1100 on 4100).
FEW_TOKEN_CASES = [(16, 33, 1152), (32, 7, 128), (33, 64, 640), (64, 4099, 256), (65, 100, 2048),
                (128, 130, 1152), (129, 257, 256), (2, 18, 14336), (16, 9000, 256),
                (32, 8200, 384), (64, 10000, 1152), (128, 8193, 640), (97, 8209, 128),
                (111, 4097, 2176), (128, 14336, 384), (200, 4100, 640), (256, 9000, 1152),
                (160, 6144, 512), (257, 300, 256), (100, 20000, 256), (400, 7000, 384),
                (90, 16500, 384), (128, 32768, 256), (128, 32769, 128), (200, 20000, 256),
                (513, 1000, 256), (1100, 4100, 256), (40, 4100, 512), (64, 40000, 256), (48, 33000, 128)]


# One token with K a multiple of 1024 up to 16384 takes the whole-row vector kernel: one to
# sixteen kilobyte loads per row, N below and above the grid's 4096 waves (several rows per
# wave), and beside it K = 17408 and K = 640 (the tiled kernels).
GEMV_CASES = [(1, 1, 1024), (1, 7, 3072), (1, 4097, 4096), (1, 14336, 4096), (1, 4096, 14336),
              (1, 300, 16384), (1, 9001, 2048), (1, 20000, 1024), (1, 130, 17408), (1, 500, 640)]


@pytest.mark.parametrize("M,N,K", GEMV_CASES)
def test_fp8_one_token(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, 17 * N + K)
    _fp8_full_compare(xb, wb, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", GEMV_CASES)
def test_int8_one_token(M, N, K):
    """INT8 sums are exact in any order: bit-exact against the oracle's chain."""
    need_gpu()
    xb, wb = _xw(M, N, K, 19 * N + K)
    xcal, _ = _xw(64, 1, K, K + 3)
    _int8_chain(xb, xcal, wb, 0.5, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", FEW_TOKEN_CASES)
def test_fp8_few_tokens(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, 11 * M + 5 * N + K)
    _fp8_full_compare(xb, wb, f"{M}x{N}x{K}")


# Regression: the two-waves-per-SIMD kernel refills an LDS stage while other waves of the
# workgroup compute. A refill that starts before every wave has read the stage changes
# results from run to run, so the same launch is repeated and must give identical bits.
@pytest.mark.parametrize("M,N,K", [(256, 8193, 640), (2048, 4096, 1024), (512, 6144, 4096),
                                   (2048, 28672, 512), (128, 4096, 4096), (100, 14336, 1024),
                                   (256, 4096, 2048), (200, 14336, 512), (512, 4096, 1024),
                                   (300, 4100, 512), (128, 28672, 1024)])
def test_fp8_repeat_identical(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, M + N + K)
    xq, sx = w8.quantize_per_token(to_dev_bf16(xb))
    wq, sw = w8.quantize_weight_per_channel(to_dev_bf16(wb))
    y0 = w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    ref = y0.clone()
    for r in range(12):
        w8.gemm(xq, sx, wq, sw, out=y0)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), ref.view(torch.int16)), f"{M}x{N}x{K}: run {r + 1} differs"
    oxq, osx = Q.quantize_per_token_fp8(xb)
    owq, osw = Q.quantize_weight_per_channel_fp8(wb)
    rows = np.arange(0, M, max(1, M // 64))
    _assert_tol(bf16_to_f64(ref)[rows], G.gemm_fp8_ref(oxq[rows], osx[rows], owq, osw), f"{M}x{N}x{K}")


@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_fp8_prefill_full_size_sampled(i):
    """The 8B prefill linears at full size, in the bench's launch configuration; codes of
    sampled rows are compared exactly and a sampled output block within tolerance."""
    need_gpu()
    name, xb, wb = synthetic.prefill(i)
    M, K = xb.shape
    N = wb.shape[0]
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    xq, sx = w8.quantize_per_token(x)
    wq, sw = w8.quantize_weight_per_channel(w)
    y = w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + i)
    rows = np.sort(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
    cols = np.sort(np.concatenate([[0, N - 1], rng.choice(N, 254, replace=False)]))
    oxq, osx = Q.quantize_per_token_fp8(xb[rows])
    owq, osw = Q.quantize_weight_per_channel_fp8(wb[cols])
    gxq = bits_u8(xq[torch.as_tensor(rows, device="cuda:0")])
    gwq = bits_u8(wq[torch.as_tensor(cols, device="cuda:0")])
    assert np.array_equal(gxq, oxq), first_mismatch(gxq, oxq)
    assert np.array_equal(gwq, owq), first_mismatch(gwq, owq)
    assert np.array_equal(f32(sx)[rows], osx) and np.array_equal(f32(sw)[cols], osw)
    yg = bf16_to_f64(y)[np.ix_(rows, cols)]
    _assert_tol(yg, G.gemm_fp8_ref(oxq, osx, owq, osw), f"prefill {name}")


@pytest.mark.parametrize("N", synthetic.DECODE_NS)
def test_fp8_decode_sweep(N):
    need_gpu()
    xall = synthetic.decode_x()
    wb = synthetic.decode_w(N)
    w = to_dev_bf16(wb)
    wq, sw = w8.quantize_weight_per_channel(w)
    owq, osw = Q.quantize_weight_per_channel_fp8(wb)
    torch.cuda.synchronize()
    assert np.array_equal(bits_u8(wq), owq) and np.array_equal(f32(sw), osw)
    for M in synthetic.DECODE_MS:
        xb = xall[:M]
        xq, sx = w8.quantize_per_token(to_dev_bf16(xb))
        y = w8.gemm(xq, sx, wq, sw)
        torch.cuda.synchronize()
        oxq, osx = Q.quantize_per_token_fp8(xb)
        assert np.array_equal(bits_u8(xq), oxq)
        _assert_tol(bf16_to_f64(y), G.gemm_fp8_ref(oxq, osx, owq, osw), f"decode M={M} N={N}")


# ----------------------------------------------------------------------------- INT8
def _int8_chain(xb, xcal, wb, alpha, what):
    """SmoothQuant + INT8 W8A8 on both sides, every stage compared bit for bit."""
    x, xc, w = to_dev_bf16(xb), to_dev_bf16(xcal), to_dev_bf16(wb)
    ax = w8.channel_absmax(xc)
    aw = w8.channel_absmax(w)
    s = w8.smoothquant_scales(ax, aw, alpha)
    xh = w8.smooth_apply(x, s, "activation")
    wh = w8.smooth_apply(w, s, "weight")
    xq, sx = w8.quantize_per_token(xh, "int8")
    wq, sw = w8.quantize_weight_per_channel(wh, "int8")
    y = w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    oax, oaw = S.channel_absmax(xcal), S.channel_absmax(wb)
    assert np.array_equal(f32(ax), oax) and np.array_equal(f32(aw), oaw)
    os_ = S.smooth_scales(oax, oaw, alpha)
    assert np.array_equal(f32(s).view(np.uint32), os_.view(np.uint32)), first_mismatch(f32(s), os_)
    oxh, owh = S.smooth_activations(xb, os_), S.smooth_weights(wb, os_)
    assert np.array_equal(bf16_bits(xh), oxh), first_mismatch(bf16_bits(xh), oxh)
    assert np.array_equal(bf16_bits(wh), owh), first_mismatch(bf16_bits(wh), owh)
    oxq, osx = Q.quantize_per_token_int8(oxh)
    owq, osw = Q.quantize_weight_per_channel_int8(owh)
    assert np.array_equal(bits_i8(xq), oxq) and np.array_equal(f32(sx), osx)
    assert np.array_equal(bits_i8(wq), owq) and np.array_equal(f32(sw), osw)
    oy = G.gemm_int8_ref(oxq, osx, owq, osw)
    gy = bf16_bits(y)
    assert np.array_equal(gy, oy), f"{what}: " + first_mismatch(gy, oy)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (17, 130, 384), (300, 549, 1024), (64, 256, 14336),
                                   (513, 129, 1024), (260, 4100, 256), (2049, 1000, 512), (2049, 3000, 512),
                                   (1999, 6001, 384), (2048, 6144, 256)])
def test_int8_ragged(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, M + N + K)
    xcal, _ = _xw(64, 1, K, K)
    _int8_chain(xb, xcal, wb, 0.5, f"{M}x{N}x{K}")


# The INT8 GEMM shares the two-waves-per-SIMD schedule (and its stage refills) with the
# MXFP4 one: repeated launches must give identical bits, equal to the oracle's.
@pytest.mark.parametrize("M,N,K", [(2048, 4096, 1024), (512, 6144, 4096), (2048, 6144, 1024),
                                   (128, 4096, 4096), (100, 14336, 1024), (256, 4096, 2048),
                                   (512, 4096, 1024), (100, 24000, 512)])
def test_int8_repeat_identical(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, 3 * M + N + K)
    xq, sx = w8.quantize_per_token(to_dev_bf16(xb), "int8")
    wq, sw = w8.quantize_weight_per_channel(to_dev_bf16(wb), "int8")
    y0 = w8.gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    ref = y0.clone()
    for r in range(12):
        w8.gemm(xq, sx, wq, sw, out=y0)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), ref.view(torch.int16)), f"{M}x{N}x{K}: run {r + 1} differs"
    oxq, osx = Q.quantize_per_token_int8(xb)
    owq, osw = Q.quantize_weight_per_channel_int8(wb)
    rows = np.arange(0, M, max(1, M // 64))
    oy = G.gemm_int8_ref(oxq[rows], osx[rows], owq, osw)
    gy = bf16_bits(ref)[rows]
    assert np.array_equal(gy, oy), f"{M}x{N}x{K}: " + first_mismatch(gy, oy)


@pytest.mark.parametrize("M,N,K", FEW_TOKEN_CASES)
def test_int8_few_tokens(M, N, K):
    need_gpu()
    xb, wb = _xw(M, N, K, 13 * M + 3 * N + K)
    xcal, _ = _xw(64, 1, K, K + 1)
    _int8_chain(xb, xcal, wb, 0.5, f"{M}x{N}x{K}")


@pytest.mark.parametrize("N", synthetic.DECODE_NS)
def test_int8_smoothquant_decode_sweep(N):
    need_gpu()
    xall = synthetic.decode_x()
    xcal = synthetic.decode_calibration()
    wb = synthetic.decode_w(N)
    for M in synthetic.DECODE_MS:
        _int8_chain(xall[:M], xcal, wb, 0.5, f"decode M={M} N={N}")


def test_smoothquant_general_alpha():
    need_gpu()
    xcal, wb = _xw(64, 96, 256, 5)
    ax, aw = w8.channel_absmax(to_dev_bf16(xcal)), w8.channel_absmax(to_dev_bf16(wb))
    for alpha in (0.0, 0.25, 0.85, 1.0):
        s = f32(w8.smoothquant_scales(ax, aw, alpha))
        os_ = S.smooth_scales(S.channel_absmax(xcal), S.channel_absmax(wb), alpha)
        if alpha in (0.0, 1.0):
            assert np.array_equal(s, os_)
        else:
            np.testing.assert_allclose(s, os_, rtol=2e-6)


# ----------------------------------------------------------------------------- block-scaled
def _block_compare(xb, wb, what, rows=None, wblocks=None):
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    xq, sx = w8.quantize_per_token_group(x)
    wq, sw = w8.quantize_weight_block(w)
    y = w8.gemm_blockscaled(xq, sx, wq, sw)
    torch.cuda.synchronize()
    M, N = xb.shape[0], wb.shape[0]
    rows = np.arange(M) if rows is None else rows
    cols = np.arange(N) if wblocks is None else np.concatenate(
        [np.arange(b * 128, min(N, (b + 1) * 128)) for b in wblocks])
    oxq, osx = Q.quantize_per_token_group_fp8(xb[rows])
    owq, osw = Q.quantize_weight_block_fp8(wb[cols])
    assert np.array_equal(bits_u8(xq)[rows], oxq) and np.array_equal(f32(sx)[rows], osx)
    assert np.array_equal(bits_u8(wq)[cols], owq)
    gsw = f32(sw)[np.arange(N)[cols][::128] // 128]
    assert np.array_equal(gsw, osw)
    _assert_tol(bf16_to_f64(y)[np.ix_(rows, cols)], G.gemm_blockscaled_ref(oxq, osx, owq, osw), what)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (17, 130, 384), (300, 549, 1024), (64, 256, 7168)])
def test_blockscaled_ragged(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M * 3 + N + K)
    xb = _bf16(rng.standard_t(3, size=(M, K)))
    wb = _bf16(rng.standard_normal((N, K)) * 0.02)
    _block_compare(xb, wb, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(513, 384, 2048), (256, 130, 1280)])
def test_blockscaled_scales_span_binades(M, N, K):
    """Every 1 x 128 activation group, token and 128 x 128 weight block at its own power of
    two (2^-12 .. 2^12): applying a neighbouring group's, row's or block's scale in the
    promotion moves the output by orders of magnitude."""
    need_gpu()
    rng = np.random.default_rng(M + 7 * N + K)
    G_ = K // 128
    xs = np.exp2(rng.integers(-12, 13, size=(M, G_))).repeat(128, axis=1)
    ws = np.exp2(rng.integers(-12, 13, size=((N + 127) // 128, G_))).repeat(128, axis=0)
    ws = ws.repeat(128, axis=1)[:N]
    xb = _bf16(rng.standard_normal((M, K)) * xs)
    wb = _bf16(rng.standard_normal((N, K)) * 0.02 * ws)
    _block_compare(xb, wb, f"binade-scaled {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(512, 1024, 1024), (1024, 2048, 4096)])
def test_blockscaled_repeat_identical(M, N, K):
    """The block-scaled GEMM shares the FP8 kernel's stage refills and adds its own
    double-buffered scale area in LDS: repeated launches must give identical bits."""
    need_gpu()
    rng = np.random.default_rng(M + N + K + 1)
    xb = _bf16(rng.standard_t(3, size=(M, K)))
    wb = _bf16(rng.standard_normal((N, K)) * 0.02)
    xq, sx = w8.quantize_per_token_group(to_dev_bf16(xb))
    wq, sw = w8.quantize_weight_block(to_dev_bf16(wb))
    y0 = w8.gemm_blockscaled(xq, sx, wq, sw)
    torch.cuda.synchronize()
    ref = y0.clone()
    for r in range(12):
        w8.gemm_blockscaled(xq, sx, wq, sw, out=y0)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), ref.view(torch.int16)), f"{M}x{N}x{K}: run {r + 1} differs"
    _block_compare(xb, wb, f"repeat {M}x{N}x{K}")


def test_blockscaled_full_size_sampled():
    need_gpu()
    xb, wb = synthetic.blockscaled()
    rng = np.random.default_rng(44)
    rows = np.sort(np.concatenate([[0, xb.shape[0] - 1], rng.choice(xb.shape[0], 62, replace=False)]))
    _block_compare(xb, wb, "block-scaled 4096x18432x7168", rows=rows, wblocks=[0, 77, 143])


# ----------------------------------------------------------------------------- MXFP4
def _mx_compare(xb, wb, what, rows=None, cols=None):
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    xq, sx = w8.quantize_mxfp4(x)
    wq, sw = w8.quantize_mxfp4(w)
    y = w8.gemm_mxfp4(xq, sx, wq, sw)
    torch.cuda.synchronize()
    rows = np.arange(xb.shape[0]) if rows is None else rows
    cols = np.arange(wb.shape[0]) if cols is None else cols
    oxq, osx = Q.quantize_mxfp4(xb[rows])
    owq, osw = Q.quantize_mxfp4(wb[cols])
    assert np.array_equal(bits_u8(xq)[rows], oxq) and np.array_equal(bits_u8(sx)[rows], osx)
    assert np.array_equal(bits_u8(wq)[cols], owq) and np.array_equal(bits_u8(sw)[cols], osw)
    _assert_tol(bf16_to_f64(y)[np.ix_(rows, cols)], G.gemm_mxfp4_ref(oxq, osx, owq, osw), what)


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (17, 130, 512), (300, 549, 1024), (64, 256, 8192)])
def test_mxfp4_ragged(M, N, K):
    need_gpu()
    xb = synthetic.mxfp4_x(M, K)
    wb = _bf16(np.random.default_rng(N + K).standard_normal((N, K)) * 0.02)
    _mx_compare(xb, wb, f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(17, 130, 512), (300, 549, 1024), (513, 384, 2048)])
def test_mxfp4_scales_span_binades(M, N, K):
    """Every (row, 32-element block) of both operands at its own power of two in
    2^-12 .. 2^12, so that the E8M0 scales of W vary as much as those of X: applying a
    neighbouring row's or block's scale in the scaled MFMA moves the output by orders of
    magnitude. Ragged and multi-tile shapes."""
    need_gpu()
    rng = np.random.default_rng(M + 5 * N + K)
    xs = np.exp2(rng.integers(-12, 13, size=(M, K // 32))).repeat(32, axis=1)
    ws = np.exp2(rng.integers(-12, 13, size=(N, K // 32))).repeat(32, axis=1)
    xb = _bf16(rng.standard_normal((M, K)) * xs)
    wb = _bf16(rng.standard_normal((N, K)) * 0.02 * ws)
    _mx_compare(xb, wb, f"binade-scaled mxfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(17, 130, 512), (300, 549, 1024), (4096, 4100, 256)])
def test_mxfp4_non_finite_blocks(M, N, K):
    """Infinities and NaNs scattered over both operands: their blocks carry the E8M0 NaN
    code, and the GEMM gives NaN in exactly the rows of X and columns of W that hold one,
    the oracle's value within the tolerance everywhere else. The last shape runs on the
    256 x 256 one-wave-per-SIMD kernel, the others on the two-waves-per-SIMD kernel."""
    need_gpu()
    rng = np.random.default_rng(M + 3 * N + K)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K)) * 0.02
    for a, vals in ((x, (np.inf, -np.inf, np.nan)), (w, (np.nan, np.inf, -np.inf))):
        idx = rng.choice(a.size, size=max(3, a.shape[0] // 40), replace=False)
        a.flat[idx] = rng.choice(vals, size=len(idx))
    xb, wb = _bf16(x), _bf16(w)
    xq, sx = w8.quantize_mxfp4(to_dev_bf16(xb))
    wq, sw = w8.quantize_mxfp4(to_dev_bf16(wb))
    y = w8.gemm_mxfp4(xq, sx, wq, sw)
    torch.cuda.synchronize()
    oxq, osx = Q.quantize_mxfp4(xb)
    owq, osw = Q.quantize_mxfp4(wb)
    assert np.array_equal(bits_u8(sx), osx) and np.array_equal(bits_u8(xq), oxq)
    assert np.array_equal(bits_u8(sw), osw) and np.array_equal(bits_u8(wq), owq)
    ref = G.gemm_mxfp4_ref(oxq, osx, owq, osw)
    nan_ref = np.isnan(ref)
    assert np.array_equal(nan_ref, np.isnan(x).any(1)[:, None] | np.isinf(x).any(1)[:, None]
                          | (np.isnan(w).any(1) | np.isinf(w).any(1))[None, :])
    yg = bf16_to_f64(y)
    assert np.array_equal(np.isnan(yg), nan_ref), f"{M}x{N}x{K}: NaN pattern differs"
    _assert_tol(yg[~nan_ref], ref[~nan_ref], f"non-finite mxfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,binades", [(4097, 4100, 512, False), (4096, 4352, 768, True),
                                            (4352, 4096, 256, True)])
def test_mxfp4_wide_tiles(M, N, K, binades):
    """Shapes with at least one round of 256 x 256 tiles, which the one-wave-per-SIMD MXFP4
    kernel takes: ragged M and N, one to three K steps, scales of both operands at their
    own powers of two per (row, 32-block); sampled rows and columns that include every tile
    edge at both ends."""
    need_gpu()
    rng = np.random.default_rng(M + 3 * N + K)
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((N, K)) * 0.02
    if binades:
        x *= np.exp2(rng.integers(-12, 13, size=(M, K // 32))).repeat(32, axis=1)
        w *= np.exp2(rng.integers(-12, 13, size=(N, K // 32))).repeat(32, axis=1)
    xb, wb = _bf16(x), _bf16(w)
    edges = lambda n: np.unique(np.clip(np.concatenate([np.arange(0, n, 256), np.arange(255, n, 256), [n - 1]]), 0, n - 1))
    rows = np.unique(np.concatenate([edges(M), rng.choice(M, 40, replace=False)]))
    cols = np.unique(np.concatenate([edges(N), rng.choice(N, 40, replace=False)]))
    _mx_compare(xb, wb, f"mxfp4 wide tiles {M}x{N}x{K}", rows=rows, cols=cols)


def test_mxfp4_wide_tiles_repeat_identical():
    """The one-wave-per-SIMD MXFP4 kernel refills a stage while waves still compute on
    fragments read from the other; repeated launches must give identical bits."""
    need_gpu()
    rng = np.random.default_rng(77)
    xb = synthetic.mxfp4_x(4096, 1024)
    wb = _bf16(rng.standard_normal((4096, 1024)) * 0.02)
    xq, sx = w8.quantize_mxfp4(to_dev_bf16(xb))
    wq, sw = w8.quantize_mxfp4(to_dev_bf16(wb))
    y0 = w8.gemm_mxfp4(xq, sx, wq, sw)
    torch.cuda.synchronize()
    ref = y0.clone()
    for r in range(10):
        w8.gemm_mxfp4(xq, sx, wq, sw, out=y0)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), ref.view(torch.int16)), f"run {r + 1} differs"
    rows = np.arange(0, 4096, 61)
    oxq, osx = Q.quantize_mxfp4(xb[rows])
    owq, osw = Q.quantize_mxfp4(wb)
    _assert_tol(bf16_to_f64(ref)[rows], G.gemm_mxfp4_ref(oxq, osx, owq, osw), "mxfp4 repeat 4096^2 x 1024")


def test_mxfp4_full_size_sampled():
    need_gpu()
    xb, wb = synthetic.mxfp4()
    rng = np.random.default_rng(55)
    rows = np.sort(np.concatenate([[0, 8191], rng.choice(8192, 62, replace=False)]))
    cols = np.sort(np.concatenate([[0, 8191], rng.choice(8192, 190, replace=False)]))
    _mx_compare(xb, wb, "mxfp4 8192^3", rows=rows, cols=cols)
