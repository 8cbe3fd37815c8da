"""GPU parity at the largest operand the library accepts: 2^31 bytes of codes in one matrix
(the GEMM kernels address an operand with 32-bit byte offsets). The operands are seeded
random codes of each format; the oracle computes sampled output columns (or rows), INT8
bit for bit and the floating-point formats within |y - y_ref| <= 1e-2 (|y_ref| + rms)."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import gemm as G
from oracle import nvfp4 as NV
from oracle import quant as Q
from oracle import w4a16 as W
from tests.gpu_util import bf16_bits, bf16_to_f64, bits_u8, f32, need_gpu, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

LIMIT = 2 ** 31
TOL = 1e-2


@pytest.fixture(scope="module")
def raw():
    """2^31 seeded random bytes, reshaped into each test's largest operand."""
    return synthetic.random_bytes(LIMIT, synthetic.seed(9, 0, 2))


def _rng(i):
    return np.random.default_rng(synthetic.seed(9, i, 1))


def _fp8_codes(b):
    """E4M3FN codes with exponent field <= 7 (|v| <= 1.875), never NaN."""
    return b & np.uint8(0xBF)


def _int8_codes(b):
    return np.maximum(b.view(np.int8), np.int8(-127))


def _sample(n, rng, count=62):
    """First and last index, the 128 / 192 / 256 tile edges near both ends, and random ones."""
    edges = [0, 127, 128, 191, 192, 255, 256, n - 257, n - 256, n - 193, n - 192, n - 129,
             n - 128, n - 1]
    return np.unique(np.concatenate([edges, rng.choice(n, count, replace=False)]))


def _check_tol(y, y_ref, what):
    ok, worst = G.within_tolerance(y, y_ref, TOL)
    assert ok, f"{what}: worst error / bound = {worst:.3f}"


@pytest.mark.parametrize("M", [16, 100, 200, 300])
def test_fp8_weight_at_limit(raw, M):
    """W 131072 x 16384 E4M3FN: the narrow-tile kernel at M = 16 (16 x 128 tiles) and 100
    (128 x 128 tiles, eight waves), the prefill kernels at 200 and 300 (narrow tiles would
    take several rounds of the CUs on 131072 outputs)."""
    need_gpu()
    N, K = 131072, 16384
    rng = _rng(1)
    wq = _fp8_codes(raw).reshape(N, K)
    xq = _fp8_codes(synthetic.random_bytes(M * K, synthetic.seed(9, 1, 1))).reshape(M, K)
    sx = np.exp2(rng.uniform(-8, -2, M)).astype(np.float32)
    sw = np.exp2(rng.uniform(-8, -2, N)).astype(np.float32)
    dw = to_dev(wq, torch.float8_e4m3fn)
    y = w8.gemm(to_dev(xq, torch.float8_e4m3fn), to_dev(sx), dw, to_dev(sw))
    torch.cuda.synchronize()
    del dw
    cols = _sample(N, rng)
    _check_tol(bf16_to_f64(y[:, torch.from_numpy(cols).to(y.device)]),
               G.gemm_fp8_ref(xq, sx, wq[cols], sw[cols]), f"fp8 {M}x{N}x{K}")


def test_fp8_activation_at_limit(raw):
    """X 131072 x 16384 E4M3FN against a 16-row weight: the prefill kernel, ragged N."""
    need_gpu()
    M, N, K = 131072, 16, 16384
    rng = _rng(2)
    xq = _fp8_codes(raw).reshape(M, K)
    wq = _fp8_codes(synthetic.random_bytes(N * K, synthetic.seed(9, 2, 2))).reshape(N, K)
    sx = np.exp2(rng.uniform(-8, -2, M)).astype(np.float32)
    sw = np.exp2(rng.uniform(-8, -2, N)).astype(np.float32)
    dx = to_dev(xq, torch.float8_e4m3fn)
    y = w8.gemm(dx, to_dev(sx), to_dev(wq, torch.float8_e4m3fn), to_dev(sw))
    torch.cuda.synchronize()
    del dx
    rows = _sample(M, rng)
    _check_tol(bf16_to_f64(y[torch.from_numpy(rows).to(y.device)]),
               G.gemm_fp8_ref(xq[rows], sx[rows], wq, sw), f"fp8 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [16, 100, 300])
def test_int8_weight_at_limit(raw, M):
    """W 131072 x 16384 INT8, outputs bit for bit: few-token kernel at 16, tiled at 300."""
    need_gpu()
    N, K = 131072, 16384
    rng = _rng(3)
    wq = _int8_codes(raw).reshape(N, K)
    xq = _int8_codes(synthetic.random_bytes(M * K, synthetic.seed(9, 3, 1))).reshape(M, K)
    sx = np.exp2(rng.uniform(-12, -6, M)).astype(np.float32)
    sw = np.exp2(rng.uniform(-12, -6, N)).astype(np.float32)
    dw = to_dev(wq, torch.int8)
    y = w8.gemm(to_dev(xq, torch.int8), to_dev(sx), dw, to_dev(sw))
    torch.cuda.synchronize()
    del dw
    cols = _sample(N, rng)
    got = bf16_bits(y)[:, cols]
    want = G.gemm_int8_ref(xq, sx, wq[cols], sw[cols])
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"int8 {M}x{N}x{K}: {len(bad)} mismatches, first {bad[0]}"


def test_blockscaled_weight_at_limit(raw):
    """W 131072 x 16384 E4M3FN with 128 x 128 block scales, X 300 x 16384 with 1 x 128."""
    need_gpu()
    M, N, K = 300, 131072, 16384
    rng = _rng(4)
    wq = _fp8_codes(raw).reshape(N, K)
    xq = _fp8_codes(synthetic.random_bytes(M * K, synthetic.seed(9, 4, 1))).reshape(M, K)
    sx = np.exp2(rng.uniform(-8, -2, (M, K // 128))).astype(np.float32)
    sw = np.exp2(rng.uniform(-8, -2, (N // 128, K // 128))).astype(np.float32)
    dw = to_dev(wq, torch.float8_e4m3fn)
    y = w8.gemm_blockscaled(to_dev(xq, torch.float8_e4m3fn), to_dev(sx), dw, to_dev(sw))
    torch.cuda.synchronize()
    del dw
    blocks = np.array([0, 1, 517, N // 128 - 1])
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    _check_tol(bf16_to_f64(y[:, torch.from_numpy(cols).to(y.device)]),
               G.gemm_blockscaled_ref(xq, sx, wq[cols], sw[blocks]), f"block {M}x{N}x{K}")


def test_mxfp4_weight_at_limit(raw):
    """W 131072 x 32768 E2M1 (2^31 packed bytes) with E8M0 scales, X 300 x 32768."""
    need_gpu()
    M, N, K = 300, 131072, 32768
    rng = _rng(5)
    wq = raw.reshape(N, K // 2)
    xq = synthetic.random_bytes(M * K // 2, synthetic.seed(9, 5, 1)).reshape(M, K // 2)
    sx = rng.integers(120, 128, (M, K // 32), dtype=np.uint8)
    sw = rng.integers(120, 128, (N, K // 32), dtype=np.uint8)
    dw = to_dev(wq)
    y = w8.gemm_mxfp4(to_dev(xq), to_dev(sx), dw, to_dev(sw))
    torch.cuda.synchronize()
    del dw
    cols = _sample(N, rng)
    _check_tol(bf16_to_f64(y[:, torch.from_numpy(cols).to(y.device)]),
               G.gemm_mxfp4_ref(xq, sx, wq[cols], sw[cols]), f"mxfp4 {M}x{N}x{K}")


def test_nvfp4_weight_at_limit(raw):
    """W 131072 x 32768 E2M1 with E4M3 block scales and fp32 tensor scales, X 300 x 32768."""
    need_gpu()
    M, N, K = 300, 131072, 32768
    rng = _rng(6)
    wq = raw.reshape(N, K // 2)
    xq = synthetic.random_bytes(M * K // 2, synthetic.seed(9, 6, 1)).reshape(M, K // 2)
    sx = rng.integers(0x28, 0x48, (M, K // 16), dtype=np.uint8)     # E4M3 0.0625 .. 3.75
    sw = rng.integers(0x28, 0x48, (N, K // 16), dtype=np.uint8)
    gx, gw = np.float32(1.0 / 2688), np.float32(0.02 / 2688)
    dw = to_dev(wq)
    y = w8.gemm_nvfp4(to_dev(xq), to_dev(sx), to_dev(np.array([gx])), dw, to_dev(sw),
                      to_dev(np.array([gw])))
    torch.cuda.synchronize()
    del dw
    cols = _sample(N, rng)
    _check_tol(bf16_to_f64(y[:, torch.from_numpy(cols).to(y.device)]),
               NV.gemm_nvfp4_ref(xq, sx, gx, wq[cols], sw[cols], gw), f"nvfp4 {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 16, 100])
def test_w4a16_weight_at_limit(raw, M):
    """W 131072 x 32768 INT4 (2^31 packed bytes, every nibble incl. -8) with fp16 scales."""
    need_gpu()
    N, K = 131072, 32768
    rng = _rng(7)
    wq = raw.reshape(N, K // 2)
    s = np.exp2(rng.uniform(-10, -4, (N, K // 128))).astype(np.float16)
    xb = synthetic.random_bf16((M, K), synthetic.seed(9, 7, 1))
    dw = to_dev(wq)
    y = w8.gemm_w4a16(to_dev_bf16(xb), dw, to_dev(s))
    torch.cuda.synchronize()
    del dw
    cols = _sample(N, rng)
    _check_tol(bf16_to_f64(y[:, torch.from_numpy(cols).to(y.device)]),
               W.gemm_w4a16_ref(xb, wq[cols], s[cols]), f"w4a16 {M}x{N}x{K}")


def test_w4a16_activation_at_limit(raw):
    """X bf16 131072 x 8192 (2^31 bytes, |x| in [2^-7, 2)) against a 16-row INT4 weight: the
    LDS-staged kernel at its largest activation offsets."""
    need_gpu()
    M, N, K = 131072, 16, 8192
    rng = _rng(8)
    xb = ((raw.view(np.uint16) & np.uint16(0x83FF)) | np.uint16(0x3C00)).reshape(M, K)
    wq = synthetic.random_bytes(N * K // 2, synthetic.seed(9, 8, 2)).reshape(N, K // 2)
    s = np.exp2(rng.uniform(-10, -4, (N, K // 128))).astype(np.float16)
    dx = to_dev_bf16(xb)
    y = w8.gemm_w4a16(dx, to_dev(wq), to_dev(s))
    torch.cuda.synchronize()
    del dx
    rows = _sample(M, rng)
    _check_tol(bf16_to_f64(y[torch.from_numpy(rows).to(y.device)]),
               W.gemm_w4a16_ref(xb[rows], wq, s), f"w4a16 {M}x{N}x{K}")


def test_quantize_per_token_at_limit(raw):
    """X bf16 65536 x 16384 (2^31 bytes): codes and scales of sampled rows bit for bit."""
    need_gpu()
    M, K = 65536, 16384
    # random sign and mantissa, exponent 112..127 (|x| in [2^-15, 2)): never NaN or Inf
    xb = ((raw.view(np.uint16) & np.uint16(0x87FF)) | np.uint16(0x3800)).reshape(M, K)
    dx = to_dev_bf16(xb)
    xq, sx = w8.quantize_per_token(dx)
    torch.cuda.synchronize()
    del dx
    rows = _sample(M, _rng(8))
    oq, os_ = Q.quantize_per_token_fp8(xb[rows])
    sel = torch.from_numpy(rows).to(xq.device)
    assert np.array_equal(f32(sx[sel]), os_)
    assert np.array_equal(bits_u8(xq[sel]), oq)
