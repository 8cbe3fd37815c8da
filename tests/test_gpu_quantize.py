"""GPU parity: the HIP quantizers against the oracle, bit for bit (codes and scales)."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import formats as F
from oracle import quant as Q
from tests.gpu_util import bits_u8, bits_i8, f32, first_mismatch, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def _check_rows_fp8(xb, fn=w8.quantize_per_token):
    q, s = fn(to_dev_bf16(xb), "e4m3fn")
    torch.cuda.synchronize()
    qo, so = Q.quantize_rows_fp8(xb)
    gq, gs = bits_u8(q), f32(s)
    assert np.array_equal(gs.view(np.uint32), so.view(np.uint32)), first_mismatch(gs, so)
    assert np.array_equal(gq, qo), first_mismatch(gq, qo)


def _check_rows_int8(xb, fn=w8.quantize_per_token):
    q, s = fn(to_dev_bf16(xb), "int8")
    torch.cuda.synchronize()
    qo, so = Q.quantize_rows_int8(xb)
    gq, gs = bits_i8(q), f32(s)
    assert np.array_equal(gs.view(np.uint32), so.view(np.uint32)), first_mismatch(gs, so)
    assert np.array_equal(gq, qo), first_mismatch(gq, qo)


def test_tiny_config_fp8_codes_and_scales():
    need_gpu()
    x, w = synthetic.tiny()
    _check_rows_fp8(x)
    _check_rows_fp8(w, w8.quantize_weight_per_channel)


@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (17, 256), (300, 4096), (5, 14336),
                                 (9, 16384), (4, 16896), (2, 40960), (64, 7168)])
def test_fp8_and_int8_shapes(M, K):
    need_gpu()
    rng = np.random.default_rng(M * 100003 + K)
    x = rng.standard_normal((M, K))
    ch = rng.choice(K, size=max(1, K // 1000), replace=False)
    x[:, ch] *= rng.uniform(50, 500, size=len(ch))
    xb = _bf16(x)
    _check_rows_fp8(xb)
    _check_rows_int8(xb)


def test_prefill_activations_full_size():
    """Per-token quantization of the full 8B prefill activations (2048 x 4096, 2048 x 14336)."""
    need_gpu()
    for i in (0, 3):
        _, x, _ = synthetic.prefill(i, n_limit=1)
        _check_rows_fp8(x)


def test_all_bf16_patterns_through_the_encoder():
    """Rows whose amax is 448 (s = 1 exactly) carry every finite bf16 value of magnitude
    <= 448, so x / s = x and the encoder sees all of them; rows with other amax values
    scale the same patterns by non-trivial fp32 scales."""
    need_gpu()
    allv = synthetic.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16)).astype(np.float64)
    v = allv[np.isfinite(allv) & (np.abs(allv) <= 448)]
    v = np.concatenate([v, np.zeros((-len(v)) % 1023)])
    rows = v.reshape(-1, 1023)
    rows = np.concatenate([rows, np.full((rows.shape[0], 1), 448.0)], axis=1)   # [R, 1024]
    xb = _bf16(rows)
    _check_rows_fp8(xb)
    _check_rows_int8(xb)
    big = rows.copy()
    big[:, -1] = 3.0e4                 # amax 3e4: every pattern divided by s = 3e4 / 448
    _check_rows_fp8(_bf16(big))
    small = rows * 2.0 ** -100         # tiny magnitudes, subnormal bf16 included
    _check_rows_fp8(_bf16(small))


def test_edge_rows():
    need_gpu()
    K = 256
    rows = []
    rows.append(np.zeros(K))                                    # all zero
    rows.append(-np.zeros(K))                                   # all negative zero
    r = np.zeros(K); r[7] = -3.0; rows.append(r)                # single negative max
    r = np.full(K, 1.0); rows.append(r)                         # all equal
    mids = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (mids[:-1] + mids[1:]) / 2                           # E4M3 midpoints (s = 1)
    r = np.zeros(K); r[:len(mids)] = mids; r[-1] = 448.0; rows.append(r)
    r = np.zeros(K); r[:len(mids)] = -mids; r[-1] = -448.0; rows.append(r)
    r = np.linspace(-1e-8, 1e-8, K); rows.append(r)             # below the 1e-8 floor
    r = np.full(K, 2.0 ** -130); r[0] = 2.0 ** -126; rows.append(r)
    r = np.full(K, 3.0e38); r[1::2] *= -1; rows.append(r)       # near bf16 max
    xb = _bf16(np.array(rows))
    _check_rows_fp8(xb)
    _check_rows_int8(xb)


def test_non_finite_inputs_do_not_fault():
    need_gpu()
    x = np.random.default_rng(7).standard_normal((4, 64))
    x[0, 3] = np.nan
    x[1, 5] = np.inf
    x[2, :] = np.nan
    xb = _bf16(x)
    q, s = w8.quantize_per_token(to_dev_bf16(xb))
    torch.cuda.synchronize()
    gq = bits_u8(q)
    assert (gq[0, 3] & 0x7F) == 0x7F            # NaN element -> NaN code
    assert np.all((gq[2] & 0x7F) == 0x7F)
    assert np.isinf(f32(s)[1])
    qo, _ = Q.quantize_rows_fp8(xb[3:4])
    assert np.array_equal(gq[3:4], qo)          # untouched row still exact


def test_empty_rows():
    need_gpu()
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda:0")
    q, s = w8.quantize_per_token(x)
    assert q.shape == (0, 128) and s.shape == (0,)


# ----------------------------------------------------------------------------- groups / blocks
@pytest.mark.parametrize("M,K", [(1, 128), (5, 384), (33, 7168), (300, 1024)])
def test_group_quant(M, K):
    need_gpu()
    xb = _bf16(np.random.default_rng(M + K).standard_t(3, size=(M, K)))
    q, s = w8.quantize_per_token_group(to_dev_bf16(xb))
    torch.cuda.synchronize()
    qo, so = Q.quantize_per_token_group_fp8(xb)
    assert np.array_equal(f32(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(bits_u8(q), qo), first_mismatch(bits_u8(q), qo)


@pytest.mark.parametrize("N,K", [(1, 128), (130, 256), (256, 7168), (333, 384)])
def test_weight_block_quant(N, K):
    need_gpu()
    wb = _bf16(np.random.default_rng(N * 7 + K).standard_normal((N, K)) * 0.02)
    q, s = w8.quantize_weight_block(to_dev_bf16(wb))
    torch.cuda.synchronize()
    qo, so = Q.quantize_weight_block_fp8(wb)
    assert np.array_equal(f32(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(bits_u8(q), qo), first_mismatch(bits_u8(q), qo)


# ----------------------------------------------------------------------------- MXFP4
@pytest.mark.parametrize("R,K", [(1, 32), (3, 96), (64, 8192), (257, 512)])
def test_mxfp4_quant(R, K):
    need_gpu()
    xb = synthetic.mxfp4_x(R, K)
    q, s = w8.quantize_mxfp4(to_dev_bf16(xb))
    torch.cuda.synchronize()
    qo, so = Q.quantize_mxfp4(xb)
    assert np.array_equal(bits_u8(s), so), first_mismatch(bits_u8(s), so)
    assert np.array_equal(bits_u8(q), qo), first_mismatch(bits_u8(q), qo)


def test_mxfp4_quant_non_finite_blocks():
    """Every non-finite bf16 pattern (both infinities, every NaN payload) once in a block of
    otherwise finite values, and blocks whose only non-finite element sits in each of the
    four 8-element chunks: the E8M0 NaN code and zero element codes, bit for bit, with the
    neighbouring blocks untouched."""
    need_gpu()
    allv = synthetic.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16)).astype(np.float64)
    bad = allv[~np.isfinite(allv)]
    rng = np.random.default_rng(11)
    x = rng.standard_normal((len(bad) // 4 + 4, 4 * 32)) * 3.0
    for i, b in enumerate(bad):                 # block i % 4 of row i // 4, element (7 i) % 32
        x[i // 4, 32 * (i % 4) + (7 * i) % 32] = b
    for c in range(4):                          # last rows: one infinity in chunk c of block c
        x[-4 + c, 32 * c + 8 * c + 3] = np.inf if c % 2 else -np.inf
    xb = _bf16(x)
    q, s = w8.quantize_mxfp4(to_dev_bf16(xb))
    torch.cuda.synchronize()
    qo, so = Q.quantize_mxfp4(xb)
    assert np.count_nonzero(so == 255) == len(bad) + 4
    assert np.array_equal(bits_u8(s), so), first_mismatch(bits_u8(s), so)
    assert np.array_equal(bits_u8(q), qo), first_mismatch(bits_u8(q), qo)


def test_mxfp4_quant_all_bf16_patterns():
    need_gpu()
    allv = synthetic.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16)).astype(np.float64)
    v = allv[np.isfinite(allv)]
    v = np.concatenate([v, np.zeros((-len(v)) % 512)])
    xb = _bf16(v.reshape(-1, 32 * 16))
    q, s = w8.quantize_mxfp4(to_dev_bf16(xb))
    torch.cuda.synchronize()
    qo, so = Q.quantize_mxfp4(xb)
    assert np.array_equal(bits_u8(s), so), first_mismatch(bits_u8(s), so)
    assert np.array_equal(bits_u8(q), qo), first_mismatch(bits_u8(q), qo)
