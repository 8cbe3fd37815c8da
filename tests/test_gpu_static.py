"""GPU parity: static per-tensor quantization, its saturation count and running amax, and
delayed scaling, against the oracle. Codes, counts, amax and scales bit for bit (NaN
elements: NaN-ness of the code only)."""

import numpy as np
import pytest
import torch

import synthetic
import fp4_w8a8_quantized_amd as w8
from oracle import static_scale as S
from oracle.formats import e4m3_decode
from tests.gpu_util import bits_i8, bits_u8, need_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu


def _x(M, K, seed, spread=4.0):
    rng = np.random.default_rng(seed)
    return synthetic.to_bf16_bits(rng.standard_normal((M, K)) * np.exp2(rng.uniform(-spread, spread, (M, 1))))


def _scalar(v, dtype=torch.float32):
    return torch.tensor([v], dtype=dtype, device="cuda")


def _codes_equal(fmt, got, ref):
    if fmt == "e4m3fn":
        nan_g, nan_r = np.isnan(e4m3_decode(got)), np.isnan(e4m3_decode(ref))
        return np.array_equal(nan_g, nan_r) and np.array_equal(got[~nan_g], ref[~nan_r])
    return np.array_equal(got, ref)


@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
@pytest.mark.parametrize("M,K", [(1, 8), (3, 40), (300, 4096), (2048, 14336)])
def test_static_quantize(fmt, M, K):
    need_gpu()
    xb = _x(M, K, M * 7 + K)
    x = to_dev_bf16(xb)
    amax_all = float(S.tensor_amax(xb))
    qmax = 448.0 if fmt == "e4m3fn" else 127.0
    # a scale that fits and one calibrated on a quarter of the range (saturates)
    for s in (np.float32(amax_all / qmax), np.float32(amax_all / qmax / 4)):
        sat = _scalar(0, torch.int32)
        amax = _scalar(0.0)
        q = w8.quantize_static(x, _scalar(float(s)), fmt, saturated=sat, amax=amax)
        torch.cuda.synchronize()
        fn = S.quantize_static_fp8 if fmt == "e4m3fn" else S.quantize_static_int8
        rq, rsat, ramax = fn(xb, s)
        got = bits_u8(q) if fmt == "e4m3fn" else bits_i8(q)
        assert _codes_equal(fmt, got, rq), f"{fmt} {M}x{K} s={s}"
        assert int(sat.item()) == rsat, (int(sat.item()), rsat)
        assert np.float32(amax.item()) == ramax


@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
def test_counter_and_amax_accumulate_and_special_values(fmt):
    need_gpu()
    row = [0.0, -0.0, 1.0, -1.0, 500.0, -1000.0, float("inf"), float("-inf"), float("nan"), 448.0,
           449.0, 127.5, -127.5, 2.0 ** -12, 3e38, -3e38]
    xb = synthetic.to_bf16_bits(np.array([row], np.float64))
    x = to_dev_bf16(xb)
    sat = _scalar(5, torch.int32)                       # accumulates on top of 5
    amax = _scalar(2.0)                                 # running max starts at 2
    q = w8.quantize_static(x, _scalar(1.0), fmt, saturated=sat, amax=amax)
    w8.quantize_static(x, _scalar(1.0), fmt, saturated=sat, amax=amax)
    torch.cuda.synchronize()
    fn = S.quantize_static_fp8 if fmt == "e4m3fn" else S.quantize_static_int8
    rq, rsat, ramax = fn(xb, np.float32(1.0))
    got = bits_u8(q) if fmt == "e4m3fn" else bits_i8(q)
    assert _codes_equal(fmt, got, rq), (got, rq)
    assert int(sat.item()) == 5 + 2 * rsat
    assert float(amax.item()) == max(2.0, float(ramax))


@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
def test_delayed_scaling_loop(fmt):
    need_gpu()
    H, steps = 3, 7
    hist_ref = np.array([1.0, 0.5, 0.25], np.float32) * (448 if fmt == "e4m3fn" else 127)
    history = torch.from_numpy(hist_ref.copy()).cuda()
    amax = _scalar(0.0)
    sat = _scalar(0, torch.int32)
    qmax = np.float32(448.0 if fmt == "e4m3fn" else 127.0)
    scale_ref = np.float32(max(float(hist_ref.max()), 1e-8) / qmax)
    scale = _scalar(float(scale_ref))
    sat_ref = 0
    fn = S.quantize_static_fp8 if fmt == "e4m3fn" else S.quantize_static_int8
    for step in range(steps):
        xb = _x(64, 512, 100 + step, spread=3.0 + step)  # growing range: later steps saturate
        q = w8.quantize_static(to_dev_bf16(xb), scale, fmt, saturated=sat, amax=amax)
        rq, rsat, ramax = fn(xb, scale_ref)
        sat_ref += rsat
        w8.delayed_scale_update(history, amax, step, scale, fmt)
        hist_ref, scale_ref = S.delayed_scale_update(hist_ref, ramax, step, fmt)
        torch.cuda.synchronize()
        got = bits_u8(q) if fmt == "e4m3fn" else bits_i8(q)
        assert _codes_equal(fmt, got, rq), f"step {step}"
        assert np.array_equal(history.cpu().numpy(), hist_ref), f"step {step}"
        assert np.float32(scale.item()) == scale_ref, f"step {step}"
        assert float(amax.item()) == 0.0
    assert int(sat.item()) == sat_ref and sat_ref > 0


@pytest.mark.parametrize("fmt", ["e4m3fn", "int8"])
@pytest.mark.parametrize("s", [2.0 ** -70, 2.0 ** -60, 1e-3, 3.0, 2.0 ** 60, 2.0 ** 61, 1e30])
def test_extreme_scales(fmt, s):
    """Both sides of the quotient shortcut's range [2^-60, 2^60], with quotients that
    overflow fp32 and infinite inputs."""
    need_gpu()
    rng = np.random.default_rng(int(np.log2(s) + 100))
    v = rng.standard_normal(4096) * np.exp2(rng.uniform(-80, 120, 4096))
    v[:4] = [np.inf, -np.inf, 3.0e38, -1e-38]
    xb = synthetic.to_bf16_bits(v.reshape(8, 512))
    sat = _scalar(0, torch.int32)
    amax = _scalar(0.0)
    q = w8.quantize_static(to_dev_bf16(xb), _scalar(float(np.float32(s))), fmt, saturated=sat, amax=amax)
    torch.cuda.synchronize()
    fn = S.quantize_static_fp8 if fmt == "e4m3fn" else S.quantize_static_int8
    rq, rsat, ramax = fn(xb, np.float32(s))
    got = bits_u8(q) if fmt == "e4m3fn" else bits_i8(q)
    assert _codes_equal(fmt, got, rq)
    assert int(sat.item()) == rsat
    assert np.float32(amax.item()) == ramax
