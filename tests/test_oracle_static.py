"""Pins for the static-scale quantizer, its saturation count and delayed scaling."""

import numpy as np

import synthetic
from oracle import quant as Q
from oracle import static_scale as S


def _bits(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def test_one_row_with_its_own_amax_scale_equals_the_dynamic_quantizer():
    # A single row quantized with s = fp32(max|x|)/448 (resp. /127) is per-token dynamic
    # quantization of that row: the codes must agree exactly.
    rng = np.random.default_rng(3)
    for _ in range(5):
        x = _bits(rng.standard_normal((1, 512)) * rng.uniform(0.01, 100))
        q_dyn, s_dyn = Q.quantize_per_token_fp8(x)
        q, sat, amax = S.quantize_static_fp8(x, s_dyn[0])
        assert np.array_equal(q, q_dyn) and sat == 0
        qi_dyn, si_dyn = Q.quantize_per_token_int8(x)
        qi, sat_i, _ = S.quantize_static_int8(x, si_dyn[0])
        assert np.array_equal(qi, qi_dyn) and sat_i == 0


def test_saturation_count_fp8_hand_example():
    x = _bits([[500.0, -1000.0, 448.0, 450.0, 1.0, -448.0, 0.0, 2.0 ** 20]])
    q, sat, amax = S.quantize_static_fp8(x, 1.0)
    assert sat == 4                                   # 500, -1000, 450, 2^20 were clipped
    assert list(q[0]) == [0x7E, 0xFE, 0x7E, 0x7E, 0x38, 0xFE, 0x00, 0x7E]
    assert amax == 2.0 ** 20
    q2, sat2, _ = S.quantize_static_fp8(x, 4096.0)    # |x|/4096 <= 256: nothing clipped
    assert sat2 == 0


def test_saturation_count_int8_hand_example():
    # rne: 127 -> 127, 127.25 -> 127, 127.5 -> 128 (ties to even), 128 -> 128, -200 -> -200
    x = _bits([[127.0, 127.25, 127.5, 128.0, -200.0, -126.5, 0.0, 1.0]])
    q, sat, amax = S.quantize_static_int8(x, 1.0)
    assert sat == 3
    assert list(q[0]) == [127, 127, 127, 127, -127, -126, 0, 1]   # -126.5 -> -126 (even)
    assert amax == 200.0


def test_amax_and_nan():
    x = _bits([[1.0, float("nan"), -3.0], [2.0, 0.5, -0.25]])
    q, sat, amax = S.quantize_static_fp8(x, 1.0)
    assert amax == 3.0 and sat == 0 and q[0, 1] in (0x7F, 0xFF)
    qi, sat_i, _ = S.quantize_static_int8(x, 1.0)
    assert qi[0, 1] == 0 and sat_i == 0


def test_delayed_scaling_window():
    h = np.zeros(3, np.float32)
    h, s = S.delayed_scale_update(h, 448.0, 0, "e4m3fn")
    assert s == np.float32(1.0) and list(h) == [448.0, 0.0, 0.0]
    h, s = S.delayed_scale_update(h, 896.0, 1, "e4m3fn")
    assert s == np.float32(2.0)
    h, s = S.delayed_scale_update(h, 100.0, 2, "e4m3fn")
    assert s == np.float32(2.0)                        # 896 still in the window
    h, s = S.delayed_scale_update(h, 100.0, 3, "e4m3fn")   # overwrites slot 0 (448)
    assert s == np.float32(2.0)
    h, s = S.delayed_scale_update(h, 100.0, 4, "e4m3fn")   # overwrites slot 1 (896)
    assert s == np.float32(np.float32(100.0) / np.float32(448.0))
    _, s = S.delayed_scale_update(np.zeros(2, np.float32), 254.0, 7, "int8")
    assert s == np.float32(2.0)
    _, s = S.delayed_scale_update(np.zeros(2, np.float32), 0.0, 0, "e4m3fn")
    assert s == np.float32(np.float32(1e-8) / np.float32(448.0))
