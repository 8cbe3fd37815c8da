"""Pins for the extended-epilogue oracle (bias, activation, FP8 requantized output).

Each check stands on something other than the oracle's own formula: the already pinned
plain references (options off), closed forms and an independent library routine for
SiLU, and hand-computed INT8 examples whose every intermediate is exact in fp32.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import epilogue as E
from oracle import gemm as G
from oracle import quant as Q
from oracle.formats import bf16_to_f64, e4m3_decode

import synthetic


def _tiny(seed=5, M=7, N=9, K=256):
    rng = np.random.default_rng(seed)
    xb = synthetic.to_bf16_bits(rng.standard_normal((M, K)))
    wb = synthetic.to_bf16_bits(rng.standard_normal((N, K)) * 0.05)
    return xb, wb


def test_options_off_reduce_to_the_plain_references():
    xb, wb = _tiny()
    xq, sx = Q.quantize_per_token_fp8(xb)
    wq, sw = Q.quantize_weight_per_channel_fp8(wb)
    assert np.array_equal(E.fp8_path_ref(xq, sx, wq, sw), G.gemm_fp8_ref(xq, sx, wq, sw))
    xi, sxi = Q.quantize_per_token_int8(xb)
    wi, swi = Q.quantize_weight_per_channel_int8(wb)
    assert np.array_equal(E.int8_path_ref(xi, sxi, wi, swi), G.gemm_int8_ref(xi, sxi, wi, swi))


def test_silu_closed_forms_and_an_independent_routine():
    assert E.silu64(0.0) == 0.0
    assert math.isclose(float(E.silu64(1.0)), 1.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(float(E.silu64(-1.0)), -1.0 / (1.0 + math.e), rel_tol=1e-15)
    assert float(E.silu64(40.0)) == 40.0                      # sigmoid(40) rounds to 1
    assert abs(float(E.silu64(-40.0)) + 40.0 * math.exp(-40.0)) < 1e-30
    v = np.random.default_rng(0).standard_normal(1000) * 8
    np.testing.assert_allclose(E.silu64(v), v * scipy.special.expit(v), rtol=1e-14, atol=1e-300)


def _int8_case(acc_row, sx, sw, K=128):
    """INT8 operands whose single output is sum(acc_row) (x codes acc_row, w codes 1)."""
    xq = np.zeros((1, K), np.int8)
    xq[0, :len(acc_row)] = acc_row
    wq = np.zeros((1, K), np.int8)
    wq[0, :len(acc_row)] = 1
    return xq, np.array([sx], np.float32), wq, np.array([sw], np.float32)


def test_bias_then_activation_order():
    # acc = -4, s_x = s_w = 0.5 -> v = -1; bias +2 -> 1; ReLU -> 1 (ReLU before the bias
    # would give 2). bf16(1.0) = 0x3F80.
    args = _int8_case([-4], 0.5, 0.5)
    bias = np.array([0x4000], np.uint16)                      # bf16 2.0
    assert E.int8_path_ref(*args, bias_bits=bias, act="relu")[0, 0] == 0x3F80
    assert E.int8_path_ref(*args, act="relu")[0, 0] == 0x0000  # ReLU(-1) = 0
    assert E.int8_path_ref(*args, bias_bits=bias)[0, 0] == 0x3F80
    # the FP8-operand path gives the same exact value
    xq = np.zeros((1, 128), np.uint8)
    xq[0, 0] = 0x40                                           # E4M3 2.0
    wq = np.zeros((1, 128), np.uint8)
    wq[0, 0] = 0xC0                                           # E4M3 -2.0
    y = E.fp8_path_ref(xq, np.array([0.25]), wq, np.array([1.0]), bias_bits=bias, act="relu")
    assert y[0, 0] == 1.0                                     # relu(0.25 * -4 + 2)


@pytest.mark.parametrize("acc_row,sx,s_out,code", [
    ([1], 1.0, 1.0, 0x38),                 # 1.0 exactly
    ([17], 1.0 / 16, 1.0, 0x38),           # 1.0625: tie between 1.0 and 1.125 -> even (1.0)
    ([19], 1.0 / 16, 1.0, 0x3A),           # 1.1875: tie between 1.125 and 1.25 -> even (1.25)
    ([100] * 5, 1.0, 1.0, 0x7E),           # 500 saturates to 448
    ([-100] * 6, 1.0, 1.0, 0xFE),          # -600 saturates to -448
    ([20], 1.0, 2.0, 0x52),                # 20 / 2 = 10 = 1.25 * 2^3
    ([3], 1.0, 512.0, 0x03),               # 3/512 = 3 * 2^-9, a subnormal
    ([3], 1.0, 1024.0, 0x02),              # 1.5 * 2^-9: subnormal tie -> even (2 * 2^-9)
])
def test_fp8_output_codes(acc_row, sx, s_out, code):
    args = _int8_case(acc_row, sx, 1.0)
    got = E.int8_path_ref(*args, s_out=s_out)[0, 0]
    assert got == code, (hex(got), hex(code))


def test_fp8_output_clamp_on_the_fp8_operand_path():
    xq = np.zeros((1, 128), np.uint8)
    xq[0, :4] = 0x7E                                          # 448 each
    wq = np.zeros((2, 128), np.uint8)
    wq[0, :4] = 0x7E
    wq[1, :4] = 0xFE
    z = E.fp8_path_ref(xq, np.array([1.0]), wq, np.array([1.0, 1.0]), s_out=1.0)
    assert z[0, 0] == 448.0 and z[0, 1] == -448.0             # 4 * 448^2 clamps both ways
    z = E.fp8_path_ref(xq, np.array([1.0]), wq, np.array([1.0, 1.0]), s_out=4 * 448.0 * 448.0 / 2)
    assert z[0, 0] == 2.0 and e4m3_decode(np.array([0x40]))[0] == 2.0


def test_e4m3_spacing():
    assert E.e4m3_spacing(1.0) == 0.125
    assert E.e4m3_spacing(1.9) == 0.125
    assert E.e4m3_spacing(448.0) == 32.0
    assert E.e4m3_spacing(2.0 ** -6) == 2.0 ** -9             # smallest normal binade
    assert E.e4m3_spacing(2.0 ** -8) == 2.0 ** -9             # subnormals
    assert E.e4m3_spacing(0.0) == 2.0 ** -9


def test_silu_int8_path_is_silu_of_the_fp32_value():
    xb, wb = _tiny(7)
    xi, sxi = Q.quantize_per_token_int8(xb)
    wi, swi = Q.quantize_weight_per_channel_int8(wb)
    v = E.int8_path_values(xi, sxi, wi, swi).astype(np.float64)
    s = E.int8_path_values(xi, sxi, wi, swi, act="silu").astype(np.float64)
    np.testing.assert_allclose(s, v * scipy.special.expit(v), rtol=2 ** -23, atol=1e-30)
    bias = synthetic.to_bf16_bits(np.linspace(-1, 1, wb.shape[0]))
    vb = E.int8_path_values(xi, sxi, wi, swi, bias_bits=bias).astype(np.float64)
    np.testing.assert_allclose(vb - v, np.broadcast_to(bf16_to_f64(bias), v.shape), atol=1e-5)
