"""Pins for oracle/smoothquant.py: the closed forms printed on the pages."""

import numpy as np
import torch

import synthetic
from oracle import formats as F
from oracle import smoothquant as S
from tests import golden


def test_exercise_channel_112():
    ex = golden.load("smoothquant_exercise.txt")
    a = golden.floats(ex, "act_max")[0]
    w = golden.floats(ex, "w_max")[0]
    for alpha, s_exp, xa, wa in zip(golden.floats(ex, "alpha"), golden.floats(ex, "s"),
                                    golden.floats(ex, "act_after"), golden.floats(ex, "w_after")):
        s = float(S.smooth_scales(np.array([a]), np.array([w]), alpha)[0])
        assert abs(s - s_exp) <= 0.005 * s_exp, (alpha, s, s_exp)
        # smoothed maxima, as the page rounds them (from its 2-decimal s)
        assert abs(a / s_exp - xa) <= 0.006 and abs(w * s_exp - wa) <= 0.006


def test_worked_example_factors():
    ex = golden.load("smoothquant_worked_example.txt")
    s = S.smooth_scales(np.array(golden.floats(ex, "act_max")), np.array(golden.floats(ex, "w_max")),
                        golden.floats(ex, "alpha")[0])
    for got, exp in zip(s, golden.floats(ex, "s")):
        assert abs(float(got) - exp) <= 0.0006 * exp


def test_alpha_half_equalises_ranges():
    rng = np.random.default_rng(20)
    x = synthetic.random_bf16((64, 32), 21)
    w = synthetic.random_bf16((48, 32), 22, 0.02)
    ax, aw = S.channel_absmax(x), S.channel_absmax(w)
    s = S.smooth_scales(ax, aw, 0.5).astype(np.float64)
    xs = F.bf16_to_f64(x) / s[None, :]
    ws = F.bf16_to_f64(w) * s[None, :]
    geo = np.sqrt(ax.astype(np.float64) * aw.astype(np.float64))
    np.testing.assert_allclose(np.abs(xs).max(0), geo, rtol=1e-6)
    np.testing.assert_allclose(np.abs(ws).max(0), geo, rtol=1e-6)
    # the rescaling is exact before rounding: (X / s)(W s)^T = X W^T
    np.testing.assert_allclose(xs @ ws.T, F.bf16_to_f64(x) @ F.bf16_to_f64(w).T, rtol=1e-10, atol=1e-12)
    del rng


def test_alpha_limits():
    a = np.array([80.0, 0.5], np.float32)
    w = np.array([0.02, 0.04], np.float32)
    np.testing.assert_array_equal(S.smooth_scales(a, w, 1.0), a)
    np.testing.assert_array_equal(S.smooth_scales(a, w, 0.0), np.float32(1) / w)
    # the 1e-5 floor applies to both maxima
    s = S.smooth_scales(np.array([0.0], np.float32), np.array([0.0], np.float32), 0.5)
    assert s[0] == np.float32(np.sqrt(np.float32(1e-5))) / np.float32(np.sqrt(np.float32(1e-5)))


def test_channel_absmax_bruteforce():
    x = synthetic.random_bf16((17, 9), 23)
    xf = F.bf16_to_f32(x)
    exp = [max(abs(float(xf[r, j])) for r in range(17)) for j in range(9)]
    assert S.channel_absmax(x).tolist() == exp


def test_smooth_apply_rounding_matches_torch():
    x = synthetic.random_bf16((33, 40), 24, 5.0)
    s = np.random.default_rng(25).uniform(0.1, 30, 40).astype(np.float32)
    xt = torch.from_numpy(F.bf16_to_f32(x).copy())
    st = torch.from_numpy(s)
    exp_x = (xt / st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    exp_w = (xt * st).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(S.smooth_activations(x, s), exp_x)
    assert np.array_equal(S.smooth_weights(x, s), exp_w)
