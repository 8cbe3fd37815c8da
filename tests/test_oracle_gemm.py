"""Pins for oracle/gemm.py: brute force, the scale-factoring identity, the SmoothQuant
worked example's printed product, and reductions between the variants."""

import itertools

import numpy as np

import synthetic
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from tests import golden


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def test_fp8_ref_matches_bruteforce_nonsquare():
    rng = np.random.default_rng(10)
    x = _bf16(rng.standard_normal((3, 128)))
    w = _bf16(rng.standard_normal((5, 128)) * 0.02)
    xq, sx = Q.quantize_per_token_fp8(x)
    wq, sw = Q.quantize_weight_per_channel_fp8(w)
    y = G.gemm_fp8_ref(xq, sx, wq, sw)
    yb = G.gemm_fp8_bruteforce(xq, sx, wq, sw)
    assert y.shape == (3, 5)
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-15)


def test_scale_factoring_identity():
    """Dequantize-then-multiply equals multiply-then-scale (page: the finest scales that
    factor out of the matmul are per-token and per-output-channel)."""
    x, w = synthetic.tiny()
    xq, sx = Q.quantize_per_token_fp8(x)
    wq, sw = Q.quantize_weight_per_channel_fp8(w)
    xhat = F.e4m3_decode(xq) * sx[:, None].astype(np.float64)
    what = F.e4m3_decode(wq) * sw[:, None].astype(np.float64)
    lhs = xhat @ what.T
    rhs = G.gemm_fp8_ref(xq, sx, wq, sw)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # and it stays within FP8's error budget of the unquantized product: each element
    # is off by at most 2^-4 of itself (normal range) plus half a subnormal step, 2^-10 s
    xf = F.bf16_to_f64(x)
    wf = F.bf16_to_f64(w)
    ex = np.abs(xf) * 2.0 ** -4 + 2.0 ** -10 * sx[:, None]
    ew = np.abs(wf) * 2.0 ** -4 + 2.0 ** -10 * sw[:, None]
    bound = ex @ np.abs(wf).T + np.abs(xf) @ ew.T + ex @ ew.T
    assert np.all(np.abs(rhs - xf @ wf.T) <= bound)


def test_per_input_channel_scale_does_not_factor():
    """A per-input-channel scale cannot be pulled out of the K reduction (page: scales per
    input channel do not factor out); a per-row one can."""
    rng = np.random.default_rng(11)
    a = rng.standard_normal((4, 8))
    b = rng.standard_normal((3, 8))
    c = rng.uniform(0.5, 2, 8)
    assert not np.allclose((a * c) @ b.T, np.diag(np.ones(4)) @ (a @ b.T) * c.mean())
    r = rng.uniform(0.5, 2, 4)
    np.testing.assert_allclose((a * r[:, None]) @ b.T, np.diag(r) @ (a @ b.T))


def test_int8_acc_exact_and_epilogue_order():
    rng = np.random.default_rng(12)
    xq = rng.integers(-127, 128, (7, 14336)).astype(np.int8)
    wq = rng.integers(-127, 128, (9, 14336)).astype(np.int8)
    acc = G.gemm_int8_acc(xq, wq)
    assert np.array_equal(acc, G.gemm_int8_acc_bruteforce(xq, wq))
    big = np.full((1, 14336), 127, np.int8)
    assert G.gemm_int8_acc(big, -big)[0, 0] == -14336 * 127 * 127
    acc_loop = np.array([[sum(int(a) * int(b) for a, b in zip(xq[m], wq[n])) for n in range(2)] for m in range(2)])
    assert np.array_equal(acc[:2, :2], acc_loop)
    # epilogue: fp32(fp32(acc) * s_x) * s_w, each product rounded, then bf16 RNE
    sx = rng.uniform(1e-3, 1e-2, 7).astype(np.float32)
    sw = rng.uniform(1e-4, 1e-3, 9).astype(np.float32)
    y = G.int8_epilogue_bf16(acc, sx, sw)
    for m in range(7):
        for n in range(9):
            t = np.float32(np.float32(acc[m, n]) * sx[m])
            v = np.float32(t * sw[n])
            assert y[m, n] == F.f64_to_bf16_rne(np.array([float(v)]))[0]


def test_int8_epilogue_rounding_order_hand_case():
    """A hand case where the order of the INT8 epilogue's roundings shows in the bf16
    output ("FP8 and INT8 Inference" §5 writes Y_int32 x s_x x s_w, left to right). With
    acc = -13999889 (exact in fp32), s_x = 0x3B201C75 and s_w = 0x3A8B6513 (bit patterns of
    fp32 scales): each product of a 24-bit integer or significand and a 24-bit significand
    is exact in fp64, so the roundings below are exactly the ones they name.
      left to right:  t = fp32(acc s_x), v = fp32(t s_w)      -> bf16 0xC212
      scales first:   v = fp32(acc fp32(s_x s_w))             -> bf16 0xC211
      one rounding:   v = fp32(acc s_x s_w)                   -> bf16 0xC211
    The oracle must give the left-to-right result; a dropped intermediate rounding or a
    product of the two scales taken first fails here."""
    acc = -13999889
    sx = np.array([0x3B201C75], np.uint32).view(np.float32)[0]
    sw = np.array([0x3A8B6513], np.uint32).view(np.float32)[0]

    def bf16_rne(v32):
        u = int(np.float32(v32).view(np.uint32))
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF

    t = np.float32(float(acc) * float(sx))                       # exact fp64 product, one rounding
    left_to_right = bf16_rne(np.float32(float(t) * float(sw)))
    scales_first = bf16_rne(np.float32(float(acc) * float(np.float32(float(sx) * float(sw)))))
    from fractions import Fraction
    exact = Fraction(acc) * Fraction(float(sx)) * Fraction(float(sw))
    one_rounding = bf16_rne(np.float32(float(exact)))            # exact < 2^53 ulps: float() is RNE
    assert (left_to_right, scales_first, one_rounding) == (0xC212, 0xC211, 0xC211)
    y = G.int8_epilogue_bf16(np.array([[acc]], np.int64), np.array([sx]), np.array([sw]))
    assert int(y[0, 0]) == 0xC212


def test_smoothquant_worked_example_product():
    """The printed 2x2 product of the smoothed 4-bit example: the activation codes come
    from the printed quantized activations; an exhaustive search over all 4-bit weight
    codes through the oracle's integer GEMM + scale epilogue finds exactly the weight
    codes that reproduce the printed product."""
    ex = golden.load("smoothquant_worked_example.txt")
    lv = golden.ints(ex, "levels")[0]
    step = np.sqrt(58 * 0.020) / lv
    assert abs(step - golden.floats(ex, "step_approx")[0]) < 5e-4
    xd = np.array([golden.floats(ex, "xq_dequant_row0"), golden.floats(ex, "xq_dequant_row1")])
    xq = np.rint(xd / step).astype(np.int8)
    assert np.allclose(xq * step, xd, atol=5e-4)
    prod = np.array([golden.floats(ex, "product_row0"), golden.floats(ex, "product_row1")])
    cands = np.array(list(itertools.product(range(-lv, lv + 1), repeat=3)), np.int8)
    acc = G.gemm_int8_acc(xq, cands)                        # [2, 3375]
    y = acc * step * step
    for n in range(2):
        hits = np.where(np.all(np.abs(np.round(y, 3) - prod[:, n][:, None]) < 5e-4 + 1e-9, axis=0))[0]
        assert len(hits) == 1
        assert cands[hits[0]].tolist() == golden.ints(ex, f"wq_reconstructed_row{n}")


def test_blockscaled_bruteforce_and_reduction():
    rng = np.random.default_rng(13)
    M, K, N = 3, 256, 130
    x = _bf16(rng.standard_t(3, size=(M, K)))
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    xq, sx = Q.quantize_per_token_group_fp8(x)
    wq, sw = Q.quantize_weight_block_fp8(w)
    y = G.gemm_blockscaled_ref(xq, sx, wq, sw)
    a = F.e4m3_decode(xq); b = F.e4m3_decode(wq)
    for m in range(M):
        for n in (0, 77, 128, 129):
            tot = 0.0
            for g in range(2):
                part = sum(a[m, k] * b[n, k] for k in range(g * 128, (g + 1) * 128))
                tot += float(sx[m, g]) * float(sw[n // 128, g]) * part
            assert abs(tot - y[m, n]) <= 1e-12 * (abs(tot) + 1)
    # K = 128, N <= 128 and rows sharing one amax: block scaling == per-token/per-channel
    w2 = rng.standard_normal((64, 128)) * 0.02
    w2[:, 5] = 0.3
    w2b = _bf16(w2)
    xq1, sx1 = Q.quantize_per_token_group_fp8(x[:, :128])
    wq1, sw1 = Q.quantize_weight_block_fp8(w2b)
    xq2, sx2 = Q.quantize_per_token_fp8(x[:, :128])
    wq2, sw2 = Q.quantize_weight_per_channel_fp8(w2b)
    y1 = G.gemm_blockscaled_ref(xq1, sx1, wq1, sw1)
    y2 = G.gemm_fp8_ref(xq2, sx2, wq2, sw2)
    np.testing.assert_allclose(y1, y2, rtol=1e-14, atol=0)


def test_mxfp4_ref_bruteforce():
    rng = np.random.default_rng(14)
    M, K, N = 3, 96, 4
    x = synthetic.mxfp4_x(M, K)
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    xq, sx = Q.quantize_mxfp4(x)
    wq, sw = Q.quantize_mxfp4(w)
    y = G.gemm_mxfp4_ref(xq, sx, wq, sw)
    ca = F.unpack_e2m1(xq); cb = F.unpack_e2m1(wq)
    for m in range(M):
        for n in range(N):
            tot = 0.0
            for blk in range(K // 32):
                part = sum(float(F.e2m1_decode(ca[m, k])) * float(F.e2m1_decode(cb[n, k]))
                           for k in range(blk * 32, (blk + 1) * 32))
                tot += 2.0 ** (int(sx[m, blk]) - 127) * 2.0 ** (int(sw[n, blk]) - 127) * part
            assert tot == y[m, n]


def test_tolerance_rule():
    y_ref = np.array([[1.0, -2.0], [0.0, 100.0]])
    rms = np.sqrt(np.mean(y_ref ** 2))
    ok, worst = G.within_tolerance(y_ref + 0.009 * (np.abs(y_ref) + rms), y_ref)
    assert ok and worst < 1
    bad = y_ref.copy()
    bad[1, 0] += 0.011 * rms
    assert not G.within_tolerance(bad, y_ref)[0]
