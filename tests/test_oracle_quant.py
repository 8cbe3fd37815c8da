"""Pins for oracle/quant.py: brute force, page worked example, and invariants."""

import math

import numpy as np

import synthetic
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from tests import golden


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def _scalar_e4m3_nearest(v: float) -> int:
    """Nearest finite E4M3FN value to v (clamped to 448), ties to the even code."""
    table = [(c, float(F.e4m3_decode(c))) for c in range(0x7F)]
    a = min(abs(v), 448.0)
    best = min(table, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return best[0] | (0x80 if math.copysign(1.0, v) < 0 else 0)


def _bruteforce_rows_fp8(x_bits):
    """Per-row quantization with Python loops and fp32 scalar arithmetic."""
    x = F.bf16_to_f32(x_bits)
    R, K = x.shape
    codes = np.zeros((R, K), np.uint8)
    scales = np.zeros(R, np.float32)
    for r in range(R):
        amax = np.float32(0.0)
        for k in range(K):
            amax = max(amax, np.float32(abs(x[r, k])))
        s = np.float32(max(amax, np.float32(1e-8))) / np.float32(448.0)
        scales[r] = s
        for k in range(K):
            codes[r, k] = _scalar_e4m3_nearest(float(np.float32(x[r, k]) / s))
    return codes, scales


def test_per_token_fp8_matches_bruteforce_tiny():
    x, w = synthetic.tiny()
    q, s = Q.quantize_per_token_fp8(x[:6])
    qb, sb = _bruteforce_rows_fp8(x[:6])
    assert np.array_equal(s, sb)
    assert np.array_equal(q, qb)
    qw, sw = Q.quantize_weight_per_channel_fp8(w[:5])
    qwb, swb = _bruteforce_rows_fp8(w[:5])
    assert np.array_equal(sw, swb) and np.array_equal(qw, qwb)


def test_amax_element_maps_to_448_with_its_sign():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 300))
    idx = rng.integers(0, 300, 64)
    sign = rng.choice([-1.0, 1.0], 64)
    x[np.arange(64), idx] = sign * 50.0                # the largest magnitude, either sign
    q, s = Q.quantize_per_token_fp8(_bf16(x))
    got = q[np.arange(64), idx]
    assert np.all(got == np.where(sign < 0, 0xFE, 0x7E))
    assert np.all(s == np.float32(50.0) / np.float32(448.0))
    # no other element reaches the top code
    q2 = q.copy()
    q2[np.arange(64), idx] = 0
    assert np.all((q2 & 0x7F) < 0x7E)


def test_zero_row_and_signed_zero():
    x = np.zeros((3, 16))
    x[1] = -0.0
    x[2, 3] = 1.0
    q, s = Q.quantize_per_token_fp8(_bf16(x))
    assert s[0] == np.float32(1e-8) / np.float32(448.0) and s[1] == s[0]
    assert np.all(q[0] == 0x00) and np.all(q[1] == 0x80)
    assert q[2, 3] == 0x7E and s[2] == np.float32(1.0) / np.float32(448.0)


def test_power_of_two_equivariance_and_row_independence():
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((8, 256)) * 3)
    q, s = Q.quantize_per_token_fp8(x)
    x4 = _bf16(F.bf16_to_f64(x) * 4.0)
    q4, s4 = Q.quantize_per_token_fp8(x4)
    assert np.array_equal(q, q4) and np.array_equal(s * 4, s4)
    perm = rng.permutation(8)
    qp, sp = Q.quantize_per_token_fp8(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    # one row scaled up only changes that row: scales are per row, not per column
    xr = F.bf16_to_f64(x).copy()
    xr[2] *= 1000
    qr, sr = Q.quantize_per_token_fp8(_bf16(xr))
    keep = np.arange(8) != 2
    assert np.array_equal(qr[keep], q[keep]) and np.array_equal(sr[keep], s[keep])


def test_quotient_is_a_division_not_a_reciprocal_product():
    """x / s is one fp32 division (the emulation divides by s); find a row where a
    reciprocal-multiply would pick a different code and check the division wins."""
    rng = np.random.default_rng(5)
    found = 0
    for _ in range(200):
        x = _bf16(rng.standard_normal((64, 512)))
        q, s = Q.quantize_per_token_fp8(x)
        xf = F.bf16_to_f32(x)
        by_rcp = F.e4m3_encode((xf * (np.float32(1) / s)[:, None]).astype(np.float32))
        by_div = F.e4m3_encode((xf / s[:, None]).astype(np.float32))
        assert np.array_equal(q, by_div)
        found += int(np.sum(by_rcp != by_div))
        if found:
            break
    assert found > 0


# ----------------------------------------------------------------------------- INT8
def test_worked_example_int8_per_tensor():
    ex = golden.load("fp8_int8_tiny_example.txt")
    x = np.array(golden.floats(ex, "input"))
    q, s = Q.quantize_rows_int8(_bf16(x[None, :]))
    deq = q[0].astype(np.float64) * float(s[0])
    # the bf16 input of 0.05 is 0.0500488..., which does not change any printed digit
    assert [f"{v:.4f}" for v in deq] == ex["int8_dequant"]
    assert [f"{abs((a - b) / b):.3f}" for a, b in zip(deq, x)] == ex["int8_rel_err"]


def test_int8_ties_clamp_and_bruteforce():
    x = np.array([[127.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -127.0]])
    q, s = Q.quantize_rows_int8(_bf16(x))
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 2, 4, -2, 0, 0, 2, -127]
    rng = np.random.default_rng(6)
    xb = _bf16(rng.standard_normal((5, 64)) * 7)
    q, s = Q.quantize_rows_int8(xb)
    xf = F.bf16_to_f32(xb)
    for r in range(5):
        amax = max(abs(float(v)) for v in xf[r])
        sr = np.float32(max(np.float32(amax), np.float32(1e-8))) / np.float32(127)
        assert s[r] == sr
        for k in range(64):
            v = float(np.float32(xf[r, k]) / sr)
            assert q[r, k] == max(-127, min(127, round(v)))   # Python round is half-even
    assert np.abs(q).max() == 127 and q.min() >= -127


# ----------------------------------------------------------------------------- groups / blocks
def test_group_quant_bruteforce_and_reduction():
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_t(3, size=(4, 384)))
    q, s = Q.quantize_per_token_group_fp8(x, 128)
    assert s.shape == (4, 3)
    for g in range(3):
        qb, sb = _bruteforce_rows_fp8(x[:, g * 128:(g + 1) * 128])
        assert np.array_equal(q[:, g * 128:(g + 1) * 128], qb) and np.array_equal(s[:, g], sb)
    # K = 128: one group per row is exactly per-token quantization
    q1, s1 = Q.quantize_per_token_group_fp8(x[:, :128], 128)
    qt, st = Q.quantize_per_token_fp8(x[:, :128])
    assert np.array_equal(q1, qt) and np.array_equal(s1[:, 0], st)


def test_weight_block_quant_bruteforce():
    rng = np.random.default_rng(8)
    N, K = 200, 256                                  # partial last row block
    w = _bf16(rng.standard_normal((N, K)) * 0.02)
    q, s = Q.quantize_weight_block_fp8(w, 128)
    assert s.shape == (2, 2)
    wf = F.bf16_to_f32(w)
    for b in range(2):
        for g in range(2):
            blk = wf[b * 128:(b + 1) * 128, g * 128:(g + 1) * 128]
            amax = np.float32(max(abs(float(v)) for v in blk.ravel()))
            sb = np.float32(max(amax, np.float32(1e-8))) / np.float32(448)
            assert s[b, g] == sb
            qb = q[b * 128:(b + 1) * 128, g * 128:(g + 1) * 128]
            for (i, j) in [(0, 0), (5, 77), (blk.shape[0] - 1, 127)]:
                assert qb[i, j] == _scalar_e4m3_nearest(float(np.float32(blk[i, j]) / sb))
            exp = F.e4m3_encode((blk / sb).astype(np.float32))
            assert np.array_equal(qb, exp)


def test_weight_block_equals_per_channel_when_rows_share_amax():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((100, 128)) * 0.02
    w[np.arange(100), rng.integers(0, 128, 100)] = 0.25 * rng.choice([-1, 1], 100)
    wb = _bf16(w)
    qb, sb = Q.quantize_weight_block_fp8(wb, 128)
    qc, sc = Q.quantize_weight_per_channel_fp8(wb)
    assert np.all(sc == sb[0, 0])
    assert np.array_equal(qb, qc)


# ----------------------------------------------------------------------------- MXFP4
def _bruteforce_mx_block(vals):
    amax = max(abs(float(v)) for v in vals)
    if amax == 0:
        e = 0
    else:
        e = math.frexp(amax)[1] - 1 - 2
        e = max(-127, min(127, e))
    table = [(c, float(F.e2m1_decode(c))) for c in range(8)]
    codes = []
    for v in vals:
        a = min(abs(float(v)) / 2.0 ** e, 6.0)
        c = min(table, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))[0]
        codes.append(c | (8 if math.copysign(1.0, float(v)) < 0 else 0))
    return e + 127, codes


def test_mxfp4_bruteforce_and_properties():
    x = synthetic.mxfp4_x(4, 256)
    qp, sc = Q.quantize_mxfp4(x)
    assert qp.shape == (4, 128) and sc.shape == (4, 8)
    codes = F.unpack_e2m1(qp)
    xf = F.bf16_to_f32(x)
    for r in range(4):
        for b in range(8):
            e, c = _bruteforce_mx_block(xf[r, b * 32:(b + 1) * 32])
            assert sc[r, b] == e
            assert codes[r, b * 32:(b + 1) * 32].tolist() == c
            # the largest element lands on 4 or 6 (codes 6, 7), never above 6
            j = int(np.argmax(np.abs(xf[r, b * 32:(b + 1) * 32])))
            assert (c[j] & 7) in (6, 7)


def test_mxfp4_non_finite_blocks():
    """A block with an infinity or a NaN gets the E8M0 NaN code 255 and zero element codes;
    the other blocks of the row are quantized as if it were not there."""
    x = np.zeros((3, 96))
    x[0, 5] = np.inf                            # block 0 of row 0
    x[0, 40] = 3.0                              # block 1 of row 0: unaffected
    x[1, 70] = np.nan                           # block 2 of row 1
    x[1, 71] = 1.0
    x[2, 10] = -np.inf                          # row 2, block 0
    x[2, 64:96] = 0.5                           # row 2, block 2: unaffected
    qp, sc = Q.quantize_mxfp4(_bf16(x))
    codes = F.unpack_e2m1(qp)
    assert sc[0].tolist() == [255, 126, 127] and np.all(codes[0, :32] == 0)
    assert codes[0, 40] == 7                    # 3 / 2^-1 = 6
    assert sc[1].tolist() == [127, 127, 255] and np.all(codes[1, 64:] == 0)
    assert sc[2].tolist() == [255, 127, 124]    # 127 + floor(log2 0.5) - 2
    assert np.all(codes[2, :32] == 0)
    assert np.all(codes[2, 64:] == 6)           # 0.5 / 2^-3 = 4, grid code 6
    # decoding: NaN for the marked blocks only
    dec = F.e2m1_decode(codes) * np.repeat(F.e8m0_decode(sc), 32, axis=1)
    assert np.all(np.isnan(dec[0, :32])) and np.all(np.isfinite(dec[0, 32:]))
    assert np.all(np.isnan(dec[1, 64:])) and np.all(np.isfinite(dec[1, :64]))


def test_mxfp4_non_finite_block_through_the_gemm():
    """A NaN-scaled block of X makes its row of the output NaN, one of W its column; every
    other output equals the reference without the non-finite element's row or column."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 128))
    w = rng.standard_normal((4, 128)) * 0.05
    x[2, 33] = np.inf
    w[1, 100] = np.nan
    xq, sx = Q.quantize_mxfp4(_bf16(x))
    wq, sw = Q.quantize_mxfp4(_bf16(w))
    y = G.gemm_mxfp4_ref(xq, sx, wq, sw)
    assert np.all(np.isnan(y[2])) and np.all(np.isnan(y[:, 1]))
    keep_r = [0, 1, 3, 4]
    keep_c = [0, 2, 3]
    ref = G.gemm_mxfp4_ref(xq[keep_r], sx[keep_r], wq[keep_c], sw[keep_c])
    assert np.array_equal(y[np.ix_(keep_r, keep_c)], ref)


def test_mxfp4_zero_block():
    x = np.zeros((1, 64))
    x[0, 40] = 3.0
    qp, sc = Q.quantize_mxfp4(_bf16(x))
    assert sc[0, 0] == 127 and np.all(qp[0, :16] == 0)
    assert sc[0, 1] == 127 - 1                 # floor(log2 3) - 2 = -1
    assert F.unpack_e2m1(qp)[0, 40] == 7       # 3 / 2^-1 = 6
