"""Pins for oracle/formats.py: page values, exhaustive brute force and library casts."""

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests import golden

PV = golden.load("e4m3_page_values.txt")
MX = golden.load("mx_formats.txt")


# ----------------------------------------------------------------------------- helpers
def _positive_table():
    """All finite non-negative E4M3FN codes (0x00..0x7E) and their values, from decode."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return codes, F.e4m3_decode(codes)


def _nearest_code_bruteforce(v, codes, vals, maxv):
    """Nearest grid value to |v| after clamping to maxv; ties to the even code."""
    a = np.minimum(np.abs(v.astype(np.float64)), maxv)
    d = np.abs(a[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return codes[pick]


def _all_bf16_as_f32():
    b = np.arange(65536, dtype=np.uint32) << 16
    return b.view(np.float32)


# ----------------------------------------------------------------------------- E4M3 decode
def test_e4m3_page_values():
    assert F.e4m3_decode(golden.ints(PV, "max_finite_code"))[0] == golden.floats(PV, "max_finite")[0]
    assert F.e4m3_decode(golden.ints(PV, "neg_max_finite_code"))[0] == golden.floats(PV, "neg_max_finite")[0]
    for c in golden.ints(PV, "nan_codes"):
        assert np.isnan(F.e4m3_decode(c))
    assert F.e4m3_decode(golden.ints(PV, "min_normal_code"))[0] == golden.floats(PV, "min_normal")[0]
    one = golden.ints(PV, "one_code")[0]
    assert F.e4m3_decode(one) == 1.0
    assert F.e4m3_decode(one + 1) - F.e4m3_decode(one) == golden.floats(PV, "ulp_at_one")[0]
    z0, z1 = golden.ints(PV, "zero_codes")
    assert F.e4m3_decode(z0) == 0 and not np.signbit(F.e4m3_decode(z0))
    assert F.e4m3_decode(z1) == 0 and np.signbit(F.e4m3_decode(z1))
    assert F.e4m3_decode(0x01) == golden.floats(PV, "min_subnormal")[0]
    e, m, bias = (golden.ints(PV, k)[0] for k in ("max_exponent_field", "max_mantissa_field", "bias"))
    assert F.e4m3_decode((e << 3) | m) == (1 + m / 8) * 2.0 ** (e - bias) == 448.0


def test_e4m3_decode_structure():
    vals = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(vals).sum() == 2
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert np.array_equal(vals[0x80:0xFF], -pos)
    # 8 evenly spaced values per binade (3 mantissa bits)
    for e in range(1, 15):
        seg = pos[e * 8:(e + 1) * 8]
        assert np.allclose(np.diff(seg), seg[0] / 8)


def test_e4m3_decode_matches_torch_cast():
    c = torch.arange(256, dtype=torch.uint8)
    t = c.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(t), np.isnan(mine))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], mine[ok])
    assert np.array_equal(np.signbit(t[ok]), np.signbit(mine[ok]))


# ----------------------------------------------------------------------------- E4M3 encode
def test_e4m3_encode_exhaustive_bf16_vs_bruteforce():
    v = _all_bf16_as_f32()
    finite = np.isfinite(v)
    codes, vals = _positive_table()
    got = F.e4m3_encode(v)
    exp = _nearest_code_bruteforce(v[finite], codes, vals, 448.0)
    exp = np.where(np.signbit(v[finite]), exp | 0x80, exp).astype(np.uint8)
    assert np.array_equal(got[finite], exp)
    assert np.all(got[np.isnan(v)] == 0x7F)
    assert got[np.where(v == np.inf)[0][0]] == 0x7E
    assert got[np.where(v == -np.inf)[0][0]] == 0xFE


def test_e4m3_encode_midpoints_and_neighbours():
    codes, vals = _positive_table()
    mids = (vals[:-1] + vals[1:]) / 2                      # exact in fp32 (5 significant bits)
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)
    lo = np.nextafter(m32, np.float32(0))
    hi = np.nextafter(m32, np.float32(np.inf))
    # a tie goes to the even code of the pair
    exp_mid = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])
    assert np.array_equal(F.e4m3_encode(m32), exp_mid)
    assert np.array_equal(F.e4m3_encode(lo), codes[:-1])
    assert np.array_equal(F.e4m3_encode(hi), codes[1:])
    assert np.array_equal(F.e4m3_encode(-m32), exp_mid | 0x80)
    # saturation: everything from 448 up maps to 0x7E
    big = np.array([448.0, 460.0, 463.99, 464.0, 470.0, 1e6, 3e38], np.float32)
    assert np.all(F.e4m3_encode(big) == 0x7E)
    assert np.all(F.e4m3_encode(-big) == 0xFE)


def test_e4m3_round_trip():
    c = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(c)), c)


def test_e4m3_relative_error_bound():
    rng = np.random.default_rng(0)
    v = np.exp2(rng.uniform(-6, np.log2(448), 200000)).astype(np.float32)
    v = np.concatenate([v, _all_bf16_as_f32()])
    v = v[(np.abs(v) >= 2.0 ** -6) & (np.abs(v) <= 448)]
    q = F.e4m3_decode(F.e4m3_encode(v))
    rel = np.abs(q - v) / np.abs(v)
    assert rel.max() <= golden.floats(PV, "rel_err_bound_e4m3")[0]


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(100000) * 50,
        np.exp2(rng.uniform(-14, 8.8, 100000)) * rng.choice([-1, 1], 100000),
    ]).astype(np.float32)
    v = np.clip(v, -448, 448)          # the torch cast does not saturate, so stay in range
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(v), t)


def test_worked_example_fp8_unscaled():
    ex = golden.load("fp8_int8_tiny_example.txt")
    x = np.array(golden.floats(ex, "input"))
    q = F.e4m3_decode(F.e4m3_encode(x))
    assert [f"{v:.4f}" for v in q] == ex["fp8_dequant"]
    assert [f"{abs((a - b) / b):.3f}" for a, b in zip(q, x)] == ex["fp8_rel_err"]


# ----------------------------------------------------------------------------- E2M1 / E8M0
def test_e2m1_table_from_page():
    mags = golden.floats(MX, "e2m1_magnitudes")
    vals = F.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == mags
    assert np.array_equal(vals[8:], -np.array(mags))
    assert np.signbit(vals[8])
    # the grid of fp_round(x, 1, 0, 6): step 0.5 below 2, 1 in [2,4), 2 in [4,8), max 6
    assert np.array_equal(F.fp_round(np.array(mags), 1, 0, 6.0), mags)


def test_e2m1_encode_exhaustive_bf16_vs_bruteforce():
    v = _all_bf16_as_f32()
    finite = np.isfinite(v)
    codes = np.arange(8, dtype=np.uint8)
    vals = F.e2m1_decode(codes)
    exp = _nearest_code_bruteforce(v[finite], codes, vals, 6.0)
    exp = np.where(np.signbit(v[finite]), exp | 8, exp).astype(np.uint8)
    assert np.array_equal(F.e2m1_encode(v[finite]), exp)


def test_e2m1_relative_error_bound():
    v = np.linspace(1.0, 6.0, 100001)
    q = F.e2m1_decode(F.e2m1_encode(v))
    assert (np.abs(q - v) / v).max() <= golden.floats(PV, "rel_err_bound_e2m1")[0]


def test_e2m1_pack_order():
    codes = np.array([[1, 2, 3, 4, 15, 0]], np.uint8)
    p = F.pack_e2m1(codes)
    assert p.tolist() == [[0x21, 0x43, 0x0F]]
    assert np.array_equal(F.unpack_e2m1(p), codes)


def test_e8m0_decode_and_torch_cast():
    bias = golden.ints(MX, "mxfp4_scale_bias")[0]
    c = np.arange(256, dtype=np.uint8)
    d = F.e8m0_decode(c)
    assert d[bias] == 1.0 and d[bias + 1] == 2.0 and d[bias - 1] == 0.5 and np.isnan(d[255])
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(d[:255], t[:255]) and np.isnan(t[255])


def test_mx_bits_per_weight():
    blk = golden.ints(MX, "mxfp4_block")[0]
    assert (4 * blk + 8) / blk == golden.floats(MX, "mxfp4_bpw")[0]
    nblk = golden.ints(MX, "nvfp4_block")[0]
    assert (4 * nblk + 8) / nblk == golden.floats(MX, "nvfp4_bpw")[0]


# ----------------------------------------------------------------------------- bfloat16
def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, size=400000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half 0x8000) with both parities of the kept LSB
    ties = (rng.integers(0, 2 ** 16, size=20000).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties])
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    t = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f64_to_bf16_rne(v.astype(np.float64)), t)


def test_bf16_widen_exact():
    b = np.arange(65536, dtype=np.uint16)
    f = F.bf16_to_f64(b)
    ok = ~np.isnan(f)
    assert np.array_equal(F.f64_to_bf16_rne(f[ok]), b[ok])
