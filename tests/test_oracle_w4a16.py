"""Pins for oracle/w4a16.py: the metadata sizes printed on [P-LOWBIT] §2.3 and §3.3, a
hand-computed group, nearest-integer brute force, two's-complement packing, and a
triple-loop GEMM."""

import math

import numpy as np

import synthetic
from oracle import w4a16 as W


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def test_metadata_sizes_printed_on_the_page():
    """4096 x 4096 at G = 128: 262,144 bytes of scales (3.125%); the layer reads 8.25 MiB
    instead of 32 MiB in fp16 (3.88x). At G = 32: 1,048,576 bytes (12.5%)."""
    w = _bf16(np.ones((4096, 4096)))
    packed, s = W.quantize_int4_groups(w)
    assert s.nbytes == 262_144
    assert s.nbytes / packed.nbytes == 0.03125
    assert (packed.nbytes + s.nbytes) / 2**20 == 8.25
    assert round(4096 * 4096 * 2 / (packed.nbytes + s.nbytes), 2) == 3.88
    _, s32 = W.quantize_int4_groups(_bf16(np.ones((64, 256))), group=32)
    assert s32.nbytes / (64 * 256 / 2) == 0.125


def test_hand_computed_group():
    """amax 7 -> S = 1; 7 -> 7, -3.5 (tie) -> -4, 1.75 -> 2, 0.5 (tie) -> 0, -0.75 -> -1,
    2.5 (tie) -> 2, -7 -> -7; the rest of the group is zero."""
    row = np.zeros(128)
    row[:7] = [7.0, -3.5, 1.75, 0.5, -0.75, 2.5, -7.0]
    packed, s = W.quantize_int4_groups(_bf16(row[None, :]))
    assert s[0, 0] == np.float16(1.0)
    assert W.unpack_int4(packed)[0, :8].tolist() == [7, -4, 2, 0, -1, 2, -7, 0]
    # scale rounding to fp16: amax 1.0 -> S = fp16(1/7) = 0.14282..., 1.0 / S = 7.0017 -> 7
    packed, s = W.quantize_int4_groups(_bf16(np.full((1, 128), 1.0)))
    assert s[0, 0] == np.float16(1.0 / 7.0) and W.unpack_int4(packed)[0, 0] == 7


def test_codes_are_nearest_integers_to_x_over_stored_scale():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((5, 256)) * np.exp2(rng.uniform(-10, 10, (5, 2))).repeat(128, axis=1)
    xb = _bf16(v)
    packed, s = W.quantize_int4_groups(xb)
    q = W.unpack_int4(packed)
    x = synthetic.bf16_bits_to_f32(xb)
    for r in range(5):
        for g in range(2):
            sc = np.float32(s[r, g])
            assert sc == np.float32(np.float16(np.float32(np.max(np.abs(x[r, 128 * g:128 * g + 128]))) / np.float32(7)))
            for k in range(128 * g, 128 * g + 128):
                t = float(np.float32(x[r, k] / sc))
                want = min(range(-7, 8), key=lambda c: (abs(c - t), c & 1))
                assert q[r, k] == want, (r, k, t)
            assert np.max(np.abs(q[r, 128 * g:128 * g + 128])) == 7


def test_packing_is_twos_complement_low_nibble_first():
    row = np.zeros(128)
    row[:4] = [-7.0, 7.0, -1.0, 3.0]
    packed, _ = W.quantize_int4_groups(_bf16(row[None, :]))
    assert packed[0, 0] == (0x9 | (0x7 << 4)) and packed[0, 1] == (0xF | (0x3 << 4))


def test_zero_group_and_saturating_scale():
    v = np.zeros((1, 256))
    v[0, 128:] = 1e6                                  # amax / 7 = 142857 > 65504
    packed, s = W.quantize_int4_groups(_bf16(v))
    assert s[0, 0] == np.float16(1.0) and not W.unpack_int4(packed)[0, :128].any()
    assert s[0, 1] == np.float16(65504.0)
    assert (W.unpack_int4(packed)[0, 128:] == 7).all()     # 1e6 / 65504 = 15.3 -> 7


def test_dequantized_error_at_most_half_a_step():
    rng = np.random.default_rng(6)
    xb = _bf16(rng.standard_normal((8, 512)) * 0.02)
    packed, s = W.quantize_int4_groups(xb)
    err = np.abs(W.dequantize_int4(packed, s) - synthetic.bf16_bits_to_f32(xb))
    step = np.repeat(s.astype(np.float64), 128, axis=1)
    assert np.all(err <= 0.5 * step * (1 + 1e-3) + 1e-12)


def test_gemm_matches_triple_loop():
    rng = np.random.default_rng(7)
    xb = _bf16(rng.standard_normal((3, 256)))
    wb = _bf16(rng.standard_normal((4, 256)) * 0.02)
    packed, s = W.quantize_int4_groups(wb)
    y = W.gemm_w4a16_ref(xb, packed, s)
    x = synthetic.bf16_bits_to_f32(xb).astype(np.float64)
    q = W.unpack_int4(packed)
    for m in range(3):
        for n in range(4):
            acc = 0.0
            for g in range(2):
                acc += float(s[n, g]) * sum(x[m, k] * q[n, k] for k in range(128 * g, 128 * g + 128))
            assert math.isclose(y[m, n], acc, rel_tol=1e-12, abs_tol=1e-300)
