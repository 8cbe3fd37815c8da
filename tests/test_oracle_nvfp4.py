"""Pins for oracle/nvfp4.py: hand-computed blocks, nearest-value brute force, the storage
cost printed on [P-LOWBIT] §2.4, the zero-scale rule of the [P-FP8FP4] emulation, and a
triple-loop GEMM."""

import math

import numpy as np

import synthetic
from oracle import formats as F
from oracle import nvfp4 as N
from oracle import quant as Q

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
SIGNED_GRID = GRID + [-v for v in GRID]            # 16 values: one block
GRID_CODES = list(range(8)) + [8 | c for c in range(8)]


def _bf16(v):
    return synthetic.to_bf16_bits(np.asarray(v, np.float64))


def _nearest_code(v: float, table, vmax: float) -> int:
    """Index of the nearest entry of a non-negative value table to |v| (|v| clamped to
    vmax), ties to the even index."""
    a = min(abs(v), vmax)
    return min(range(len(table)), key=lambda i: (abs(table[i] - a), i & 1))


def test_grid_blocks_scaled_by_powers_of_two():
    """A block holding the E2M1 grid times 2^-k has scale code 0x7E - 8k (448 * 2^-k) and
    element codes equal to the grid's, when the tensor's amax is 6 (g = 6 / 2688)."""
    ks = [0, 3, 10, 14]
    rows = [np.concatenate([np.array(SIGNED_GRID) * 2.0 ** -k for k in ks[:2]]),
            np.concatenate([np.array(SIGNED_GRID) * 2.0 ** -k for k in ks[2:]])]
    xb = _bf16(np.array(rows))
    packed, scodes, g = N.quantize_nvfp4(xb)
    assert g == np.float32(6.0) / np.float32(2688.0)
    assert scodes.tolist() == [[0x7E, 0x7E - 24], [0x7E - 80, 0x7E - 112]]
    codes = F.unpack_e2m1(packed)
    for r in range(2):
        for b in range(2):
            assert codes[r, 16 * b:16 * b + 16].tolist() == GRID_CODES
    deq = N.dequantize_nvfp4(packed, scodes, g)
    x = F.bf16_to_f64(xb)
    assert np.all(np.abs(deq - x) <= 1e-6 * np.abs(x))


def test_block_scale_and_elements_are_nearest_values():
    """Each block's scale code is the E4M3 value nearest to (amax_b / 6) / g, and each
    element code is the E2M1 value nearest to x / s_b, both with ties to the even code."""
    rng = np.random.default_rng(5)
    v = rng.standard_normal((6, 64)) * np.exp2(rng.uniform(-12, 12, (6, 4))).repeat(16, axis=1)
    v[2, 5] = 0.0
    xb = _bf16(v)
    packed, scodes, g = N.quantize_nvfp4(xb)
    x = F.bf16_to_f32(xb)
    e4m3_table = [float(F.e4m3_decode(c)) for c in range(0x7F)]
    codes = F.unpack_e2m1(packed)
    for r in range(6):
        for b in range(4):
            blk = x[r, 16 * b:16 * b + 16]
            amax = np.float32(np.max(np.abs(blk)))
            t = np.float32(np.float32(amax / np.float32(6.0)) / g)
            assert scodes[r, b] == _nearest_code(float(t), e4m3_table, 448.0)
            s = np.float32(np.float32(e4m3_table[scodes[r, b]]) * g)
            s = np.float32(1.0) if s == 0 else s
            for i in range(16):
                q = float(np.float32(blk[i] / s))
                want = _nearest_code(q, GRID, 6.0) | (8 if math.copysign(1.0, q) < 0 else 0)
                assert codes[r, 16 * b + i] == want, (r, b, i, q)


def test_tensor_max_encodes_to_six_with_scale_448():
    rng = np.random.default_rng(11)
    xb = _bf16(rng.standard_normal((8, 128)) * 3.0)
    packed, scodes, g = N.quantize_nvfp4(xb)
    x = F.bf16_to_f64(xb)
    r, k = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert scodes[r, k // 16] == 0x7E
    assert F.unpack_e2m1(packed)[r, k] & 7 == 7
    deq = N.dequantize_nvfp4(packed, scodes, g)
    assert abs(deq[r, k] - x[r, k]) <= 1e-6 * abs(x[r, k])


def test_error_at_most_one_grid_half_step():
    """|x - dequant| <= s_b for unsaturated elements (the widest E2M1 step below 6 is 2)."""
    rng = np.random.default_rng(12)
    xb = _bf16(rng.standard_normal((16, 256)) * np.exp2(rng.uniform(-6, 6, (16, 1))))
    packed, scodes, g = N.quantize_nvfp4(xb)
    s = np.repeat(N.block_scales(scodes, g).astype(np.float64), 16, axis=1)
    err = np.abs(N.dequantize_nvfp4(packed, scodes, g) - F.bf16_to_f64(xb))
    assert np.all(err <= s * (1 + 1e-6))


def test_storage_is_four_and_a_half_bits_per_element():
    """[P-LOWBIT] §2.4: 8-bit scale per 16 elements = 0.5 bpw, 4.5 bpw in all."""
    xb = _bf16(np.ones((4, 256)))
    packed, scodes, _ = N.quantize_nvfp4(xb)
    assert (packed.nbytes + scodes.nbytes) * 8 / xb.size == 4.5


def test_zero_tensor_and_zero_scale_rule():
    packed, scodes, g = N.quantize_nvfp4(_bf16(np.zeros((2, 32))))
    assert g == 1.0 and not packed.any() and not scodes.any()
    # A block whose scale rounds to E4M3 zero uses s = 1 ([P-FP8FP4] nvfp4): with a tensor
    # amax of 2^20, g = 2^20 / 2688 and (1 / 6) / g = 4.3e-4 < 2^-10, so a block of ones has
    # scale code 0, s = 1, and keeps its ones exactly (E2M1 code 2).
    v = np.ones((1, 32))
    v[0, 0] = 2.0 ** 20
    packed, scodes, g = N.quantize_nvfp4(_bf16(v))
    assert g == np.float32(2.0 ** 20) / np.float32(2688.0)
    assert scodes[0, 1] == 0
    assert F.unpack_e2m1(packed)[0, 16:].tolist() == [2] * 16
    assert N.dequantize_nvfp4(packed, scodes, g)[0, 16:].tolist() == [1.0] * 16


def test_supplied_tensor_scale_saturates():
    """g four times below the natural one: t = 4 * 448 saturates to code 0x7E, s = 448 g =
    100 / 24, and 100 / s = 24 saturates to E2M1 6 (code 7), i.e. 25."""
    xb = _bf16(np.full((1, 16), 100.0))
    g = np.float32(np.float32(100.0) / np.float32(2688.0)) / np.float32(4.0)
    packed, scodes, g_out = N.quantize_nvfp4(xb, g=g)
    assert g_out == g and scodes[0, 0] == 0x7E
    assert F.unpack_e2m1(packed)[0].tolist() == [7] * 16
    assert np.allclose(N.dequantize_nvfp4(packed, scodes, g), 25.0, rtol=1e-6)


def test_nvfp4_error_below_mxfp4():
    """[P-FP8FP4] measured NVFP4 well below MXFP4 (KL 0.25 vs 0.84); on the same synthetic
    activations (outlier channels, per-token ranges) NVFP4's squared error is lower."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((256, 1024)) * np.exp2(rng.uniform(-3, 3, (256, 1)))
    v[:, rng.choice(1024, 4, replace=False)] *= 100.0
    x = _bf16(v)
    ref = F.bf16_to_f64(x)
    p, s, g = N.quantize_nvfp4(x)
    e_nv = np.sum((N.dequantize_nvfp4(p, s, g) - ref) ** 2)
    pm, sm = Q.quantize_mxfp4(x)
    deq_mx = F.e2m1_decode(F.unpack_e2m1(pm)) * np.repeat(F.e8m0_decode(sm), 32, axis=1)
    e_mx = np.sum((deq_mx - ref) ** 2)
    assert e_nv < 0.7 * e_mx, (e_nv, e_mx)


def test_gemm_matches_triple_loop():
    rng = np.random.default_rng(21)
    xb = _bf16(rng.standard_normal((3, 48)) * np.exp2(rng.uniform(-4, 4, (3, 1))))
    wb = _bf16(rng.standard_normal((5, 48)) * 0.02)
    xq, xs, gx = N.quantize_nvfp4(xb)
    wq, ws, gw = N.quantize_nvfp4(wb)
    y = N.gemm_nvfp4_ref(xq, xs, gx, wq, ws, gw)
    a = F.e2m1_decode(F.unpack_e2m1(xq))
    b = F.e2m1_decode(F.unpack_e2m1(wq))
    sa = N.block_scales(xs, gx).astype(np.float64)
    sb = N.block_scales(ws, gw).astype(np.float64)
    for m in range(3):
        for n in range(5):
            acc = 0.0
            for blk in range(3):
                part = sum(a[m, k] * b[n, k] for k in range(16 * blk, 16 * blk + 16))
                acc += sa[m, blk] * sb[n, blk] * part
            assert math.isclose(y[m, n], acc, rel_tol=1e-12, abs_tol=1e-300)


def test_gemm_of_grid_values_is_the_plain_product():
    rng = np.random.default_rng(22)
    xv = rng.choice(SIGNED_GRID, size=(4, 64))
    wv = rng.choice(SIGNED_GRID, size=(6, 64)) * 0.25
    xv[:, ::16], wv[:, ::16] = 6.0, 1.5               # every block's amax: 6 and 6 / 4
    xq, xs, gx = N.quantize_nvfp4(_bf16(xv))
    wq, ws, gw = N.quantize_nvfp4(_bf16(wv))
    y = N.gemm_nvfp4_ref(xq, xs, gx, wq, ws, gw)
    exact = xv @ wv.T
    assert np.all(np.abs(y - exact) <= 1e-5 * (np.abs(exact) + 1))
