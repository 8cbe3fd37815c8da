"""Pins for oracle/roofline.py: the numbers the pages print."""

from oracle import roofline as R
from tests import golden

V = golden.load("roofline_values.txt")


def f(k):
    return golden.floats(V, k)


def test_8b_step_bounds():
    P, beta = f("params")[0], f("beta")[0]
    pib, pif = f("pi_bf16")[0], f("pi_fp8")[0]
    pis = [pib, pib, pif]
    for bits, pi, ms in zip(f("batch1_bits"), pis, f("batch1_ms")):
        assert round(R.step_time_lower_bound(P, 1, bits, beta, pi) * 1e3, 2) == ms
    # batch 512: bf16, W4A16 (16-bit math) and FP8
    for bits, pi, ms in zip([16, 4.25, 8], [pib, pib, pif], f("batch512_ms")):
        assert round(R.step_time_lower_bound(P, 512, bits, beta, pi) * 1e3, 2) == ms


def test_ridges_and_crossover():
    r = [R.ridge_point(f("a100_fp16")[0], f("a100_bw")[0]), R.ridge_point(f("a100_int8")[0], f("a100_bw")[0]),
         R.ridge_point(f("h100_fp16")[0], f("h100_bw")[0]), R.ridge_point(f("h100_fp8")[0], f("h100_bw")[0])]
    assert [round(v) for v in r] == [int(v) for v in f("ridge")]
    b = [R.crossover_batch(f("a100_fp16")[0], f("a100_bw")[0]), R.crossover_batch(f("h100_fp16")[0], f("h100_bw")[0])]
    assert [round(v, 1) for v in b] == f("bstar")
    eta = f("eta")[0]
    # batch where W4A16's intensity reaches the (rounded) fp16 ridge
    ceil = [153 / R.intensity_w4a16(1, eta), 295 / R.intensity_w4a16(1, eta)]
    assert [round(v, 1) for v in ceil] == f("w4a16_ceiling_batch")
    assert round(R.intensity_w4a16(32, eta)) == f("tryit04_i_w4a16")[0]
    assert R.intensity_w8a8(32) == f("tryit04_i_fp8")[0]


def test_metadata_overheads():
    n = 4096
    b8 = R.scale_overhead_bytes(n, n, None, 2)
    assert b8 == f("int8_per_channel_bytes")[0]
    assert round(100 * b8 / (n * n), 4) == f("int8_per_channel_pct")[0]
    b128 = R.scale_overhead_bytes(n, n, 128, 2)
    b32 = R.scale_overhead_bytes(n, n, 32, 2)
    payload4 = n * n // 2
    assert b128 == f("int4_g128_bytes")[0] and 100 * b128 / payload4 == f("int4_g128_pct")[0]
    assert b32 == f("int4_g32_bytes")[0] and 100 * b32 / payload4 == f("int4_g32_pct")[0]
    assert (payload4 + b128) / 2 ** 20 == f("int4_g128_total_mib")[0]
    assert round(n * n * 2 / (payload4 + b128), 2) == f("int4_g128_compression")[0]


def test_gemm_flops():
    assert R.gemm_flops(2048, 6144, 4096) == 2 * 2048 * 6144 * 4096
