"""C-ABI host tests (no GPU): the library loads, exports every call declared in
include/w8a8.h, and rejects bad arguments on the host before enqueuing anything."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

import fp4_w8a8_quantized_amd as w8  # noqa: E402

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EHIP, EARG = range(7)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w8.library_path):
        pytest.fail("libw8a8.so is not built (run __graft_entry__.build())")
    return w8.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:w8a8_status|const char\*)\s+(w8a8_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["w8a8_quantize_per_token", "w8a8_quantize_weight_per_channel", "w8a8_gemm", "w8a8_linear",
              "w8a8_gemm_ex",
              "w8a8_quantize_per_token_group", "w8a8_quantize_weight_block", "w8a8_gemm_blockscaled",
              "w8a8_quantize_mxfp4", "w8a8_gemm_mxfp4", "w8a8_channel_absmax",
              "w8a8_smoothquant_scales", "w8a8_smooth_apply", "w8a8_status_string",
              "w8a8_quantize_nvfp4", "w8a8_gemm_nvfp4", "w8a8_quantize_int4", "w8a8_gemm_w4a16"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) - {"w8a8_status_string"} == set(w8._SIGNATURES)


def test_status_strings(L):
    assert w8.status_string(OK) == "ok"
    for s in range(1, 7):
        assert w8.status_string(s) not in ("ok", "unknown status")
    assert w8.status_string(99) == "unknown status"


# Fake, never-dereferenced addresses: validation must fail before any launch.
A = 0x10000          # 16-byte aligned
MIS = 0x10008        # 8-byte aligned only


def test_quantize_validation(L):
    q = L.w8a8_quantize_per_token
    assert q(None, 4, 128, 0, A, A, None) == ENULL
    assert q(A, 4, 128, 0, None, A, None) == ENULL
    assert q(A, 4, 128, 0, A, None, None) == ENULL
    assert q(A, -1, 128, 0, A, A, None) == ESHAPE
    assert q(A, 4, -16, 0, A, A, None) == ESHAPE
    assert q(A, 4, 100, 0, A, A, None) == EUNSUP          # K % 16 != 0
    assert q(A, 4, 128, 7, A, A, None) == EUNSUP          # unknown format
    assert q(MIS, 4, 128, 0, A, A, None) == EALIGN
    assert q(A, 4, 128, 1, A, MIS, None) == EALIGN
    assert q(A, 1 << 40, 1 << 20, 0, A, A, None) == ESHAPE
    assert q(None, 0, 128, 0, None, None, None) == OK     # empty: nothing to do
    w = L.w8a8_quantize_weight_per_channel
    assert w(None, 4, 128, 0, A, A, None) == ENULL
    assert w(A, 4, 40, 1, A, A, None) == EUNSUP


def test_gemm_validation(L):
    g = L.w8a8_gemm
    assert g(None, A, A, A, 4, 4, 128, 0, A, None) == ENULL
    assert g(A, A, A, A, 4, 4, 128, 0, None, None) == ENULL
    assert g(A, A, A, A, 4, 4, 100, 0, A, None) == EUNSUP   # K % 128
    assert g(A, A, A, A, 4, 4, 0, 0, A, None) == EUNSUP     # K == 0
    assert g(A, A, A, A, 4, 4, 128, 3, A, None) == EUNSUP   # format
    assert g(A, A, A, A, -4, 4, 128, 0, A, None) == ESHAPE
    assert g(A, A, A, A, 4, 1 << 40, 128, 0, A, None) == ESHAPE
    assert g(A, A, MIS, A, 4, 4, 128, 0, A, None) == EALIGN
    assert g(A, A, A, A, 4, 4, 128, 0, MIS, None) == EALIGN
    assert g(None, None, None, None, 0, 4, 128, 0, None, None) == OK
    assert g(None, None, None, None, 4, 0, 128, 1, None, None) == OK


def test_linear_validation(L):
    f = L.w8a8_linear
    ok = (A, A, A, 4, 4, 128, 0, A, A, A, None)
    assert f(None, *ok[1:]) == ENULL                                   # x
    assert f(A, A, A, 4, 4, 128, 0, None, A, A, None) == ENULL         # xq
    assert f(A, A, A, 4, 4, 128, 0, A, None, A, None) == ENULL         # sx
    assert f(A, A, A, 4, 4, 128, 0, A, A, None, None) == ENULL         # y
    assert f(A, A, A, 4, 4, 100, 0, A, A, A, None) == EUNSUP           # K % 128
    assert f(A, A, A, 4, 4, 128, 2, A, A, A, None) == EUNSUP           # format
    assert f(A, A, A, -1, 4, 128, 0, A, A, A, None) == ESHAPE
    assert f(A, A, A, 1 << 40, 4, 1 << 20, 0, A, A, A, None) == ESHAPE
    assert f(MIS, *ok[1:]) == EALIGN
    assert f(A, A, A, 4, 4, 128, 0, MIS, A, A, None) == EALIGN
    assert f(None, None, None, 0, 4, 128, 0, None, None, None, None) == OK
    assert f(None, None, None, 4, 0, 128, 1, None, None, None, None) == OK


def test_gemm_ex_validation(L):
    g = L.w8a8_gemm_ex
    ok_args = (A, A, A, A, 4, 4, 128, 0)
    assert g(*ok_args, None, 3, 0, 1.0, A, None) == EUNSUP              # activation
    assert g(*ok_args, None, 0, 2, 1.0, A, None) == EUNSUP              # output format
    assert g(*ok_args[:7], 5, None, 0, 0, 1.0, A, None) == EUNSUP        # operand format
    assert g(*ok_args, None, 0, 1, 0.0, A, None) == EARG                # out_scale <= 0
    assert g(*ok_args, None, 0, 1, -2.0, A, None) == EARG
    assert g(*ok_args, None, 0, 1, float("nan"), A, None) == EARG
    assert g(*ok_args, None, 0, 1, float("inf"), A, None) == EARG
    assert g(*ok_args, MIS, 1, 0, 1.0, A, None) == EALIGN               # bias alignment
    assert g(A, A, A, A, 4, 4, 100, 0, None, 0, 0, 1.0, A, None) == EUNSUP   # K % 128
    assert g(A, A, A, A, 4, 4, 128, 0, None, 0, 0, 1.0, None, None) == ENULL
    assert g(None, None, None, None, 0, 4, 128, 0, None, 2, 1, 1.0, None, None) == OK


def test_static_validation(L):
    q = L.w8a8_quantize_static
    assert q(A, 4, 64, 3, A, A, None, None, None) == EUNSUP             # format
    assert q(A, 4, 60, 0, A, A, None, None, None) == EUNSUP             # K % 8
    assert q(None, 4, 64, 0, A, A, None, None, None) == ENULL
    assert q(A, 4, 64, 0, None, A, None, None, None) == ENULL           # scale
    assert q(A, 4, 64, 0, A, None, None, None, None) == ENULL
    assert q(MIS, 4, 64, 0, A, A, None, None, None) == EALIGN
    assert q(A, 4, 64, 0, 0x10002, A, None, None, None) == EALIGN       # scale 2-byte aligned
    assert q(A, 4, 64, 1, A, A, 0x10001, None, None) == EALIGN
    assert q(A, -1, 64, 0, A, A, None, None, None) == ESHAPE
    assert q(None, 0, 64, 0, None, None, None, None, None) == OK
    d = L.w8a8_delayed_scale_update
    assert d(A, 0, A, 0, 0, A, None) == EARG                            # H >= 1
    assert d(A, 1 << 25, A, 0, 0, A, None) == EARG
    assert d(A, 4, A, -1, 0, A, None) == EARG                           # step >= 0
    assert d(A, 4, A, 0, 2, A, None) == EUNSUP
    assert d(None, 4, A, 0, 0, A, None) == ENULL
    assert d(A, 4, None, 0, 0, A, None) == ENULL
    assert d(A, 4, A, 0, 0, 0x10002, None) == EALIGN


def test_blockscaled_validation(L):
    assert L.w8a8_quantize_per_token_group(A, 4, 100, A, A, None) == EUNSUP
    assert L.w8a8_quantize_per_token_group(None, 4, 128, A, A, None) == ENULL
    assert L.w8a8_quantize_weight_block(A, 4, 192, A, A, None) == EUNSUP
    assert L.w8a8_quantize_weight_block(A, 4, 256, A, MIS, None) == EALIGN
    assert L.w8a8_gemm_blockscaled(A, A, A, A, 4, 4, 64, A, None) == EUNSUP
    assert L.w8a8_gemm_blockscaled(A, None, A, A, 4, 4, 128, A, None) == ENULL


def test_mxfp4_validation(L):
    assert L.w8a8_quantize_mxfp4(A, 4, 48, A, A, None) == EUNSUP
    assert L.w8a8_quantize_mxfp4(A, 4, 64, None, A, None) == ENULL
    assert L.w8a8_gemm_mxfp4(A, A, A, A, 4, 4, 128, A, None) == EUNSUP   # K % 256
    assert L.w8a8_gemm_mxfp4(A, A, A, A, 4, 4, 256, None, None) == ENULL
    assert L.w8a8_gemm_mxfp4(A, MIS, A, A, 4, 4, 256, A, None) == EALIGN


def test_nvfp4_validation(L):
    qn = L.w8a8_quantize_nvfp4
    assert qn(A, 4, 40, 0, A, A, A, None) == EUNSUP          # K % 16
    assert qn(A, 4, 64, 2, A, A, A, None) == EUNSUP          # scale mode
    assert qn(A, 4, 64, 0, A, A, None, None) == ENULL        # g
    assert qn(A, 4, 64, 1, A, None, A, None) == ENULL
    assert qn(A, 4, 64, 0, A, A, 0x10002, None) == EALIGN    # g 4-byte aligned
    assert qn(A, 4, 64, 0, MIS, A, A, None) == EALIGN
    assert qn(A, -1, 64, 0, A, A, A, None) == ESHAPE
    assert qn(None, 0, 64, 0, None, None, None, None) == OK  # empty: nothing written
    gn = L.w8a8_gemm_nvfp4
    assert gn(A, A, A, A, A, A, 4, 4, 96, A, None) == EUNSUP   # K % 64
    assert gn(A, A, None, A, A, A, 4, 4, 64, A, None) == ENULL
    assert gn(A, A, A, A, A, 0x10002, 4, 4, 64, A, None) == EALIGN
    assert gn(A, MIS, A, A, A, A, 4, 4, 64, A, None) == EALIGN
    assert gn(A, A, A, A, A, A, 0, 4, 64, A, None) == OK


def test_w4a16_validation(L):
    assert L.w8a8_quantize_int4(A, 4, 64, A, A, None) == EUNSUP        # K % 128
    assert L.w8a8_quantize_int4(A, 4, 128, None, A, None) == ENULL
    assert L.w8a8_quantize_int4(A, 4, 128, A, MIS, None) == EALIGN
    assert L.w8a8_quantize_int4(None, 0, 128, None, None, None) == OK
    assert L.w8a8_gemm_w4a16(A, A, A, 1, 4, 64, A, None) == EUNSUP
    assert L.w8a8_gemm_w4a16(A, A, None, 1, 4, 128, A, None) == ENULL
    assert L.w8a8_gemm_w4a16(A, A, A, 1, 4, 128, MIS, None) == EALIGN
    assert L.w8a8_gemm_w4a16(A, A, A, -1, 4, 128, A, None) == ESHAPE
    assert L.w8a8_gemm_w4a16(None, None, None, 0, 4, 128, None, None) == OK


def test_smoothquant_validation(L):
    assert L.w8a8_smoothquant_scales(A, A, 8, ctypes.c_float(1.5), A, None) == EARG
    assert L.w8a8_smoothquant_scales(A, A, 8, ctypes.c_float(-0.1), A, None) == EARG
    assert L.w8a8_smoothquant_scales(A, A, 8, ctypes.c_float(float("nan")), A, None) == EARG
    assert L.w8a8_smoothquant_scales(None, A, 8, ctypes.c_float(0.5), A, None) == ENULL
    assert L.w8a8_smooth_apply(A, 4, 8, A, 2, A, None) == EARG
    assert L.w8a8_smooth_apply(A, 4, 12, A, 0, A, None) == EUNSUP
    assert L.w8a8_smooth_apply(A, 4, 8, None, 0, A, None) == ENULL
    assert L.w8a8_channel_absmax(A, 4, 12, A, None) == EUNSUP
    assert L.w8a8_channel_absmax(A, 4, 8, None, None) == ENULL


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w8.quantize_per_token(x)


def test_operand_byte_limit(L):
    """One row past 2^31 bytes of any operand is a shape error, checked before launch."""
    lim = 1 << 31
    K = 16384
    assert L.w8a8_gemm(A, A, A, A, 4, lim // K + 1, K, 0, A, None) == ESHAPE
    assert L.w8a8_gemm(A, A, A, A, lim // K + 1, 4, K, 1, A, None) == ESHAPE
    assert L.w8a8_gemm_blockscaled(A, A, A, A, 4, lim // K + 1, K, A, None) == ESHAPE
    K = 32768
    assert L.w8a8_gemm_mxfp4(A, A, A, A, 4, lim // (K // 2) + 1, K, A, None) == ESHAPE
    assert L.w8a8_gemm_nvfp4(A, A, A, A, A, A, 4, lim // (K // 2) + 1, K, A, None) == ESHAPE
    assert L.w8a8_gemm_w4a16(A, A, A, 4, lim // (K // 2) + 1, K, A, None) == ESHAPE
    assert L.w8a8_gemm_w4a16(A, A, A, lim // (2 * K) + 1, 4, K, A, None) == ESHAPE
    assert L.w8a8_quantize_per_token(A, lim // (2 * K) + 1, K, 0, A, A, None) == ESHAPE
    assert L.w8a8_quantize_int4(A, lim // (2 * K) + 1, K, A, A, None) == ESHAPE


def test_sclk_probe_validation(L):
    assert L.w8a8_sclk_probe(A, 0, 100, None) == EARG
    assert L.w8a8_sclk_probe(A, 1025, 100, None) == EARG
    assert L.w8a8_sclk_probe(A, 8, 0, None) == EARG
    assert L.w8a8_sclk_probe(A, 8, (1 << 32) + 1, None) == EARG
    assert L.w8a8_sclk_probe(None, 8, 100, None) == ENULL
    assert L.w8a8_sclk_probe(A + 8, 8, 100, None) == EALIGN


def test_stream_probe_validation(L):
    assert L.w8a8_stream_probe(A, -8, A, None) == ESHAPE
    assert L.w8a8_stream_probe(A, 12, A, None) == EUNSUP
    assert L.w8a8_stream_probe(None, 16, A, None) == ENULL
    assert L.w8a8_stream_probe(A, 16, A + 4, None) == EALIGN
    assert L.w8a8_stream_probe(A, 0, None, None) == 0
