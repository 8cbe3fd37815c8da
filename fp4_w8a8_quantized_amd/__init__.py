"""MI355X (gfx950) W8A8 quantized GEMM: Python binding of the libw8a8.so C ABI.

Marshalling only: tensors are checked for device, dtype, shape and contiguity, outputs
are allocated with torch on the input's device, and their pointers plus the current HIP
stream are handed to the C ABI (declared in include/w8a8.h). Every arithmetic step runs in
the library's HIP kernels; there is no fallback path. If the library is not built, or no
GPU is visible, calls raise.

Formats: FP8 codes are returned as ``torch.float8_e4m3fn`` tensors (OCP E4M3FN bytes),
INT8 codes as ``torch.int8``, MXFP4 codes as ``torch.uint8`` (two E2M1 codes per byte,
element 2i in the low nibble) with E8M0 scales as ``torch.uint8``.
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "library_path", "status_string", "W8A8Error",
    "quantize_per_token", "quantize_weight_per_channel", "gemm", "gemm_ex", "linear",
    "quantize_static", "delayed_scale_update",
    "quantize_per_token_group", "quantize_weight_block", "gemm_blockscaled",
    "quantize_mxfp4", "gemm_mxfp4",
    "channel_absmax", "smoothquant_scales", "smooth_apply",
    "FMT_E4M3FN", "FMT_INT8", "ACTIVATIONS",
]

FMT_E4M3FN = 0
FMT_INT8 = 1

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG_DIR, "libw8a8.so")

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p
_c_float = ctypes.c_float

# name -> argument types, in the order of include/w8a8.h
_SIGNATURES = {
    "w8a8_quantize_per_token": [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp],
    "w8a8_quantize_weight_per_channel": [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp],
    "w8a8_gemm": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp],
    "w8a8_linear": [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_vp],
    "w8a8_gemm_ex": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_int, _c_vp, _c_int,
                     _c_int, _c_float, _c_vp, _c_vp],
    "w8a8_quantize_static": [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp],
    "w8a8_delayed_scale_update": [_c_vp, _c_i64, _c_vp, _c_i64, _c_int, _c_vp, _c_vp],
    "w8a8_quantize_per_token_group": [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
    "w8a8_quantize_weight_block": [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
    "w8a8_gemm_blockscaled": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp],
    "w8a8_quantize_mxfp4": [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
    "w8a8_gemm_mxfp4": [_c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp],
    "w8a8_quantize_int4": [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp],
    "w8a8_gemm_w4a16": [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp],
    "w8a8_quantize_nvfp4": [_c_vp, _c_i64, _c_i64, _c_int, _c_vp, _c_vp, _c_vp, _c_vp],
    "w8a8_gemm_nvfp4": [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp],
    "w8a8_channel_absmax": [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp],
    "w8a8_smoothquant_scales": [_c_vp, _c_vp, _c_i64, _c_float, _c_vp, _c_vp],
    "w8a8_smooth_apply": [_c_vp, _c_i64, _c_i64, _c_vp, _c_int, _c_vp, _c_vp],
    "w8a8_sclk_probe": [_c_vp, _c_int, _c_i64, _c_vp],
    "w8a8_stream_probe": [_c_vp, _c_i64, _c_vp, _c_vp],
}

_lib = None


class W8A8Error(RuntimeError):
    """A non-zero status returned by the C ABI."""


def lib() -> ctypes.CDLL:
    """The loaded libw8a8.so (loaded on first use; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is not built: run `python -m fp4_w8a8_quantized_amd.build`")
        cdll = ctypes.CDLL(library_path)
        for name, argtypes in _SIGNATURES.items():
            fn = getattr(cdll, name)
            fn.argtypes = argtypes
            fn.restype = _c_int
        cdll.w8a8_status_string.argtypes = [_c_int]
        cdll.w8a8_status_string.restype = ctypes.c_char_p
        _lib = cdll
    return _lib


def status_string(status: int) -> str:
    return lib().w8a8_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise W8A8Error(f"{what}: {status_string(status)} (status {status})")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype, ndim: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _fmt(fmt) -> int:
    if fmt in ("e4m3fn", "fp8", FMT_E4M3FN):
        return FMT_E4M3FN
    if fmt in ("int8", FMT_INT8):
        return FMT_INT8
    raise ValueError(f"unknown format {fmt!r}")


_CODE_DTYPE = {FMT_E4M3FN: torch.float8_e4m3fn, FMT_INT8: torch.int8}


# ------------------------------------------------------------------------------ per row
def _quantize_rows(fn_name: str, x: torch.Tensor, fmt):
    f = _fmt(fmt)
    _dev(x, "x", torch.bfloat16, 2)
    R, K = x.shape
    q = torch.empty((R, K), dtype=_CODE_DTYPE[f], device=x.device)
    s = torch.empty((R,), dtype=torch.float32, device=x.device)
    _check(getattr(lib(), fn_name)(x.data_ptr(), R, K, f, q.data_ptr(), s.data_ptr(), _stream(x)), fn_name)
    return q, s


def quantize_per_token(x: torch.Tensor, fmt="e4m3fn"):
    """X bf16 [M, K] -> (codes [M, K], fp32 scales [M]); one dynamic scale per token."""
    return _quantize_rows("w8a8_quantize_per_token", x, fmt)


def quantize_weight_per_channel(w: torch.Tensor, fmt="e4m3fn"):
    """W bf16 [N, K] -> (codes [N, K], fp32 scales [N]); one scale per output channel."""
    return _quantize_rows("w8a8_quantize_weight_per_channel", w, fmt)


def gemm(xq: torch.Tensor, sx: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """y bf16 [M, N] = diag(sx) (xq wq^T) diag(sw); FP8 or INT8 chosen by the code dtype."""
    _dev(xq, "xq", (torch.float8_e4m3fn, torch.int8), 2)
    f = FMT_INT8 if xq.dtype == torch.int8 else FMT_E4M3FN
    _dev(wq, "wq", xq.dtype, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq disagree on K")
    _dev(sx, "sx", torch.float32, 1)
    _dev(sw, "sw", torch.float32, 1)
    if sx.shape[0] != M or sw.shape[0] != N:
        raise ValueError("scale lengths must be M and N")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _dev(y, "out", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check(lib().w8a8_gemm(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(), M, N, K, f,
                           y.data_ptr(), _stream(xq)), "w8a8_gemm")
    return y


ACTIVATIONS = {"none": 0, "relu": 1, "silu": 2}


def gemm_ex(xq: torch.Tensor, sx: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor,
            bias: torch.Tensor | None = None, act: str = "none", out_scale: float | None = None,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """The scaled GEMM with the full epilogue: + bias (bf16 [N]), activation ("none",
    "relu", "silu"), then bf16 [M, N], or, when out_scale is given, E4M3FN codes of
    clamp(v / out_scale, +-448) as float8_e4m3fn [M, N]."""
    _dev(xq, "xq", (torch.float8_e4m3fn, torch.int8), 2)
    f = FMT_INT8 if xq.dtype == torch.int8 else FMT_E4M3FN
    _dev(wq, "wq", xq.dtype, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq disagree on K")
    _dev(sx, "sx", torch.float32, 1)
    _dev(sw, "sw", torch.float32, 1)
    if sx.shape[0] != M or sw.shape[0] != N:
        raise ValueError("scale lengths must be M and N")
    if act not in ACTIVATIONS:
        raise ValueError(f"unknown activation {act!r}")
    bptr = None
    if bias is not None:
        _dev(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias length must be N")
        bptr = bias.data_ptr()
    fp8_out = out_scale is not None
    ydt = torch.float8_e4m3fn if fp8_out else torch.bfloat16
    y = out if out is not None else torch.empty((M, N), dtype=ydt, device=xq.device)
    _dev(y, "out", ydt, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check(lib().w8a8_gemm_ex(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(), M, N, K, f,
                              bptr, ACTIVATIONS[act], 1 if fp8_out else 0,
                              float(out_scale) if fp8_out else 1.0, y.data_ptr(), _stream(xq)),
           "w8a8_gemm_ex")
    return y


def linear(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor, out=None, xq_out=None, sx_out=None,
           return_codes: bool = False):
    """W8A8 linear layer (w8a8_linear): quantize x per token in the format of wq, then the
    scaled GEMM. Returns y, or (y, xq, sx) with return_codes."""
    fmt = FMT_INT8 if wq.dtype == torch.int8 else FMT_E4M3FN
    x = _dev(x, "x", torch.bfloat16, 2)
    wq = _dev(wq, "wq", wq.dtype, 2)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("x and wq disagree on K")
    qdt = torch.int8 if fmt == FMT_INT8 else torch.float8_e4m3fn
    xq = xq_out if xq_out is not None else torch.empty((M, K), dtype=qdt, device=x.device)
    sx = sx_out if sx_out is not None else torch.empty((M,), dtype=torch.float32, device=x.device)
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _dev(xq, "xq_out", qdt, 2)
    _dev(sx, "sx_out", torch.float32, 1)
    _dev(y, "out", torch.bfloat16, 2)
    if tuple(xq.shape) != (M, K) or tuple(sx.shape) != (M,) or tuple(y.shape) != (M, N):
        raise ValueError("xq_out must be [M, K], sx_out [M], out [M, N]")
    _check(lib().w8a8_linear(x.data_ptr(), wq.data_ptr(), _dev(sw, "sw", torch.float32, 1).data_ptr(),
                             M, N, K, fmt, xq.data_ptr(), sx.data_ptr(), y.data_ptr(), _stream(x)),
           "w8a8_linear")
    return (y, xq, sx) if return_codes else y


# ------------------------------------------------------------------------------ static scales
def quantize_static(x: torch.Tensor, scale: torch.Tensor, fmt="e4m3fn",
                    saturated: torch.Tensor | None = None, amax: torch.Tensor | None = None):
    """X bf16 [M, K] with one static scale (fp32 tensor of one element, on the GPU) ->
    codes [M, K]. `saturated` (int32/uint32, one element) accumulates the number of
    clipped elements; `amax` (fp32, one element, >= 0) the running max |x|."""
    f = _fmt(fmt)
    _dev(x, "x", torch.bfloat16, 2)
    for t, n, dt in ((scale, "scale", torch.float32), (saturated, "saturated", (torch.int32, torch.uint32)),
                     (amax, "amax", torch.float32)):
        if t is not None:
            _dev(t, n, dt, t.dim())
            if t.numel() < 1:
                raise ValueError(f"{n} must hold one element")
    M, K = x.shape
    q = torch.empty((M, K), dtype=_CODE_DTYPE[f], device=x.device)
    _check(lib().w8a8_quantize_static(x.data_ptr(), M, K, f, scale.data_ptr(), q.data_ptr(),
                                      saturated.data_ptr() if saturated is not None else None,
                                      amax.data_ptr() if amax is not None else None, _stream(x)),
           "w8a8_quantize_static")
    return q


def delayed_scale_update(history: torch.Tensor, amax: torch.Tensor, step: int, scale: torch.Tensor,
                         fmt="e4m3fn") -> None:
    """history[step % H] = amax; amax = 0; scale = max(max(history), 1e-8) / qmax (on the GPU)."""
    f = _fmt(fmt)
    _dev(history, "history", torch.float32, 1)
    _dev(amax, "amax", torch.float32, amax.dim())
    _dev(scale, "scale", torch.float32, scale.dim())
    _check(lib().w8a8_delayed_scale_update(history.data_ptr(), history.numel(), amax.data_ptr(), int(step),
                                           f, scale.data_ptr(), _stream(history)),
           "w8a8_delayed_scale_update")


# ------------------------------------------------------------------------------ block-scaled
def quantize_per_token_group(x: torch.Tensor):
    """X bf16 [M, K] -> (E4M3FN codes [M, K], fp32 scales [M, K/128]) with 1x128 groups."""
    _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=x.device)
    s = torch.empty((M, max(K // 128, 0)), dtype=torch.float32, device=x.device)
    _check(lib().w8a8_quantize_per_token_group(x.data_ptr(), M, K, q.data_ptr(), s.data_ptr(),
                                               _stream(x)), "w8a8_quantize_per_token_group")
    return q, s


def quantize_weight_block(w: torch.Tensor):
    """W bf16 [N, K] -> (E4M3FN codes [N, K], fp32 scales [ceil(N/128), K/128])."""
    _dev(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.float8_e4m3fn, device=w.device)
    s = torch.empty(((N + 127) // 128, max(K // 128, 0)), dtype=torch.float32, device=w.device)
    _check(lib().w8a8_quantize_weight_block(w.data_ptr(), N, K, q.data_ptr(), s.data_ptr(),
                                            _stream(w)), "w8a8_quantize_weight_block")
    return q, s


def gemm_blockscaled(xq, sx, wq, sw, out=None) -> torch.Tensor:
    """y bf16 [M, N] = sum_g sx[:, g] sw[n/128, g] (xq_g wq_g^T), fp32 promotion per group."""
    _dev(xq, "xq", torch.float8_e4m3fn, 2)
    _dev(wq, "wq", torch.float8_e4m3fn, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq disagree on K")
    _dev(sx, "sx", torch.float32, 2)
    _dev(sw, "sw", torch.float32, 2)
    if tuple(sx.shape) != (M, K // 128) or tuple(sw.shape) != ((N + 127) // 128, K // 128):
        raise ValueError("scale shapes must be [M, K/128] and [ceil(N/128), K/128]")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _dev(y, "out", torch.bfloat16, 2)
    _check(lib().w8a8_gemm_blockscaled(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                                       M, N, K, y.data_ptr(), _stream(xq)), "w8a8_gemm_blockscaled")
    return y


# ------------------------------------------------------------------------------ MXFP4
def quantize_mxfp4(x: torch.Tensor):
    """bf16 [R, K] -> (packed E2M1 uint8 [R, K/2], E8M0 uint8 [R, K/32])."""
    _dev(x, "x", torch.bfloat16, 2)
    R, K = x.shape
    q = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((R, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().w8a8_quantize_mxfp4(x.data_ptr(), R, K, q.data_ptr(), s.data_ptr(), _stream(x)),
           "w8a8_quantize_mxfp4")
    return q, s


def gemm_mxfp4(xq, sx, wq, sw, out=None) -> torch.Tensor:
    """y bf16 [M, N] from MXFP4 operands (packed codes + E8M0 scales per 32 along K)."""
    for t, n in ((xq, "xq"), (wq, "wq"), (sx, "sx"), (sw, "sw")):
        _dev(t, n, torch.uint8, 2)
    M, Kh = xq.shape
    N = wq.shape[0]
    K = 2 * Kh
    if wq.shape[1] != Kh or tuple(sx.shape) != (M, K // 32) or tuple(sw.shape) != (N, K // 32):
        raise ValueError("MXFP4 operand shapes disagree")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _dev(y, "out", torch.bfloat16, 2)
    _check(lib().w8a8_gemm_mxfp4(xq.data_ptr(), sx.data_ptr(), wq.data_ptr(), sw.data_ptr(),
                                 M, N, K, y.data_ptr(), _stream(xq)), "w8a8_gemm_mxfp4")
    return y


# ------------------------------------------------------------------------------ NVFP4
NVFP4_SCALE_COMPUTE, NVFP4_SCALE_GIVEN = 0, 1


def quantize_nvfp4(x: torch.Tensor, g: torch.Tensor | None = None):
    """bf16 [R, K] -> (packed E2M1 uint8 [R, K/2], E4M3 scale codes uint8 [R, K/16],
    tensor scale g fp32 [1]). With g None, g = amax / 2688 is computed from x; otherwise
    the given fp32 [1] device tensor is used (and returned)."""
    _dev(x, "x", torch.bfloat16, 2)
    R, K = x.shape
    q = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((R, K // 16), dtype=torch.uint8, device=x.device)
    if g is None:
        g_out, mode = torch.empty((1,), dtype=torch.float32, device=x.device), NVFP4_SCALE_COMPUTE
    else:
        _dev(g, "g", torch.float32, 1)
        g_out, mode = g, NVFP4_SCALE_GIVEN
    _check(lib().w8a8_quantize_nvfp4(x.data_ptr(), R, K, mode, q.data_ptr(), s.data_ptr(),
                                     g_out.data_ptr(), _stream(x)), "w8a8_quantize_nvfp4")
    return q, s, g_out


def gemm_nvfp4(xq, sx, gx, wq, sw, gw, out=None) -> torch.Tensor:
    """y bf16 [M, N] from NVFP4 operands (packed codes, E4M3 scales per 16, fp32 g each)."""
    for t, n in ((xq, "xq"), (wq, "wq"), (sx, "sx"), (sw, "sw")):
        _dev(t, n, torch.uint8, 2)
    _dev(gx, "gx", torch.float32, 1)
    _dev(gw, "gw", torch.float32, 1)
    M, Kh = xq.shape
    N = wq.shape[0]
    K = 2 * Kh
    if wq.shape[1] != Kh or tuple(sx.shape) != (M, K // 16) or tuple(sw.shape) != (N, K // 16):
        raise ValueError("NVFP4 operand shapes disagree")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _dev(y, "out", torch.bfloat16, 2)
    _check(lib().w8a8_gemm_nvfp4(xq.data_ptr(), sx.data_ptr(), gx.data_ptr(), wq.data_ptr(),
                                 sw.data_ptr(), gw.data_ptr(), M, N, K, y.data_ptr(), _stream(xq)),
           "w8a8_gemm_nvfp4")
    return y


# ------------------------------------------------------------------------------ W4A16
def quantize_int4(w: torch.Tensor):
    """bf16 [N, K] -> (packed INT4 uint8 [N, K/2], fp16 group scales [N, K/128])."""
    _dev(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
    s = torch.empty((N, K // 128), dtype=torch.float16, device=w.device)
    _check(lib().w8a8_quantize_int4(w.data_ptr(), N, K, q.data_ptr(), s.data_ptr(), _stream(w)),
           "w8a8_quantize_int4")
    return q, s


def gemm_w4a16(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, out=None) -> torch.Tensor:
    """y bf16 [M, N] = x (bf16 [M, K]) times the INT4 weights (packed [N, K/2], fp16 [N, K/128])."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(q, "q", torch.uint8, 2)
    _dev(s, "s", torch.float16, 2)
    M, K = x.shape
    N = q.shape[0]
    if q.shape[1] * 2 != K or tuple(s.shape) != (N, K // 128):
        raise ValueError("W4A16 operand shapes disagree")
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _dev(y, "out", torch.bfloat16, 2)
    _check(lib().w8a8_gemm_w4a16(x.data_ptr(), q.data_ptr(), s.data_ptr(), M, N, K, y.data_ptr(),
                                 _stream(x)), "w8a8_gemm_w4a16")
    return y


# ------------------------------------------------------------------------------ SmoothQuant
def channel_absmax(x: torch.Tensor) -> torch.Tensor:
    """max over rows of |x[:, j]| for a bf16 [R, K] matrix -> fp32 [K]."""
    _dev(x, "x", torch.bfloat16, 2)
    R, K = x.shape
    a = torch.empty((K,), dtype=torch.float32, device=x.device)
    _check(lib().w8a8_channel_absmax(x.data_ptr(), R, K, a.data_ptr(), _stream(x)),
           "w8a8_channel_absmax")
    return a


def smoothquant_scales(act_max: torch.Tensor, w_max: torch.Tensor, alpha: float = 0.5) -> torch.Tensor:
    """s_j = max(a_j, 1e-5)^alpha / max(w_j, 1e-5)^(1 - alpha) -> fp32 [K]."""
    _dev(act_max, "act_max", torch.float32, 1)
    _dev(w_max, "w_max", torch.float32, 1)
    K = act_max.shape[0]
    if w_max.shape[0] != K:
        raise ValueError("act_max and w_max lengths differ")
    s = torch.empty((K,), dtype=torch.float32, device=act_max.device)
    _check(lib().w8a8_smoothquant_scales(act_max.data_ptr(), w_max.data_ptr(), K, float(alpha),
                                         s.data_ptr(), _stream(act_max)), "w8a8_smoothquant_scales")
    return s


def smooth_apply(x: torch.Tensor, s: torch.Tensor, mode: str) -> torch.Tensor:
    """Column-wise smoothing of bf16 [R, K]: mode 'activation' divides by s, 'weight' multiplies."""
    m = {"activation": 0, "weight": 1}[mode]
    _dev(x, "x", torch.bfloat16, 2)
    _dev(s, "s", torch.float32, 1)
    R, K = x.shape
    if s.shape[0] != K:
        raise ValueError("s must have K entries")
    out = torch.empty_like(x)
    _check(lib().w8a8_smooth_apply(x.data_ptr(), R, K, s.data_ptr(), m, out.data_ptr(), _stream(x)),
           "w8a8_smooth_apply")
    return out
