// C ABI of the W8A8 library: host-side argument checks, then dispatch to the launchers.
// Every check runs before anything is enqueued; see include/w8a8.h for the contract.
#include "../../include/w8a8.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace {

// Upper bound on rows * row_bytes of any operand: the GEMM kernels address a matrix with
// 32-bit byte offsets.
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

w8a8_status hip_status(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// rows >= 0, K >= 0, rows * K * elem_bytes representable and under the operand cap.
w8a8_status check_dims(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0) return W8A8_ERR_SHAPE;
  if (K > 0 && rows > kMaxOperandBytes / (2 * K)) return W8A8_ERR_SHAPE;  // bf16 input
  return W8A8_OK;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int status) {
  switch (status) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_NULL: return "null pointer";
    case W8A8_ERR_SHAPE: return "bad shape";
    case W8A8_ERR_UNSUPPORTED: return "unsupported K granule or format";
    case W8A8_ERR_ALIGN: return "pointer not 16-byte aligned";
    case W8A8_ERR_HIP: return "HIP launch error";
    case W8A8_ERR_ARG: return "scalar argument out of range";
    default: return "unknown status";
  }
}

static w8a8_status quantize_rows_common(const void* x, int64_t R, int64_t K, int fmt, void* q,
                                        float* scale, void* stream) {
  if (fmt != W8A8_FMT_E4M3FN && fmt != W8A8_FMT_INT8) return W8A8_ERR_UNSUPPORTED;
  w8a8_status st = check_dims(R, K);
  if (st != W8A8_OK) return st;
  if (K % 16 != 0) return W8A8_ERR_UNSUPPORTED;
  if (R == 0) return W8A8_OK;
  if (!x || !q || !scale) return W8A8_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_rows(x, R, K, fmt, q, scale, as_stream(stream)));
}

w8a8_status w8a8_quantize_per_token(const void* x_bf16, int64_t M, int64_t K, int fmt, void* q,
                                    float* scale, void* stream) {
  return quantize_rows_common(x_bf16, M, K, fmt, q, scale, stream);
}

w8a8_status w8a8_quantize_weight_per_channel(const void* w_bf16, int64_t N, int64_t K, int fmt,
                                             void* q, float* scale, void* stream) {
  return quantize_rows_common(w_bf16, N, K, fmt, q, scale, stream);
}

static w8a8_status check_gemm(const void* xq, const void* sx, const void* wq, const void* sw,
                              int64_t M, int64_t N, int64_t K, int64_t k_granule,
                              int64_t row_bytes, const void* y) {
  if (M < 0 || N < 0 || K < 0) return W8A8_ERR_SHAPE;
  if (K == 0 || K % k_granule != 0) return W8A8_ERR_UNSUPPORTED;
  if (M > kMaxOperandBytes / row_bytes || N > kMaxOperandBytes / row_bytes) return W8A8_ERR_SHAPE;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return W8A8_ERR_SHAPE;
  if (((M + 255) / 256) * ((N + 127) / 128) > INT32_MAX) return W8A8_ERR_SHAPE;  // grid size
  if (M == 0 || N == 0) return W8A8_OK;
  if (!xq || !sx || !wq || !sw || !y) return W8A8_ERR_NULL;
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(sx) || !aligned16(sw) || !aligned16(y))
    return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

w8a8_status w8a8_gemm(const void* xq, const float* sx, const void* wq, const float* sw,
                      int64_t M, int64_t N, int64_t K, int fmt, void* y_bf16, void* stream) {
  if (fmt != W8A8_FMT_E4M3FN && fmt != W8A8_FMT_INT8) return W8A8_ERR_UNSUPPORTED;
  w8a8_status st = check_gemm(xq, sx, wq, sw, M, N, K, 128, K, y_bf16);
  if (st != W8A8_OK || M == 0 || N == 0) return st;
  return hip_status(w8a8::launch_gemm(xq, sx, wq, sw, M, N, K, fmt, y_bf16, as_stream(stream)));
}

w8a8_status w8a8_linear(const void* x_bf16, const void* wq, const float* sw, int64_t M, int64_t N,
                        int64_t K, int fmt, void* xq, float* sx, void* y_bf16, void* stream) {
  if (fmt != W8A8_FMT_E4M3FN && fmt != W8A8_FMT_INT8) return W8A8_ERR_UNSUPPORTED;
  w8a8_status st = check_dims(M, K);
  if (st != W8A8_OK) return st;
  st = check_gemm(xq, sx, wq, sw, M, N, K, 128, K, y_bf16);
  if (st != W8A8_OK || M == 0 || N == 0) return st;
  if (!x_bf16) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16)) return W8A8_ERR_ALIGN;
  if (w8a8::use_gemm_gemv(M, N, K))
    return hip_status(w8a8::launch_linear_gemv(x_bf16, wq, sw, N, K, fmt, xq, sx, y_bf16, as_stream(stream)));
  const hipError_t e = w8a8::launch_quantize_rows(x_bf16, M, K, fmt, xq, sx, as_stream(stream));
  if (e != hipSuccess) return W8A8_ERR_HIP;
  return hip_status(w8a8::launch_gemm(xq, sx, wq, sw, M, N, K, fmt, y_bf16, as_stream(stream)));
}

w8a8_status w8a8_gemm_ex(const void* xq, const float* sx, const void* wq, const float* sw,
                         int64_t M, int64_t N, int64_t K, int fmt, const void* bias_bf16,
                         int act, int out_fmt, float out_scale, void* y, void* stream) {
  if (fmt != W8A8_FMT_E4M3FN && fmt != W8A8_FMT_INT8) return W8A8_ERR_UNSUPPORTED;
  if (act != W8A8_ACT_NONE && act != W8A8_ACT_RELU && act != W8A8_ACT_SILU)
    return W8A8_ERR_UNSUPPORTED;
  if (out_fmt != W8A8_OUT_BF16 && out_fmt != W8A8_OUT_E4M3FN) return W8A8_ERR_UNSUPPORTED;
  if (out_fmt == W8A8_OUT_E4M3FN && !(out_scale > 0.f && out_scale <= 3.4028234663852886e38f))
    return W8A8_ERR_ARG;                                 // also rejects NaN and +inf
  w8a8_status st = check_gemm(xq, sx, wq, sw, M, N, K, 128, K, y);
  if (st != W8A8_OK || M == 0 || N == 0) return st;
  if (bias_bf16 && !aligned16(bias_bf16)) return W8A8_ERR_ALIGN;
  const w8a8::Epilogue ep{reinterpret_cast<const uint16_t*>(bias_bf16), act,
                          out_fmt == W8A8_OUT_E4M3FN ? 1 : 0, out_scale, 1.f / out_scale};
  return hip_status(w8a8::launch_gemm(xq, sx, wq, sw, M, N, K, fmt, y, as_stream(stream), ep));
}

w8a8_status w8a8_quantize_static(const void* x_bf16, int64_t M, int64_t K, int fmt,
                                 const float* scale, void* q, uint32_t* saturated,
                                 float* amax, void* stream) {
  if (fmt != W8A8_FMT_E4M3FN && fmt != W8A8_FMT_INT8) return W8A8_ERR_UNSUPPORTED;
  w8a8_status st = check_dims(M, K);
  if (st != W8A8_OK) return st;
  if (K % 8 != 0) return W8A8_ERR_UNSUPPORTED;
  if (M == 0 || K == 0) return W8A8_OK;
  if (!x_bf16 || !q || !scale) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q) || !aligned4(scale) || !aligned4(saturated) ||
      !aligned4(amax))
    return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_static(x_bf16, M, K, fmt, scale, q, saturated, amax,
                                                 as_stream(stream)));
}

w8a8_status w8a8_delayed_scale_update(float* amax_history, int64_t H, float* amax, int64_t step,
                                      int fmt, float* scale, void* stream) {
  if (fmt != W8A8_FMT_E4M3FN && fmt != W8A8_FMT_INT8) return W8A8_ERR_UNSUPPORTED;
  if (H < 1 || H > ((int64_t)1 << 24) || step < 0) return W8A8_ERR_ARG;
  if (!amax_history || !amax || !scale) return W8A8_ERR_NULL;
  if (!aligned4(amax_history) || !aligned4(amax) || !aligned4(scale)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_delayed_scale(amax_history, H, amax, step, fmt, scale,
                                               as_stream(stream)));
}

w8a8_status w8a8_quantize_per_token_group(const void* x_bf16, int64_t M, int64_t K, void* xq,
                                          float* sx, void* stream) {
  w8a8_status st = check_dims(M, K);
  if (st != W8A8_OK) return st;
  if (K == 0 || K % 128 != 0) return W8A8_ERR_UNSUPPORTED;
  if (M == 0) return W8A8_OK;
  if (!x_bf16 || !xq || !sx) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(xq) || !aligned16(sx)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_group(x_bf16, M, K, xq, sx, as_stream(stream)));
}

w8a8_status w8a8_quantize_weight_block(const void* w_bf16, int64_t N, int64_t K, void* wq,
                                       float* sw, void* stream) {
  w8a8_status st = check_dims(N, K);
  if (st != W8A8_OK) return st;
  if (K == 0 || K % 128 != 0) return W8A8_ERR_UNSUPPORTED;
  if (N == 0) return W8A8_OK;
  if ((N + 127) / 128 > 65535) return W8A8_ERR_SHAPE;
  if (!w_bf16 || !wq || !sw) return W8A8_ERR_NULL;
  if (!aligned16(w_bf16) || !aligned16(wq) || !aligned16(sw)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_block(w_bf16, N, K, wq, sw, as_stream(stream)));
}

w8a8_status w8a8_gemm_blockscaled(const void* xq, const float* sx, const void* wq,
                                  const float* sw, int64_t M, int64_t N, int64_t K,
                                  void* y_bf16, void* stream) {
  w8a8_status st = check_gemm(xq, sx, wq, sw, M, N, K, 128, K, y_bf16);
  if (st != W8A8_OK || M == 0 || N == 0) return st;
  return hip_status(w8a8::launch_gemm_blockscaled(xq, sx, wq, sw, M, N, K, y_bf16,
                                                  as_stream(stream)));
}

w8a8_status w8a8_quantize_mxfp4(const void* x_bf16, int64_t R, int64_t K, void* q_packed,
                                uint8_t* scale_e8m0, void* stream) {
  w8a8_status st = check_dims(R, K);
  if (st != W8A8_OK) return st;
  if (K % 32 != 0) return W8A8_ERR_UNSUPPORTED;
  if (R == 0 || K == 0) return W8A8_OK;
  if (!x_bf16 || !q_packed || !scale_e8m0) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q_packed) || !aligned16(scale_e8m0)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_mxfp4(x_bf16, R, K, q_packed, scale_e8m0,
                                                as_stream(stream)));
}

w8a8_status w8a8_gemm_mxfp4(const void* xq, const uint8_t* sx, const void* wq, const uint8_t* sw,
                            int64_t M, int64_t N, int64_t K, void* y_bf16, void* stream) {
  w8a8_status st = check_gemm(xq, sx, wq, sw, M, N, K, 256, K / 2, y_bf16);
  if (st != W8A8_OK || M == 0 || N == 0) return st;
  return hip_status(w8a8::launch_gemm_mxfp4(xq, sx, wq, sw, M, N, K, y_bf16, as_stream(stream)));
}

w8a8_status w8a8_quantize_nvfp4(const void* x_bf16, int64_t R, int64_t K, int scale_mode,
                                void* q_packed, uint8_t* scale_e4m3, float* g, void* stream) {
  if (scale_mode != W8A8_NVFP4_SCALE_COMPUTE && scale_mode != W8A8_NVFP4_SCALE_GIVEN)
    return W8A8_ERR_UNSUPPORTED;
  w8a8_status st = check_dims(R, K);
  if (st != W8A8_OK) return st;
  if (K % 16 != 0) return W8A8_ERR_UNSUPPORTED;
  if (R == 0 || K == 0) return W8A8_OK;
  if (!x_bf16 || !q_packed || !scale_e4m3 || !g) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q_packed) || !aligned16(scale_e4m3) || !aligned4(g))
    return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_nvfp4(x_bf16, R, K, scale_mode == W8A8_NVFP4_SCALE_GIVEN,
                                                q_packed, scale_e4m3, g, as_stream(stream)));
}

w8a8_status w8a8_gemm_nvfp4(const void* xq, const uint8_t* sx, const float* gx, const void* wq,
                            const uint8_t* sw, const float* gw, int64_t M, int64_t N, int64_t K,
                            void* y_bf16, void* stream) {
  w8a8_status st = check_gemm(xq, sx, wq, sw, M, N, K, 64, K / 2, y_bf16);
  if (st != W8A8_OK || M == 0 || N == 0) return st;
  if (!gx || !gw) return W8A8_ERR_NULL;
  if (!aligned4(gx) || !aligned4(gw)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_gemm_nvfp4(xq, sx, gx, wq, sw, gw, M, N, K, y_bf16,
                                            as_stream(stream)));
}

w8a8_status w8a8_quantize_int4(const void* w_bf16, int64_t N, int64_t K, void* q_packed,
                               uint16_t* scale_f16, void* stream) {
  w8a8_status st = check_dims(N, K);
  if (st != W8A8_OK) return st;
  if (K % 128 != 0) return W8A8_ERR_UNSUPPORTED;
  if (N == 0 || K == 0) return W8A8_OK;
  if (!w_bf16 || !q_packed || !scale_f16) return W8A8_ERR_NULL;
  if (!aligned16(w_bf16) || !aligned16(q_packed) || !aligned16(scale_f16)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_quantize_int4(w_bf16, N, K, q_packed, scale_f16, as_stream(stream)));
}

w8a8_status w8a8_gemm_w4a16(const void* x_bf16, const void* q_packed, const uint16_t* scale_f16,
                            int64_t M, int64_t N, int64_t K, void* y_bf16, void* stream) {
  if (M < 0 || N < 0 || K < 0) return W8A8_ERR_SHAPE;
  if (K == 0 || K % 128 != 0) return W8A8_ERR_UNSUPPORTED;
  if (M > kMaxOperandBytes / (2 * K) || N > kMaxOperandBytes / (K / 2)) return W8A8_ERR_SHAPE;
  if (M > INT32_MAX / 2 || N > INT32_MAX / 2) return W8A8_ERR_SHAPE;
  if (M == 0 || N == 0) return W8A8_OK;
  if (!x_bf16 || !q_packed || !scale_f16 || !y_bf16) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(q_packed) || !aligned16(scale_f16) || !aligned16(y_bf16))
    return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_gemm_w4a16(x_bf16, q_packed, scale_f16, M, N, K, y_bf16,
                                            as_stream(stream)));
}

w8a8_status w8a8_channel_absmax(const void* x_bf16, int64_t R, int64_t K, float* amax,
                                void* stream) {
  w8a8_status st = check_dims(R, K);
  if (st != W8A8_OK) return st;
  if (K % 8 != 0) return W8A8_ERR_UNSUPPORTED;
  if (K == 0) return W8A8_OK;
  if ((R + 63) / 64 > 65535) return W8A8_ERR_SHAPE;
  if (!amax || (R > 0 && !x_bf16)) return W8A8_ERR_NULL;
  if (!aligned16(amax) || (R > 0 && !aligned16(x_bf16))) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_channel_absmax(x_bf16, R, K, amax, as_stream(stream)));
}

w8a8_status w8a8_smoothquant_scales(const float* act_max, const float* w_max, int64_t K,
                                    float alpha, float* s, void* stream) {
  if (K < 0) return W8A8_ERR_SHAPE;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return W8A8_ERR_ARG;
  if (K == 0) return W8A8_OK;
  if (!act_max || !w_max || !s) return W8A8_ERR_NULL;
  if (!aligned16(act_max) || !aligned16(w_max) || !aligned16(s)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_smooth_scales(act_max, w_max, K, alpha, s, as_stream(stream)));
}

w8a8_status w8a8_smooth_apply(const void* x_bf16, int64_t R, int64_t K, const float* s, int mode,
                              void* out_bf16, void* stream) {
  if (mode != 0 && mode != 1) return W8A8_ERR_ARG;
  w8a8_status st = check_dims(R, K);
  if (st != W8A8_OK) return st;
  if (K % 8 != 0) return W8A8_ERR_UNSUPPORTED;
  if (R == 0 || K == 0) return W8A8_OK;
  if (!x_bf16 || !s || !out_bf16) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(s) || !aligned16(out_bf16)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_smooth_apply(x_bf16, R, K, s, mode, out_bf16, as_stream(stream)));
}

w8a8_status w8a8_sclk_probe(uint64_t* out, int blocks, int64_t ticks, void* stream) {
  if (blocks < 1 || blocks > 1024 || ticks < 1 || ticks > ((int64_t)1 << 32)) return W8A8_ERR_ARG;
  if (!out) return W8A8_ERR_NULL;
  if (!aligned16(out)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_sclk_probe(out, blocks, ticks, as_stream(stream)));
}

w8a8_status w8a8_stream_probe(const void* x_bf16, int64_t n, void* y, void* stream) {
  if (n < 0 || n > kMaxOperandBytes / 2) return W8A8_ERR_SHAPE;
  if (n % 8 != 0) return W8A8_ERR_UNSUPPORTED;
  if (n == 0) return W8A8_OK;
  if (!x_bf16 || !y) return W8A8_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(y)) return W8A8_ERR_ALIGN;
  return hip_status(w8a8::launch_stream_probe(x_bf16, n, y, as_stream(stream)));
}

}  // extern "C"
