// Host-only check of the C ABI's argument validation, built together with csrc/api.cpp
// under AddressSanitizer and UndefinedBehaviorSanitizer (g++, no GPU). The launchers behind
// the ABI are replaced by stubs that record the call, so that the driver can check, for
// every entry point, that invalid arguments return the documented status before anything
// is enqueued and that valid ones reach the launcher with the caller's arguments.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "w8a8.h"
#include "../../fp4_w8a8_quantized_amd/csrc/internal.h"

namespace {
int g_calls = 0;
int64_t g_a = -1, g_b = -1, g_c = -1;
const void* g_p = nullptr;
hipError_t record(const void* p, int64_t a, int64_t b, int64_t c) {
  ++g_calls;
  g_p = p;
  g_a = a;
  g_b = b;
  g_c = c;
  return hipSuccess;
}
}  // namespace

namespace w8a8 {
hipError_t launch_quantize_rows(const void* x, int64_t R, int64_t K, int fmt, void*, float*, hipStream_t) { return record(x, R, K, fmt); }
hipError_t launch_quantize_static(const void* x, int64_t M, int64_t K, int fmt, const float*, void*, uint32_t*, float*, hipStream_t) { return record(x, M, K, fmt); }
hipError_t launch_delayed_scale(float* h, int64_t H, float*, int64_t step, int fmt, float*, hipStream_t) { return record(h, H, step, fmt); }
hipError_t launch_quantize_group(const void* x, int64_t M, int64_t K, void*, float*, hipStream_t) { return record(x, M, K, 0); }
hipError_t launch_quantize_block(const void* w, int64_t N, int64_t K, void*, float*, hipStream_t) { return record(w, N, K, 0); }
hipError_t launch_quantize_mxfp4(const void* x, int64_t R, int64_t K, void*, uint8_t*, hipStream_t) { return record(x, R, K, 0); }
hipError_t launch_gemm(const void* xq, const float*, const void*, const float*, int64_t M, int64_t N, int64_t K, int, void*, hipStream_t, const Epilogue& ep) { return record(xq, M, N, K + 1000000 * ep.act); }
hipError_t launch_linear_gemv(const void* x, const void*, const float*, int64_t N, int64_t K, int fmt, void*, float*, void*, hipStream_t) { return record(x, N, K, fmt); }
// the one-token kernel's shape rule, as the library states it
bool use_gemm_gemv(int64_t M, int64_t N, int64_t K) { return M == 1 && K % 1024 == 0 && K / 1024 >= 1 && K / 1024 <= 16 && N >= 1; }
hipError_t launch_gemm_blockscaled(const void* xq, const float*, const void*, const float*, int64_t M, int64_t N, int64_t K, void*, hipStream_t) { return record(xq, M, N, K); }
hipError_t launch_gemm_mxfp4(const void* xq, const uint8_t*, const void*, const uint8_t*, int64_t M, int64_t N, int64_t K, void*, hipStream_t) { return record(xq, M, N, K); }
hipError_t launch_quantize_nvfp4(const void* x, int64_t R, int64_t K, bool given, void*, uint8_t*, float*, hipStream_t) { return record(x, R, K, given); }
hipError_t launch_gemm_nvfp4(const void* xq, const uint8_t*, const float*, const void*, const uint8_t*, const float*, int64_t M, int64_t N, int64_t K, void*, hipStream_t) { return record(xq, M, N, K); }
hipError_t launch_quantize_int4(const void* w, int64_t N, int64_t K, void*, uint16_t*, hipStream_t) { return record(w, N, K, 0); }
hipError_t launch_gemm_w4a16(const void* x, const void*, const uint16_t*, int64_t M, int64_t N, int64_t K, void*, hipStream_t) { return record(x, M, N, K); }
hipError_t launch_channel_absmax(const void* x, int64_t R, int64_t K, float*, hipStream_t) { return record(x, R, K, 0); }
hipError_t launch_smooth_scales(const float* a, const float*, int64_t K, float, float*, hipStream_t) { return record(a, K, 0, 0); }
hipError_t launch_smooth_apply(const void* x, int64_t R, int64_t K, const float*, int mode, void*, hipStream_t) { return record(x, R, K, mode); }
hipError_t launch_sclk_probe(uint64_t* out, int blocks, int64_t ticks, hipStream_t) { return record(out, blocks, ticks, 0); }
hipError_t launch_stream_probe(const void* x, int64_t n, void*, hipStream_t) { return record(x, n, 0, 0); }
}  // namespace w8a8

namespace {
int g_fail = 0;
void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::printf("FAIL line %d: %s\n", line, what);
    ++g_fail;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// A call returned `want` and reached the launcher (once) exactly when want == W8A8_OK.
#define CHECK_CALL(call, want)                                      \
  do {                                                              \
    const int before = g_calls;                                     \
    const int st = (int)(call);                                     \
    EXPECT(st == (want));                                           \
    EXPECT((g_calls - before) == ((want) == W8A8_OK ? 1 : 0));      \
  } while (0)

// A call returned `want` and enqueued nothing (empty shapes).
#define CHECK_NO_LAUNCH(call, want)                                 \
  do {                                                              \
    const int before = g_calls;                                     \
    EXPECT((int)(call) == (want));                                  \
    EXPECT(g_calls == before);                                      \
  } while (0)
}  // namespace

int main() {
  alignas(16) static uint8_t buf[4096];
  void* A = buf;                       // 16-byte aligned, never dereferenced by the stubs
  void* U = buf + 4;                   // 4-byte but not 16-byte aligned
  float* F = reinterpret_cast<float*>(buf);
  const int64_t big = int64_t(1) << 40;

  // status strings cover every code and an unknown one
  for (int s = 0; s <= 7; ++s) EXPECT(w8a8_status_string(s) != nullptr && std::strlen(w8a8_status_string(s)) > 0);

  // per-token / per-channel quantization
  CHECK_CALL(w8a8_quantize_per_token(A, 4, 128, 0, A, F, nullptr), W8A8_OK);
  EXPECT(g_a == 4 && g_b == 128 && g_p == A);
  CHECK_CALL(w8a8_quantize_per_token(A, 4, 128, 2, A, F, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_quantize_per_token(A, -1, 128, 0, A, F, nullptr), W8A8_ERR_SHAPE);
  CHECK_CALL(w8a8_quantize_per_token(A, big, big, 0, A, F, nullptr), W8A8_ERR_SHAPE);
  CHECK_CALL(w8a8_quantize_per_token(A, 4, 120, 0, A, F, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_quantize_per_token(nullptr, 4, 128, 0, A, F, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_quantize_per_token(U, 4, 128, 0, A, F, nullptr), W8A8_ERR_ALIGN);
  CHECK_NO_LAUNCH(w8a8_quantize_per_token(nullptr, 0, 128, 0, nullptr, nullptr, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_quantize_weight_per_channel(A, 3, 16, 1, A, F, nullptr), W8A8_OK);

  // GEMM and the extended epilogue
  CHECK_CALL(w8a8_gemm(A, F, A, F, 5, 7, 256, 0, A, nullptr), W8A8_OK);
  EXPECT(g_a == 5 && g_b == 7 && g_c == 256);
  CHECK_CALL(w8a8_gemm(A, F, A, F, 5, 7, 200, 0, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm(A, F, A, F, 5, 7, 0, 0, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm(A, F, A, F, 5, 7, 256, 3, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm(A, F, A, F, 5, big, 256, 0, A, nullptr), W8A8_ERR_SHAPE);
  CHECK_CALL(w8a8_gemm(A, F, nullptr, F, 5, 7, 256, 0, A, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_gemm(A, F, A, F, 5, 7, 256, 0, U, nullptr), W8A8_ERR_ALIGN);
  CHECK_NO_LAUNCH(w8a8_gemm(A, F, A, F, 0, 7, 256, 0, nullptr, nullptr), W8A8_OK);
  CHECK_NO_LAUNCH(w8a8_stream_probe(nullptr, 0, nullptr, nullptr), W8A8_OK);
  // one linear layer: one fused launch for one token (K a multiple of 1024), else the
  // quantizer and the GEMM
  {
    const int before = g_calls;
    EXPECT(w8a8_linear(A, A, F, 1, 7, 4096, 0, A, F, A, nullptr) == W8A8_OK);
    EXPECT(g_calls - before == 1 && g_p == A && g_a == 7 && g_b == 4096 && g_c == 0);
    EXPECT(w8a8_linear(A, A, F, 5, 7, 256, 1, A, F, A, nullptr) == W8A8_OK);
    EXPECT(g_calls - before == 3 && g_a == 5 && g_b == 7 && g_c == 256);   // the GEMM came last
    EXPECT(w8a8_linear(A, A, F, 1, 7, 640, 0, A, F, A, nullptr) == W8A8_OK);
    EXPECT(g_calls - before == 5);
  }
  CHECK_CALL(w8a8_linear(A, A, F, 5, 7, 200, 0, A, F, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_linear(A, A, F, 5, 7, 256, 3, A, F, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_linear(nullptr, A, F, 5, 7, 256, 0, A, F, A, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_linear(A, A, F, 5, 7, 256, 0, nullptr, F, A, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_linear(U, A, F, 5, 7, 256, 0, A, F, A, nullptr), W8A8_ERR_ALIGN);
  CHECK_CALL(w8a8_linear(A, A, F, -1, 7, 256, 0, A, F, A, nullptr), W8A8_ERR_SHAPE);
  CHECK_CALL(w8a8_linear(A, A, F, big, 7, big, 0, A, F, A, nullptr), W8A8_ERR_SHAPE);
  CHECK_NO_LAUNCH(w8a8_linear(nullptr, nullptr, nullptr, 0, 7, 256, 0, nullptr, nullptr, nullptr, nullptr), W8A8_OK);
  CHECK_NO_LAUNCH(w8a8_linear(nullptr, nullptr, nullptr, 3, 0, 256, 0, nullptr, nullptr, nullptr, nullptr), W8A8_OK);

  CHECK_CALL(w8a8_gemm_ex(A, F, A, F, 5, 7, 256, 1, A, 2, 1, 0.5f, A, nullptr), W8A8_OK);
  EXPECT(g_c == 256 + 2000000);
  CHECK_CALL(w8a8_gemm_ex(A, F, A, F, 5, 7, 256, 0, nullptr, 3, 0, 1.f, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm_ex(A, F, A, F, 5, 7, 256, 0, nullptr, 0, 2, 1.f, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm_ex(A, F, A, F, 5, 7, 256, 0, nullptr, 0, 1, 0.f, A, nullptr), W8A8_ERR_ARG);
  CHECK_CALL(w8a8_gemm_ex(A, F, A, F, 5, 7, 256, 0, nullptr, 0, 1, -1.f, A, nullptr), W8A8_ERR_ARG);
  CHECK_CALL(w8a8_gemm_ex(A, F, A, F, 5, 7, 256, 0, U, 0, 0, 1.f, A, nullptr), W8A8_ERR_ALIGN);

  // static scales and delayed scaling
  CHECK_CALL(w8a8_quantize_static(A, 4, 16, 0, F, A, reinterpret_cast<uint32_t*>(buf + 4), F + 1, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_quantize_static(A, 4, 12, 0, F, A, nullptr, nullptr, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_quantize_static(A, 4, 16, 0, nullptr, A, nullptr, nullptr, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_quantize_static(A, 4, 16, 0, F, A, reinterpret_cast<uint32_t*>(buf + 2), nullptr, nullptr), W8A8_ERR_ALIGN);
  CHECK_CALL(w8a8_delayed_scale_update(F, 16, F, 3, 0, F, nullptr), W8A8_OK);
  EXPECT(g_a == 16 && g_b == 3);
  CHECK_CALL(w8a8_delayed_scale_update(F, 0, F, 3, 0, F, nullptr), W8A8_ERR_ARG);
  CHECK_CALL(w8a8_delayed_scale_update(F, 16, F, -1, 0, F, nullptr), W8A8_ERR_ARG);
  CHECK_CALL(w8a8_delayed_scale_update(F, 16, nullptr, 3, 0, F, nullptr), W8A8_ERR_NULL);

  // block-scaled FP8
  CHECK_CALL(w8a8_quantize_per_token_group(A, 4, 256, A, F, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_quantize_per_token_group(A, 4, 192, A, F, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_quantize_weight_block(A, 300, 256, A, F, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_quantize_weight_block(A, 300, 256, nullptr, F, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_gemm_blockscaled(A, F, A, F, 5, 7, 256, A, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_gemm_blockscaled(A, F, A, F, 5, 7, 100, A, nullptr), W8A8_ERR_UNSUPPORTED);

  // MXFP4 and NVFP4
  CHECK_CALL(w8a8_quantize_mxfp4(A, 4, 64, A, buf, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_quantize_mxfp4(A, 4, 48, A, buf, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm_mxfp4(A, buf, A, buf, 5, 7, 512, A, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_gemm_mxfp4(A, buf, A, buf, 5, 7, 128, A, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_quantize_nvfp4(A, 4, 32, 1, A, buf, F, nullptr), W8A8_OK);
  EXPECT(g_c == 1);
  CHECK_CALL(w8a8_quantize_nvfp4(A, 4, 32, 2, A, buf, F, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_quantize_nvfp4(A, 4, 32, 0, A, buf, nullptr, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_gemm_nvfp4(A, buf, F, A, buf, F, 5, 7, 128, A, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_gemm_nvfp4(A, buf, nullptr, A, buf, F, 5, 7, 128, A, nullptr), W8A8_ERR_NULL);
  CHECK_CALL(w8a8_gemm_nvfp4(A, buf, F, A, buf, F, 5, 7, 96, A, nullptr), W8A8_ERR_UNSUPPORTED);

  // W4A16
  CHECK_CALL(w8a8_quantize_int4(A, 4, 256, A, reinterpret_cast<uint16_t*>(buf), nullptr), W8A8_OK);
  CHECK_CALL(w8a8_quantize_int4(A, 4, 200, A, reinterpret_cast<uint16_t*>(buf), nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_gemm_w4a16(A, A, reinterpret_cast<uint16_t*>(buf), 5, 7, 256, A, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_gemm_w4a16(A, A, reinterpret_cast<uint16_t*>(buf), 5, big, 256, A, nullptr), W8A8_ERR_SHAPE);

  // SmoothQuant preparation
  CHECK_CALL(w8a8_channel_absmax(A, 4, 16, F, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_channel_absmax(A, 4, 12, F, nullptr), W8A8_ERR_UNSUPPORTED);
  CHECK_CALL(w8a8_smoothquant_scales(F, F, 16, 0.5f, F, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_smoothquant_scales(F, F, 16, 1.5f, F, nullptr), W8A8_ERR_ARG);
  CHECK_CALL(w8a8_smooth_apply(A, 4, 16, F, 1, A, nullptr), W8A8_OK);
  EXPECT(g_c == 1);
  CHECK_CALL(w8a8_smooth_apply(A, 4, 16, F, 2, A, nullptr), W8A8_ERR_ARG);

  // measurement helpers
  CHECK_CALL(w8a8_sclk_probe(reinterpret_cast<uint64_t*>(buf), 8, 1000, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_sclk_probe(reinterpret_cast<uint64_t*>(buf), 0, 1000, nullptr), W8A8_ERR_ARG);
  CHECK_CALL(w8a8_stream_probe(A, 64, A, nullptr), W8A8_OK);
  CHECK_CALL(w8a8_stream_probe(A, 60, A, nullptr), W8A8_ERR_UNSUPPORTED);

  std::printf("api checks: %d failures, %d launcher calls\n", g_fail, g_calls);
  return g_fail == 0 ? 0 : 1;
}
