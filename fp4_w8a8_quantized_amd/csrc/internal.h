// Launchers behind the C ABI. Arguments have been validated by api.cpp; each launcher
// only enqueues kernels on `st` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

hipError_t launch_quantize_rows(const void* x, int64_t R, int64_t K, int fmt, void* q,
                                float* scale, hipStream_t st);
hipError_t launch_quantize_static(const void* x, int64_t M, int64_t K, int fmt, const float* scale,
                                  void* q, uint32_t* saturated, float* amax, hipStream_t st);
hipError_t launch_delayed_scale(float* history, int64_t H, float* amax, int64_t step, int fmt,
                                float* scale, hipStream_t st);
hipError_t launch_quantize_group(const void* x, int64_t M, int64_t K, void* q, float* sx,
                                 hipStream_t st);
hipError_t launch_quantize_block(const void* w, int64_t N, int64_t K, void* q, float* sw,
                                 hipStream_t st);
hipError_t launch_quantize_mxfp4(const void* x, int64_t R, int64_t K, void* q, uint8_t* sc,
                                 hipStream_t st);

// What the GEMM epilogue does after dequantization: add a bf16 bias (when non-null), apply
// an activation (0 none, 1 ReLU, 2 SiLU), and store bf16 or, when out_fp8, E4M3FN codes
// of clamp(v / s_out, +-448). The default is the plain bf16 epilogue.
struct Epilogue {
  const uint16_t* bias = nullptr;
  int act = 0;
  int out_fp8 = 0;
  float s_out = 1.f;
  float inv_s_out = 1.f;            // fp32(1 / s_out)
};

hipError_t launch_gemm(const void* xq, const float* sx, const void* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                       const Epilogue& ep = Epilogue{});
// launch_gemm for more tokens than the narrow tiles take (fmt 0 FP8, 1 INT8): 8 waves per
// workgroup, two per SIMD alternating between LDS reads and MFMAs.
hipError_t launch_gemm_pp(const void* xq, const float* sx, const void* wq, const float* sw,
                          int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                          const Epilogue& ep);

// 256 x 128 tiles on one wave per SIMD (128 x 64 wave tiles, fragments double-buffered,
// one barrier per K step), fmt 0 FP8 or 1 INT8.
hipError_t launch_gemm_solo(const void* xq, const float* sx, const void* wq, const float* sw,
                            int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                            const Epilogue& ep);

// One token where the vector kernel does not take K: weights streamed by 16-row workgroups
// that split K among their waves.
hipError_t launch_gemm_skinny(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                              const Epilogue& ep);
// Block-scaled FP8 on the two-waves-per-SIMD kernel (256 x 128 tiles, one weight block
// wide; each 128-K group's partial promoted with its scales).
hipError_t launch_gemm_blockscaled(const void* xq, const float* sx, const void* wq,
                                   const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                   hipStream_t st);
hipError_t launch_quantize_nvfp4(const void* x, int64_t R, int64_t K, bool given, void* q,
                                 uint8_t* sc, float* g, hipStream_t st);
hipError_t launch_gemm_nvfp4(const void* xq, const uint8_t* xs, const float* gx, const void* wq,
                             const uint8_t* ws, const float* gw, int64_t M, int64_t N, int64_t K,
                             void* y, hipStream_t st);
hipError_t launch_quantize_int4(const void* w, int64_t N, int64_t K, void* q, uint16_t* sc,
                                hipStream_t st);
hipError_t launch_gemm_w4a16(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                             int64_t K, void* y, hipStream_t st);
// W4A16 above 32 tokens (16 above 8192 outputs) with K a multiple of 1024: 32-128 token rows
// and 16-64 weight rows per workgroup, both staged in LDS one group per K step.
bool use_w4a16_mid(int64_t M, int64_t N, int64_t K);
bool use_w4a16_gemv(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_w4a16_mid(const void* x, const void* wq, const uint16_t* sc, int64_t M,
                                 int64_t N, int64_t K, void* y, hipStream_t st);
// MXFP4 on 256 x 256 tiles, one wave per SIMD (128 x 128 wave tiles, accumulators in AGPRs).
hipError_t launch_gemm_mx_solo(const void* xq, const uint8_t* sx, const void* wq, const uint8_t* sw,
                               int64_t M, int64_t N, int64_t K, void* y, hipStream_t st);
hipError_t launch_gemm_mxfp4(const void* xq, const uint8_t* sx, const void* wq,
                             const uint8_t* sw, int64_t M, int64_t N, int64_t K, void* y,
                             hipStream_t st);

hipError_t launch_channel_absmax(const void* x, int64_t R, int64_t K, float* amax,
                                 hipStream_t st);
hipError_t launch_smooth_scales(const float* a, const float* w, int64_t K, float alpha,
                                float* s, hipStream_t st);
hipError_t launch_smooth_apply(const void* x, int64_t R, int64_t K, const float* s, int mode,
                               void* out, hipStream_t st);

// Narrow output tiles sized to the token count (16-128 token rows x 16-128 weight rows, 4 or
// 8 waves, K through an LDS ring of row-contiguous stages): 2-128 tokens, and more tokens
// where one round of 64 x 64, 96 x 64, 128 x 64 or 128 x 128 tiles covers the output (use_gemm_narrow).
bool use_gemm_narrow(int64_t M, int64_t N, int64_t K);
// W4A16, 9-128 tokens with K a multiple of 512 where one round of its tiles covers the output
// (9-16 tokens only on 8193-16384 outputs): narrow tiles with row-contiguous LDS stages
// (w4a16_narrow.hip).
bool use_w4a16_narrow(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_w4a16_narrow(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                                    int64_t K, void* y, hipStream_t st);
// One token, K a multiple of 1024 up to 16384: whole weight rows per wave on the vector unit
// (gemm_gemv.hip).
bool use_gemm_gemv(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_gemv(const void* xq, const float* sx, const void* wq, const float* sw, int64_t N,
                            int64_t K, int fmt, void* y, hipStream_t st, const Epilogue& ep);
// One-token linear layer in one launch: the GEMV kernel quantizes the bf16 row itself (per
// token, bit-identical to the quantizer) and also stores the codes and the scale.
hipError_t launch_linear_gemv(const void* xbf, const void* wq, const float* sw, int64_t N, int64_t K, int fmt,
                              void* xq, float* sx, void* y, hipStream_t st);
hipError_t launch_gemm_narrow(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                              const Epilogue& ep);

// Measurement: one-wave workgroups that record real-time ticks and shader cycles over a
// window of `ticks` real-time ticks (100 MHz).
hipError_t launch_sclk_probe(uint64_t* out, int blocks, int64_t ticks, hipStream_t st);
// Measurement: read n bf16 values and write one byte each (the quantizers' traffic split).
hipError_t launch_stream_probe(const void* x, int64_t n, void* y, hipStream_t st);

}  // namespace w8a8
