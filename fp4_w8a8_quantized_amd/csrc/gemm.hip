// GEMM dispatch for the per-token / per-channel scaled forms:
//   FP8   y = epilogue( s_x[m] s_w[n] sum_k dec(xq[m,k]) dec(wq[n,k]) )
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x[m]) s_w[n] ),  acc_i32 = sum_k xq wq
// The scales are applied after the low-precision reduction, which the scale-factoring
// identity diag(s_X)(X_q W_q^T)diag(s_W) allows ("FP8 and FP4 inference, SmoothQuant and
// activation quantization", Scale granularity; "FP8 and INT8 Inference" §6-9, the GEMM
// epilogue; "Low-bit LLM Weights and Activations" §3.4).
//
// Dispatch by shape:
//  - one token (K a multiple of 1024 up to 16384): whole weight rows per wave on the vector
//    unit (gemm_gemv.hip);
//  - 2-128 tokens, and more tokens where one round of 64 x 64, 96 x 64, 128 x 64 or 128 x 128
//    tiles covers the output: narrow tiles sized to the token count (gemm_narrow.hip);
//  - one token that the vector kernel does not take: the weight-streaming split-K kernel
//    (gemm_skinny.hip);
//  - otherwise the prefill kernels (gemm_pp.hip, and gemm_solo.hip for 128-wide tiles): FP8
//    on 16x16x128 MFMAs, INT8 on pairs of 16x16x64 MFMAs over the same fragments.
#include "common.h"
#include "internal.h"

namespace w8a8 {

hipError_t launch_gemm(const void* xq, const float* sx, const void* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                       const Epilogue& ep) {
  if (use_gemm_gemv(M, N, K)) return launch_gemm_gemv(xq, sx, wq, sw, N, K, fmt, y, st, ep);
  if (use_gemm_narrow(M, N, K)) return launch_gemm_narrow(xq, sx, wq, sw, M, N, K, fmt, y, st, ep);
  if (M == 1) return launch_gemm_skinny(xq, sx, wq, sw, M, N, K, fmt, y, st, ep);
  return launch_gemm_pp(xq, sx, wq, sw, M, N, K, fmt, y, st, ep);
}

}  // namespace w8a8
