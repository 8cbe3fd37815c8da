// SmoothQuant preparation kernels (offline step of the INT8 W8A8 variant):
// per-input-channel maxima, smoothing factors s_j = a_j^alpha / w_j^(1-alpha), and the
// column rescaling X / s, W * s back to bf16 ("FP8 and FP4 inference, SmoothQuant and
// activation quantization", SmoothQuant section and the `smooth` emulation; "Low-bit LLM
// Weights and Activations" §4.2-4.3).
#include "common.h"
#include "internal.h"

namespace w8a8 {

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// Column maxima of a bf16 [R, K] matrix. Each thread owns 8 adjacent columns (one 16-byte
// chunk per row) and walks a strided subset of the rows; partial maxima meet in an
// integer atomic max (non-negative floats order like their bit patterns).
__global__ __launch_bounds__(256) void channel_absmax_kernel(const uint16_t* __restrict__ x,
                                                             int64_t R, int64_t K, int rows_per,
                                                             float* __restrict__ amax) {
  const int64_t kc = K >> 3;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= kc) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = min(R, r0 + rows_per);
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r = r0; r < r1; ++r) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x + r * K)[c];
    m[0] = fmaxf(m[0], fabsf(bf16_lo(v.x))); m[1] = fmaxf(m[1], fabsf(bf16_hi(v.x)));
    m[2] = fmaxf(m[2], fabsf(bf16_lo(v.y))); m[3] = fmaxf(m[3], fabsf(bf16_hi(v.y)));
    m[4] = fmaxf(m[4], fabsf(bf16_lo(v.z))); m[5] = fmaxf(m[5], fabsf(bf16_hi(v.z)));
    m[6] = fmaxf(m[6], fabsf(bf16_lo(v.w))); m[7] = fmaxf(m[7], fabsf(bf16_hi(v.w)));
  }
  unsigned int* out = reinterpret_cast<unsigned int*>(amax) + c * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) atomicMax(out + e, __float_as_uint(m[e]));
}

hipError_t launch_channel_absmax(const void* x, int64_t R, int64_t K, float* amax,
                                 hipStream_t st) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                     amax, K);
  if (R == 0) return hipGetLastError();
  const int64_t kc = K >> 3;
  const int rows_per = 64;
  dim3 grid((unsigned)((kc + 255) / 256), (unsigned)((R + rows_per - 1) / rows_per));
  hipLaunchKernelGGL(channel_absmax_kernel, grid, dim3(256), 0, st, (const uint16_t*)x, R, K,
                     rows_per, amax);
  return hipGetLastError();
}

// s_j in fp32. alpha = 1/2: correctly rounded square roots and one IEEE division (the
// default HIP lowering of sqrtf and '/' is correctly rounded); alpha = 0 / 1: 1/w and a.
__global__ void smooth_scales_kernel(const float* __restrict__ a, const float* __restrict__ w,
                                     int64_t K, float alpha, float* __restrict__ s) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const float aj = fmaxf(a[j], 1e-5f);
  const float wj = fmaxf(w[j], 1e-5f);
  float r;
  if (alpha == 0.5f) r = sqrtf(aj) / sqrtf(wj);
  else if (alpha == 0.0f) r = 1.0f / wj;
  else if (alpha == 1.0f) r = aj;
  else r = exp2f(alpha * log2f(aj) - (1.0f - alpha) * log2f(wj));
  s[j] = r;
}

hipError_t launch_smooth_scales(const float* a, const float* w, int64_t K, float alpha,
                                float* s, hipStream_t st) {
  hipLaunchKernelGGL(smooth_scales_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                     a, w, K, alpha, s);
  return hipGetLastError();
}

// out[r, j] = bf16(x[r, j] / s[j]) (mode 0) or bf16(x[r, j] * s[j]) (mode 1).
template <int MODE>
__global__ __launch_bounds__(256) void smooth_apply_kernel(const uint16_t* __restrict__ x,
                                                           int64_t nchunk, int64_t kc,
                                                           const float* __restrict__ s,
                                                           uint16_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nchunk) return;
  const int64_t j0 = (c % kc) * 8;
  const u32x4 v = reinterpret_cast<const u32x4*>(x)[c];
  const u32x4 s0 = *reinterpret_cast<const u32x4*>(s + j0);
  const u32x4 s1 = *reinterpret_cast<const u32x4*>(s + j0 + 4);
  const float sv[8] = {__uint_as_float(s0.x), __uint_as_float(s0.y), __uint_as_float(s0.z),
                       __uint_as_float(s0.w), __uint_as_float(s1.x), __uint_as_float(s1.y),
                       __uint_as_float(s1.z), __uint_as_float(s1.w)};
  const float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = MODE == 0 ? f[e] / sv[e] : __fmul_rn(f[e], sv[e]);
  u32x4 r = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
             pack_bf16x2(o[6], o[7])};
  reinterpret_cast<u32x4*>(out)[c] = r;
}

hipError_t launch_smooth_apply(const void* x, int64_t R, int64_t K, const float* s, int mode,
                               void* out, hipStream_t st) {
  const int64_t nchunk = (R * K) >> 3;
  const int64_t kc = K >> 3;
  dim3 grid((unsigned)((nchunk + 255) / 256)), block(256);
  if (mode == 0)
    hipLaunchKernelGGL(smooth_apply_kernel<0>, grid, block, 0, st, (const uint16_t*)x, nchunk,
                       kc, s, (uint16_t*)out);
  else
    hipLaunchKernelGGL(smooth_apply_kernel<1>, grid, block, 0, st, (const uint16_t*)x, nchunk,
                       kc, s, (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace w8a8
