// Static per-tensor activation quantization with a saturation monitor, and delayed
// scaling, on gfx950.
//
// With one calibrated scale per tensor the quantizer is a pure elementwise codec,
// x_q = enc(clamp(x / s, +-448)) ("FP8 and INT8 Inference" §5, FP8 in practice: per-tensor
// scaling), or clamp(rne(x / s), +-127) for INT8. Because traffic beyond the calibrated
// maximum saturates, the kernel counts the elements the clamp changed, the per-layer
// monitor the pages recommend ("FP8 and FP4 inference, SmoothQuant and activation
// quantization", Failure modes and how to detect them), and it folds the tensor's amax
// into a running maximum. A one-block kernel then turns that amax into the next step's
// scale through an amax history, the delayed scaling of the first page (§5), so the scale
// never goes through the host.
//
// The quotient x / s is the IEEE fp32 one. It is computed as the FMA-corrected product
// with 1/s, which an exhaustive host check over every bf16 significand of x and every fp32
// significand of s shows to be the IEEE quotient bit for bit wherever it is a normal
// number; for s in [2^-60, 2^60] every quotient that can change a code (|x / s| >= 2^-11)
// is one. Other scales divide per element. Counter and maximum are reduced per block and reach memory
// through at most one vector-memory atomic each per block.
//
// Layout of the work: each thread encodes four 16-byte chunks whose loads are all issued
// first, one block per 1024 chunks (measured on 2048 x 4096 and up: within 1-9% of the
// per-token quantizer when nothing saturates). Variants that did worse: a grid capped at
// 1024 blocks looping over one chunk per thread (2.5 against 2.9 TB/s), a grid capped at
// 512 blocks prefetching its next tile, 1024-thread blocks, eight chunks per thread, and an
// unconditional atomic maximum per block (20 us instead of 6 on 2048 x 4096: atomics on one
// address serialize). When every block saturates, its count atomic costs about 2 us per
// call at 2048 x 4096.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {

template <bool INT8>
__global__ __launch_bounds__(256) void quant_static_kernel(const u32x4* __restrict__ x,
                                                           int64_t nchunks,
                                                           const float* __restrict__ scale,
                                                           u32x2* __restrict__ q,
                                                           uint32_t* __restrict__ saturated,
                                                           float* __restrict__ amax_out) {
  const float s = scale[0];
  const float rcp = 1.0f / s;
  // For s in [2^-60, 2^60] the FMA-corrected quotient equals the IEEE one wherever it can
  // decide a code; outside that range (and for a non-finite s) divide per element.
  const bool shortcut = s >= 0x1p-60f && s <= 0x1p60f;
  uint32_t sat = 0;
  float amax = 0.0f;
  // Thread t of block b owns the chunks b * 1024 + t + 256 i, i < 4: all four loads are
  // issued before the first is encoded, so each thread keeps 64 bytes in flight.
  const int64_t c0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (c0 + 256 * i < nchunks) ? __builtin_nontemporal_load(x + c0 + 256 * i) : u32x4{0u, 0u, 0u, 0u};
  auto run = [&](auto fast) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t c = c0 + 256 * i;
      if (c >= nchunks) break;
      amax = fmaxf(amax, chunk_absmax(v[i]));
      float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                    bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = decltype(fast)::value ? div_static(f[e], s, rcp) : f[e] / s;
      u32x2 o;
      if constexpr (INT8) {
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float r = __builtin_rintf(f[e]);
          sat += (fabsf(r) > 127.0f) ? 1u : 0u;
          b[e] = int8_code(r);
        }
        o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sat += (fabsf(f[e]) > 448.0f) ? 1u : 0u;
          f[e] = clamp448(f[e]);
        }
        o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
        o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
      }
      __builtin_nontemporal_store(o, q + c);   // measured faster here than an ordinary store
    }
  };
  if (shortcut) run(std::true_type{});
  else run(std::false_type{});
  // Per-block totals. Atomics on one address serialize, so a block adds its count only
  // when it saturated something, and raises the maximum only when a plain read shows that
  // its own is larger (amax >= 0, so its bits order like the value).
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sat += __shfl_xor(sat, o, kWave);
  amax = wave_max(amax);
  __shared__ uint32_t rs[4];
  __shared__ float ra[4];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { rs[w] = sat; ra[w] = amax; }
  __syncthreads();
  if (threadIdx.x == 0) {
    sat = rs[0] + rs[1] + rs[2] + rs[3];
    amax = fmaxf(fmaxf(ra[0], ra[1]), fmaxf(ra[2], ra[3]));
    if (saturated && sat) atomicAdd(saturated, sat);
    unsigned int* am = reinterpret_cast<unsigned int*>(amax_out);
    if (amax_out && __float_as_uint(amax) > __atomic_load_n(am, __ATOMIC_RELAXED))
      atomicMax(am, __float_as_uint(amax));
  }
}

// history[step mod H] = amax; amax = 0 (ready for the next step's running maximum);
// scale = fp32(max(max(history), 1e-8)) / qmax. One block of 256 threads.
__global__ __launch_bounds__(256) void delayed_scale_kernel(float* __restrict__ history, int64_t H,
                                                            float* __restrict__ amax, int64_t step,
                                                            float qmax, float* __restrict__ scale) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  if (t == 0) history[step % H] = amax[0];
  __syncthreads();
  float m = 0.0f;
  for (int64_t i = t; i < H; i += 256) m = fmaxf(m, history[i]);
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    scale[0] = fmaxf(m, 1e-8f) / qmax;
    amax[0] = 0.0f;
  }
}

hipError_t launch_quantize_static(const void* x, int64_t M, int64_t K, int fmt, const float* scale,
                                  void* q, uint32_t* saturated, float* amax, hipStream_t st) {
  const int64_t nchunks = M * K / 8;
  const int blocks = (int)((nchunks + 1023) / 1024);   // 4 chunks per thread, 256 threads
  if (fmt == 1)
    hipLaunchKernelGGL(quant_static_kernel<true>, dim3(blocks), dim3(256), 0, st,
                       (const u32x4*)x, nchunks, scale, (u32x2*)q, saturated, amax);
  else
    hipLaunchKernelGGL(quant_static_kernel<false>, dim3(blocks), dim3(256), 0, st,
                       (const u32x4*)x, nchunks, scale, (u32x2*)q, saturated, amax);
  return hipGetLastError();
}

hipError_t launch_delayed_scale(float* history, int64_t H, float* amax, int64_t step, int fmt,
                                float* scale, hipStream_t st) {
  hipLaunchKernelGGL(delayed_scale_kernel, dim3(1), dim3(256), 0, st, history, H, amax, step,
                     fmt == 1 ? 127.0f : 448.0f, scale);
  return hipGetLastError();
}

}  // namespace w8a8
