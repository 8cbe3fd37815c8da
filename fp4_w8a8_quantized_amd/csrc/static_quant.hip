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
// Arithmetic: a chunk of eight elements takes the clamp and the saturation count only when
// its largest magnitude saturates (the quotient is monotone in |x|); every other chunk costs
// what the per-token quantizer's encode costs. Before that split the kernel ran 8-15% behind
// the per-token quantizer on the same bytes.
//
// Layout of the work: each thread encodes two or four 16-byte chunks whose loads are all
// issued first, 256 threads a block. Measured, X read from HBM: 6.6 us at 2048 x 4096 and
// 16.9 us at 2048 x 14336, against 6.8 and 17.6 us for the per-token quantizer; 33.7 us at
// 16384 x 4096 (equal). Variants that did worse: a grid capped at 1024 blocks looping over one
// chunk per thread, a grid capped at 512 blocks prefetching its next tile, 1024-thread blocks,
// eight chunks per thread, ordinary loads, and an unconditional atomic maximum per block
// (20 us instead of 6 on 2048 x 4096).
//
// Atomics on one address serialize at about 5 ns each. Each block that saturated something
// adds its count with one atomic, and that is the whole cost of saturation: about 1 us per
// 200 saturating blocks (2048 x 4096 with 200 saturated elements: 7.7 against 6.6 us).
// Reordering the block's atomics, or issuing them at agent scope, did not change it.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {

template <bool INT8, int CH, bool NTL, bool NTS>
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
  // Thread t of block b owns the chunks b * 256 * CH + t + 256 i, i < CH: all CH loads are
  // issued before the first is encoded.
  const int64_t c0 = (int64_t)blockIdx.x * (256 * CH) + threadIdx.x;
  u32x4 v[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = c0 + 256 * i;
    v[i] = c < nchunks ? (NTL ? __builtin_nontemporal_load(x + c) : x[c]) : u32x4{0u, 0u, 0u, 0u};
  }
  auto run = [&](auto fast) {
    constexpr bool F = decltype(fast)::value;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int64_t c = c0 + 256 * i;
      if (c >= nchunks) break;
      // The quotient is monotone in |x|, so an element of the chunk saturates exactly when
      // the chunk's largest magnitude does. Chunks that do not saturate (almost all of
      // them) skip the clamp and the count; their quotients cannot overflow either.
      const float cm = chunk_absmax(v[i]);
      amax = fmaxf(amax, cm);
      const float qm = F ? div_static(cm, s, rcp) : cm / s;
      const bool clips = INT8 ? __builtin_rintf(qm) > 127.0f : qm > 448.0f;
      float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                    bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
      if (!clips) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = F ? div_by_scale(f[e], s, rcp) : f[e] / s;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[e] = F ? div_static(f[e], s, rcp) : f[e] / s;
          if constexpr (INT8) {
            f[e] = __builtin_rintf(f[e]);
            sat += (fabsf(f[e]) > 127.0f) ? 1u : 0u;
          } else {
            sat += (fabsf(f[e]) > 448.0f) ? 1u : 0u;
            f[e] = clamp448(f[e]);
          }
        }
      }
      u32x2 o;
      if constexpr (INT8) {
        o.x = int8_code(f[0]) | (int8_code(f[1]) << 8) | (int8_code(f[2]) << 16) | (int8_code(f[3]) << 24);
        o.y = int8_code(f[4]) | (int8_code(f[5]) << 8) | (int8_code(f[6]) << 16) | (int8_code(f[7]) << 24);
      } else {
        o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
        o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
      }
      if constexpr (NTS) __builtin_nontemporal_store(o, q + c);
      else q[c] = o;
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

template <int CH, bool NTL, bool NTS>
static void launch_static(const void* x, int64_t nchunks, int fmt, const float* scale, void* q,
                          uint32_t* saturated, float* amax, hipStream_t st) {
  const int blocks = (int)((nchunks + 256 * CH - 1) / (256 * CH));
  if (fmt == 1)
    hipLaunchKernelGGL((quant_static_kernel<true, CH, NTL, NTS>), dim3(blocks), dim3(256), 0, st,
                       (const u32x4*)x, nchunks, scale, (u32x2*)q, saturated, amax);
  else
    hipLaunchKernelGGL((quant_static_kernel<false, CH, NTL, NTS>), dim3(blocks), dim3(256), 0, st,
                       (const u32x4*)x, nchunks, scale, (u32x2*)q, saturated, amax);
}

hipError_t launch_quantize_static(const void* x, int64_t M, int64_t K, int fmt, const float* scale,
                                  void* q, uint32_t* saturated, float* amax, hipStream_t st) {
  // Four chunks per thread up to 2^21 chunks (16 Mi elements), two above: measured on
  // 2048 x 4096 (6.6 against 6.9 us) and on 2048 x 14336 to 16384 x 4096 (2-3% the other way).
  const int64_t nchunks = M * K / 8;
  if (nchunks <= ((int64_t)1 << 21))
    launch_static<4, true, true>(x, nchunks, fmt, scale, q, saturated, amax, st);
  else
    launch_static<2, true, true>(x, nchunks, fmt, scale, q, saturated, amax, st);
  return hipGetLastError();
}

hipError_t launch_delayed_scale(float* history, int64_t H, float* amax, int64_t step, int fmt,
                                float* scale, hipStream_t st) {
  hipLaunchKernelGGL(delayed_scale_kernel, dim3(1), dim3(256), 0, st, history, H, amax, step,
                     fmt == 1 ? 127.0f : 448.0f, scale);
  return hipGetLastError();
}

}  // namespace w8a8
