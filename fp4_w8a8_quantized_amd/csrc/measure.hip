// Measurement helpers (not part of the method).
//
// Shader-clock probe: the peak a kernel is held to depends on
// the clock the chip actually ran at (the matrix cores' rate is a fixed number of
// operations per shader cycle), and under sustained low-precision MFMA load the shader
// clock settles below its 2.4 GHz maximum. Each one-wave workgroup reads the shader-cycle
// counter (s_memtime) and the constant 100 MHz real-time counter (s_memrealtime) at its
// start and again once `ticks` real-time ticks have passed, and stores the two differences.
// Launched on a second stream next to the kernels being measured, it occupies one wave
// slot on `blocks` CUs and leaves the clock to them; the exit condition is the real-time
// bound, which every wave reaches.
#include "common.h"
#include "internal.h"

namespace w8a8 {

__global__ void __launch_bounds__(64) sclk_probe_kernel(uint64_t* __restrict__ out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0, c = c0;
  while (r - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r = __builtin_amdgcn_s_memrealtime();
    c = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = r - r0;
    out[2 * blockIdx.x + 1] = c - c0;
  }
}

hipError_t launch_sclk_probe(uint64_t* out, int blocks, int64_t ticks, hipStream_t st) {
  hipLaunchKernelGGL(sclk_probe_kernel, dim3((unsigned)blocks), dim3(64), 0, st, out, (uint64_t)ticks);
  return hipGetLastError();
}

// Same-split stream: what HBM gives an elementwise codec that reads 2 bytes and writes 1
// byte per element, as the per-token and static quantizers do. Each element's output byte
// is the high byte of its bf16 input (no arithmetic to speak of). Thread t of block b
// handles the 16-byte input chunks b * 1024 + t + 256 i, i < 4, loading all four before
// storing, so that every thread keeps 64 bytes of loads in flight. Loads and stores use the
// quantizers' cache policy (non-temporal loads, ordinary stores).
__global__ void __launch_bounds__(256) stream_probe_kernel(const u32x4* __restrict__ x, int64_t nchunks,
                                                           u32x2* __restrict__ y) {
  const int64_t c0 = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (c0 + 256 * i < nchunks) ? __builtin_nontemporal_load(x + c0 + 256 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (c0 + 256 * i >= nchunks) break;
    const u32x4 a = v[i];
    u32x2 o;
    o.x = ((a.x >> 8) & 0xFFu) | ((a.x >> 16) & 0xFF00u) | (((a.y >> 8) & 0xFFu) << 16) | ((a.y >> 24) << 24);
    o.y = ((a.z >> 8) & 0xFFu) | ((a.z >> 16) & 0xFF00u) | (((a.w >> 8) & 0xFFu) << 16) | ((a.w >> 24) << 24);
    y[c0 + 256 * i] = o;
  }
}

hipError_t launch_stream_probe(const void* x, int64_t n, void* y, hipStream_t st) {
  const int64_t nchunks = n / 8;
  const int64_t blocks = (nchunks + 1023) / 1024;
  hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4*)x,
                     nchunks, (u32x2*)y);
  return hipGetLastError();
}

}  // namespace w8a8
