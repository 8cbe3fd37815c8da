// Shader-clock probe for the measurement protocol: the peak a kernel is held to depends on
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

}  // namespace w8a8
