// W8A8 GEMM for 33-512 tokens on gfx950, the same result as the other GEMMs:
//   FP8   y = epilogue( s_x[m] s_w[n] sum_k dec(xq[m,k]) dec(wq[n,k]) )
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x[m]) s_w[n] )
// ("FP8 and FP4 inference, SmoothQuant and activation quantization", Scale granularity;
// "FP8 and INT8 Inference" §5 and the epilogue of §6-9).
//
// At these token counts a 256-row tile leaves most CUs idle on 4096-wide layers (32
// tiles), and the few-token kernel, whose waves split K, re-reads X from L2 in 16-byte
// loads one step ahead and waits on them. Here a workgroup of 4 (8) waves owns up to 128
// (256) token rows and 16 NW weight rows (16-128; 128 at 4 waves only), so narrow layers
// still spread over every CU:
//  - each K step (128 bytes per row) of the X rows and of the 16 NW W rows lands in LDS by
//    direct-to-LDS loads (8 rows per 1 KB load, spread over the waves);
//  - the weights come from HBM and stream through a ring of up to 16 steps (8 for 64-row
//    panels or 8 waves, 4 for 64-row panels at 8 waves), issued one ring ahead, so that
//    each workgroup keeps 30-56 KB of them in flight; X, which the L2 holds after its
//    first reader, goes through a ring of 4 stages (6 at 4 waves on 16 weight rows),
//    issued three (five) steps ahead;
//  - the weights of a step are always issued before its X, so one hand-counted wait for
//    the step's X covers both;
//  - wave w owns token rows 32 w .. 32 w + 31 (two 16-row subtiles) against every weight
//    row, so no partial sums need to meet; its fragments come from LDS (lane l: row l & 15,
//    16-byte chunks g and g + 4, g = l >> 4, for both operands);
//  - one barrier per step publishes the step's stage and slot and retires the ones read
//    before.
// Rows past M or N re-read the last valid row; their results are never stored.
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

__device__ __forceinline__ int mid_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// One 16-byte direct global->LDS load per lane (lane l writes LDS bytes [m0 + 16 l, +16)),
// with the wait state gfx9 asks for between an SALU write of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void mid_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate (gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int mid_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void mid_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int KIND, int NW, bool OF8, int WAVES>
__global__ void __launch_bounds__(64 * WAVES)
gemm_mid_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
                int K, int ksteps, void* __restrict__ yp, Epilogue ep) {
  constexpr int kMidRowsX = 32 * WAVES;              // token rows per workgroup
  // X stages: 6 for 4 waves on 16 weight rows, else 4 (measured against 3 at 8 waves:
  // 400 x 4096 x 14336 68.6 -> 54.3 us; 6 at 4 waves on 64 weight rows was slower).
  constexpr int S = (WAVES == 4 && NW == 1) ? 6 : 4;
  constexpr int RW = 16 * NW;                        // weight rows per workgroup
  constexpr int XSTAGE = kMidRowsX * 128, WSLOT = RW * 128;
  constexpr int WS0 = (NW >= 4 || WAVES > 4) ? 8 : 16;
  constexpr int WSFIT = (160 * 1024 - S * XSTAGE) / WSLOT;
  constexpr int WS = WSFIT < WS0 ? WSFIT : WS0;      // W ring slots (LDS <= 160 KB)
  static_assert(WS >= S, "weights issued no later than the X of their step");
  constexpr int NDX = kMidRowsX / 8, NDW = RW / 8;   // 1 KB loads per step
  constexpr int LMIN = NDX / WAVES + NDW / WAVES;    // loads per wave per step, at least
  static_assert(S * XSTAGE + WS * WSLOT <= 160 * 1024, "LDS");
  static_assert(LMIN * (S - 2) < 64, "vmcnt holds at most 63");
  typedef typename std::conditional<KIND == 1, i32x4, f32x4>::type acc_t;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * XSTAGE + WS * WSLOT];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * RW, m0 = blockIdx.y * kMidRowsX;
  const int fr = lane & 15, g = lane >> 4;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Epilogue scales first: ordinary loads issued before any direct-to-LDS load, so the
  // hand-counted waits below only see the latter.
  float esm[2], esn[NW][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) esm[i] = sx[min(m0 + 32 * wave + 16 * i + fr, M - 1)];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) esn[j][r] = sw[min(n0 + 16 * j + 4 * g + r, N - 1)];

  // The loads of step ks: load d of its X rows (or W rows) is issued by wave d % WAVES; lane l
  // fetches chunk (l & 7) ^ swizzle of row 8 d + (l >> 3) of the X stage (W slot). Steps
  // past the last re-fetch the last step into a stage or slot that is never read again.
  const uint32_t wlds0 = lds0 + S * XSTAGE;
  auto dma_x = [&](int ks) {
    const uint8_t* xb = xq + (size_t)min(ks, ksteps - 1) * 128;
#pragma unroll
    for (int d = wave; d < NDX; d += WAVES) {
      const int r = 8 * d + (lane >> 3);
      const uint32_t vo = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
      mid_dma16(lds0 + (ks % S) * XSTAGE + d * 1024, vo, xb);
    }
  };
  auto dma_w = [&](int ks) {
    const uint8_t* wb = wq + (size_t)min(ks, ksteps - 1) * 128;
    for (int d = wave; d < NDW; d += WAVES) {
      const int r = 8 * d + (lane >> 3);
      const uint32_t vo = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
      mid_dma16(wlds0 + (ks % WS) * WSLOT + d * 1024, vo, wb);
    }
  };

  acc_t acc[NW][2];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[j][i] = acc_t{};

  // Prologue: the weights of steps 0 .. WS - 2, with the X of steps 0 .. S - 2 after the
  // weights of steps WS - S .. WS - 2, in the order the loop keeps (W of step j + WS - 1,
  // then X of step j + S - 1).
  for (int j = 1 - WS; j < 0; ++j) {
    dma_w(j + WS - 1);
    if (j + S - 1 >= 0) dma_x(j + S - 1);
  }
  for (int ks = 0; ks < ksteps; ++ks) {
    // The X of step ks was issued S - 1 iterations ago, after its weights: once at most the
    // loads of the last S - 2 iterations remain, both have landed for this wave; after the
    // barrier for every wave, and every wave is done with step ks - 1's stage and slot.
    __builtin_amdgcn_s_waitcnt(mid_wait(LMIN * (S - 2), 15));
    mid_barrier();
    dma_w(ks + WS - 1);
    dma_x(ks + S - 1);
    const uint8_t* X = lds + (ks % S) * XSTAGE;
    const uint8_t* W = lds + S * XSTAGE + (ks % WS) * WSLOT;
    i32x4 xl[2], xh[2], wl[NW], wh[NW];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 32 * wave + 16 * i + fr;
      xl[i] = *reinterpret_cast<const i32x4*>(X + mid_off(row, g));
      xh[i] = *reinterpret_cast<const i32x4*>(X + mid_off(row, g + 4));
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const int row = 16 * j + fr;
      wl[j] = *reinterpret_cast<const i32x4*>(W + mid_off(row, g));
      wh[j] = *reinterpret_cast<const i32x4*>(W + mid_off(row, g + 4));
    }
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (KIND == 1) {
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl[j], xl[i], acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh[j], xh[i], acc[j][i], 0, 0, 0);
        } else {
          const i32x8 a = {wl[j][0], wl[j][1], wl[j][2], wl[j][3], wh[j][0], wh[j][1], wh[j][2], wh[j][3]};
          const i32x8 b = {xl[i][0], xl[i][1], xl[i][2], xl[i][3], xh[i][0], xh[i][1], xh[i][2], xh[i][3]};
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j][i], 0, 0, 0, 0, 0, 0);
        }
      }
  }
  __builtin_amdgcn_s_waitcnt(mid_wait(0, 0));       // the re-fetches past the end

  // Epilogue, straight from registers: lane l holds token row 32 w + 16 i + (l & 15) and
  // the four consecutive outputs n0 + 16 j + 4 (l >> 4) + r.
  epi_dispatch(ep.act, ep.bias != nullptr, [&](auto act_c, auto bias_c) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool BIAS = decltype(bias_c)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = m0 + 32 * wave + 16 * i + fr;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const int n = n0 + 16 * j + 4 * g;
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (KIND == 1) v[r] = mul_rn(mul_rn((float)acc[j][i][r], esm[i]), esn[j][r]);
          else v[r] = acc[j][i][r] * (esm[i] * esn[j][r]);
          if constexpr (BIAS) v[r] = add_rn(v[r], bf16_lo(ep.bias[min(n + r, N - 1)]));
          v[r] = epi_act<ACT>(v[r]);
        }
        if constexpr (OF8) {
          constexpr bool EX = (KIND == 1);
          const uint32_t o = pack_e4m3x4(epi_requant<EX>(v[0], ep.s_out, ep.inv_s_out), epi_requant<EX>(v[1], ep.s_out, ep.inv_s_out),
                                         epi_requant<EX>(v[2], ep.s_out, ep.inv_s_out), epi_requant<EX>(v[3], ep.s_out, ep.inv_s_out));
          uint8_t* yr = reinterpret_cast<uint8_t*>(yp) + (size_t)m * N;
          if ((N & 3) == 0) {
            *reinterpret_cast<uint32_t*>(yr + n) = o;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) yr[n + r] = (uint8_t)((o >> (8 * r)) & 0xFFu);
          }
        } else {
          uint16_t* yr = reinterpret_cast<uint16_t*>(yp) + (size_t)m * N;
          const uint32_t o[2] = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          if ((N & 3) == 0) {
            *reinterpret_cast<u32x2*>(yr + n) = u32x2{o[0], o[1]};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) yr[n + r] = (uint16_t)((o[r >> 1] >> (16 * (r & 1))) & 0xFFFFu);
          }
        }
      }
    }
  });
}

template <int KIND, int NW, int WAVES>
hipError_t launch_mid_cfg(const void* xq, const float* sx, const void* wq, const float* sw,
                          int64_t M, int64_t N, int64_t K, void* y, hipStream_t st,
                          const Epilogue& ep) {
  const dim3 grid((unsigned)((N + 16 * NW - 1) / (16 * NW)), (unsigned)((M + 32 * WAVES - 1) / (32 * WAVES)));
  const dim3 block(64 * WAVES);
  if (ep.out_fp8)
    hipLaunchKernelGGL((gemm_mid_kernel<KIND, NW, true, WAVES>), grid, block, 0, st, (const uint8_t*)xq,
                       sx, (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, (int)(K / 128), y, ep);
  else
    hipLaunchKernelGGL((gemm_mid_kernel<KIND, NW, false, WAVES>), grid, block, 0, st, (const uint8_t*)xq,
                       sx, (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, (int)(K / 128), y, ep);
  return hipGetLastError();
}

template <int KIND, int WAVES>
hipError_t launch_mid_nw(const void* xq, const float* sx, const void* wq, const float* sw,
                         int64_t M, int64_t N, int64_t K, void* y, hipStream_t st,
                         const Epilogue& ep) {
  const int rw = mid_weight_rows(M, N);
  if (rw == 16) return launch_mid_cfg<KIND, 1, WAVES>(xq, sx, wq, sw, M, N, K, y, st, ep);
  if (rw == 32) return launch_mid_cfg<KIND, 2, WAVES>(xq, sx, wq, sw, M, N, K, y, st, ep);
  if (rw == 64) return launch_mid_cfg<KIND, 4, WAVES>(xq, sx, wq, sw, M, N, K, y, st, ep);
  if constexpr (WAVES == 4)
    if (rw == 128) return launch_mid_cfg<KIND, 8, WAVES>(xq, sx, wq, sw, M, N, K, y, st, ep);
  return hipErrorInvalidValue;                      // the dispatcher sends no such shape
}

}  // namespace

// Weight rows per workgroup: 16, 32, 64 or (up to 128 tokens) 128, the fewest that keep
// the workgroups (one row of them per 256 tokens) to one round over the 256 CUs; 0 if none
// does. Every workgroup re-reads its tokens' X, so fewer, wider workgroups cost little
// (128 x 28672 x 4096: 37 us on 128-row panels, 39 us on the 256-row tiled kernel).
int mid_weight_rows(int64_t M, int64_t N) {
  const int64_t rows = (M + 255) / 256;
  const int max_rw = M <= 128 ? 128 : 64;           // 128 rows: 4 waves only (LDS)
  for (int rw = 16; rw <= max_rw; rw *= 2)
    if (rows * ((N + rw - 1) / rw) <= 256) return rw;
  return 0;
}

// 4 waves up to 128 tokens, 8 waves (rows of workgroups 256 tokens tall) above.
hipError_t launch_gemm_mid(const void* xq, const float* sx, const void* wq, const float* sw,
                           int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                           const Epilogue& ep) {
  if (M <= 128)
    return fmt == 1 ? launch_mid_nw<1, 4>(xq, sx, wq, sw, M, N, K, y, st, ep)
                    : launch_mid_nw<0, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
  return fmt == 1 ? launch_mid_nw<1, 8>(xq, sx, wq, sw, M, N, K, y, st, ep)
                  : launch_mid_nw<0, 8>(xq, sx, wq, sw, M, N, K, y, st, ep);
}

}  // namespace w8a8
