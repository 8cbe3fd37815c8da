// W8A8 GEMM on narrow output tiles sized to the token count, the same result as the other
// GEMMs:
//   FP8   y = epilogue( s_x[m] s_w[n] sum_k dec(xq[m,k]) dec(wq[n,k]) )
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x[m]) s_w[n] )
// ("FP8 and FP4 inference, SmoothQuant and activation quantization", Scale granularity;
// "FP8 and INT8 Inference" §5 and the epilogue of §6-9).
//
// Where it is used. Below the ridge point the weights dominate the traffic ("Low-bit LLM
// Weights and Activations" §5). The weight-streaming kernel gives each workgroup 16 weight
// rows, so layers wider than 4096 outputs take more than one round of workgroups over the
// 256 CUs, and the 33-512-token kernel gives each workgroup all token rows against 16-128
// weight rows, so that it reads (M + 16..128) K bytes per CU. Here a workgroup owns BM token
// rows (16, 32, 64 or 128: the token count rounded up, or 128-row tiles above 128 tokens)
// against BN = 64 or 128 weight rows:
//  - 4 waves in a WM x WN grid (WM = 2 from 32 token rows), each owning a (BM / WM) x
//    (BN / WN) part of the tile as 16 x 16 subtiles (16x16x128 FP8 MFMAs, or two 16x16x64
//    INT8 MFMAs per K step);
//  - each K step of the BM X rows and the BN W rows lands in one LDS stage by direct-to-LDS
//    loads (8 rows per 1 KB load, spread over the waves); a ring of ST stages is issued
//    ST - 1 steps ahead, so one barrier per step both publishes a stage and retires the one
//    read before it (measured: 8 stages of 10 KB beat 12 and 15 on 16 x 64 tiles);
//  - fragments: lane l reads row l & 15 and the 16-byte chunks g and g + 4 (g = l >> 4) of
//    the step, for both operands; rows sit 128 B apart with chunk c at slot c ^ ((row >> 1) & 7);
//  - the epilogue runs from registers.
// Workgroup ids are dealt round-robin over the 8 XCDs; they are remapped so that the row
// tiles that share a weight panel run on one XCD. Rows past M or N re-read the last valid
// row; their results are never stored.
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

__device__ __forceinline__ int nw_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// One 16-byte direct global->LDS load per lane (lane l writes LDS bytes [m0 + 16 l, +16)),
// with the wait state gfx9 asks for between an SALU write of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void nw_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate (gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int nw_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void nw_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int KIND, int BM, int BN, int ST, bool OF8>
__global__ void __launch_bounds__(256)
gemm_narrow_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                   const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
                   int K, int ksteps, int tiles_m, void* __restrict__ yp, Epilogue ep) {
  constexpr int WM = BM >= 32 ? 2 : 1, WN = 4 / WM;
  constexpr int TM = BM / WM, TN = BN / WN;          // wave tile
  constexpr int SM = TM / 16, SN = TN / 16;          // 16 x 16 subtiles per wave
  static_assert(SM >= 1 && SN >= 1 && SM * 16 * WM == BM && SN * 16 * WN == BN, "tile shape");
  constexpr int XST = BM * 128, STAGE = (BM + BN) * 128;
  constexpr int NDX = BM / 8, ND = (BM + BN) / 8;    // 1 KB loads per step
  constexpr int NQ = (ND + 3) / 4;                   // loads per wave per step, at most
  constexpr int NDR = ND % 4;                        // waves below NDR issue NQ, others NQ - 1
  constexpr int LA = NQ, LB = NDR == 0 ? NQ : NQ - 1;
  static_assert(ST >= 3 && LA * (ST - 2) < 64, "vmcnt holds at most 63");
  static_assert(ST * STAGE <= 160 * 1024, "LDS");
  typedef typename std::conditional<KIND == 1, i32x4, f32x4>::type acc_t;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[ST * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane & 15, g = lane >> 4;

  // Logical workgroup id: consecutive logical ids (the row tiles of a weight panel) share
  // an XCD and its L2.
  int b = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int tm = b % tiles_m, tn = b / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Epilogue scales first: ordinary loads issued before any direct-to-LDS load, so that the
  // hand-counted waits below only see the latter.
  float esm[SM], esn[SN][4];
#pragma unroll
  for (int i = 0; i < SM; ++i) esm[i] = sx[min(m0 + wm * TM + 16 * i + fr, M - 1)];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) esn[j][r] = sw[min(n0 + wn * TN + 16 * j + 4 * g + r, N - 1)];

  // The loads of K step s (load d is issued by wave d % 4): lane l fetches chunk
  // (l & 7) ^ swizzle of row 8 d' + (l >> 3) of the X rows (d < NDX) or the W rows.
  auto dma = [&](int s) {
    const size_t kb = (size_t)s * 128;
    const uint32_t sb = lds0 + (s % ST) * STAGE;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int d = wave + 4 * q;
      if (d < ND) {
        const bool isx = d < NDX;
        const int dd = isx ? d : d - NDX;
        const int r = 8 * dd + (lane >> 3);
        const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
        const uint32_t vo = (uint32_t)row * (uint32_t)K + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
        nw_dma16(sb + (isx ? 0 : XST) + dd * 1024, vo, (isx ? xq : wq) + kb);
      }
    }
  };
  // Step s has landed for this wave once at most the loads of the steps after it that were
  // already issued remain: ST - 2 steps in the steady state, none near the end.
  auto wait_step = [&](int s) {
    if (s + ST - 2 < ksteps) {
      if (wave < NDR || NDR == 0) __builtin_amdgcn_s_waitcnt(nw_wait(LA * (ST - 2), 15));
      else __builtin_amdgcn_s_waitcnt(nw_wait(LB * (ST - 2), 15));
    } else {
      __builtin_amdgcn_s_waitcnt(nw_wait(0, 15));
    }
  };

  acc_t acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = acc_t{};

  for (int s = 0; s < ST - 1 && s < ksteps; ++s) dma(s);
  for (int s = 0; s < ksteps; ++s) {
    wait_step(s);
    nw_barrier();                                    // step s visible; stage of s - 1 free
    if (s + ST - 1 < ksteps) dma(s + ST - 1);
    const uint8_t* X = lds + (s % ST) * STAGE;
    const uint8_t* W = X + XST;
    i32x4 xl[SM], xh[SM], wl[SN], wh[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int row = wm * TM + 16 * i + fr;
      xl[i] = *reinterpret_cast<const i32x4*>(X + nw_off(row, g));
      xh[i] = *reinterpret_cast<const i32x4*>(X + nw_off(row, g + 4));
    }
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int row = wn * TN + 16 * j + fr;
      wl[j] = *reinterpret_cast<const i32x4*>(W + nw_off(row, g));
      wh[j] = *reinterpret_cast<const i32x4*>(W + nw_off(row, g + 4));
    }
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        if constexpr (KIND == 1) {
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl[j], xl[i], acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh[j], xh[i], acc[j][i], 0, 0, 0);
        } else {
          const i32x8 a = {wl[j][0], wl[j][1], wl[j][2], wl[j][3], wh[j][0], wh[j][1], wh[j][2], wh[j][3]};
          const i32x8 bx = {xl[i][0], xl[i][1], xl[i][2], xl[i][3], xh[i][0], xh[i][1], xh[i][2], xh[i][3]};
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bx, acc[j][i], 0, 0, 0, 0, 0, 0);
        }
      }
  }

  // Epilogue from registers: lane l holds token row m0 + wm TM + 16 i + (l & 15) and the four
  // consecutive outputs n0 + wn TN + 16 j + 4 (l >> 4) + r.
  epi_dispatch(ep.act, ep.bias != nullptr, [&](auto act_c, auto bias_c) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool BIAS = decltype(bias_c)::value;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int m = m0 + wm * TM + 16 * i + fr;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int n = n0 + wn * TN + 16 * j + 4 * g;
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

template <int KIND, int BM, int BN, int ST>
hipError_t launch_nw(const void* xq, const float* sx, const void* wq, const float* sw, int64_t M,
                     int64_t N, int64_t K, void* y, hipStream_t st, const Epilogue& ep) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles = tiles_m * (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(256);
  if (ep.out_fp8)
    hipLaunchKernelGGL((gemm_narrow_kernel<KIND, BM, BN, ST, true>), grid, block, 0, st, (const uint8_t*)xq, sx,
                       (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, (int)(K / 128), tiles_m, y, ep);
  else
    hipLaunchKernelGGL((gemm_narrow_kernel<KIND, BM, BN, ST, false>), grid, block, 0, st, (const uint8_t*)xq, sx,
                       (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, (int)(K / 128), tiles_m, y, ep);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_nw_kind(int bm, int bn, const void* xq, const float* sx, const void* wq, const float* sw,
                          int64_t M, int64_t N, int64_t K, void* y, hipStream_t st, const Epilogue& ep) {
  // Stage counts: as many 1 KB-row stages as fit in about 80-128 KB (more measured slower).
#define W8A8_NW(TBM, TBN, TST) \
  if (bm == TBM && bn == TBN) return launch_nw<KIND, TBM, TBN, TST>(xq, sx, wq, sw, M, N, K, y, st, ep);
  W8A8_NW(16, 64, 8)
  W8A8_NW(16, 128, 6)
  W8A8_NW(32, 64, 8)
  W8A8_NW(32, 128, 5)
  W8A8_NW(64, 64, 6)
  W8A8_NW(64, 128, 4)
  W8A8_NW(128, 64, 4)
  W8A8_NW(128, 128, 4)
#undef W8A8_NW
  return hipErrorInvalidValue;
}

}  // namespace

// Where the narrow-tile kernel measured faster than the others (K = 4096 and 14336, N in
// {4096, 6144, 14336, 28672}, MI355X): up to 64 tokens on layers wider than 4096 outputs
// (the weight-streaming kernel needs more than one round of 16-row workgroups there: 32 x
// 6144 15.7 -> 11.2 us, 1 x 14336 17.3 -> 14.1 us, 64 x 28672 32.1 -> 28.9 us), 65-128
// tokens above 8192 outputs (128 x 14336 21.5 -> 19.8 us), and 256-512 tokens where one
// round of 128 x 64 tiles covers the output (512 x 4096 21.2 -> 18.4 us, 256 x 4096 x 14336
// 58.5 -> 50.7 us). It lost at 4096 outputs up to 192 tokens and where tiles need a
// second round.
bool use_gemm_narrow(int64_t M, int64_t N, int64_t K) {
  (void)K;
  if (M <= 64) return N > 4096;
  if (M <= 128) return N > 8192;
  if (M >= 256 && M <= 512) return ((M + 127) / 128) * ((N + 63) / 64) <= 256;
  return false;
}

// Tile: token rows = the token count rounded up to 16, 32, 64 or 128 (128-row tiles above
// 128 tokens); weight rows 64, or 128 where 64 would need more than one round of tiles.
hipError_t launch_gemm_narrow(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                              const Epilogue& ep) {
  const int bm = M <= 16 ? 16 : M <= 32 ? 32 : M <= 64 ? 64 : 128;
  const int64_t tiles64 = ((M + bm - 1) / bm) * ((N + 63) / 64);
  const int bn = tiles64 > 256 ? 128 : 64;
  if (fmt == 1) return launch_nw_kind<1>(bm, bn, xq, sx, wq, sw, M, N, K, y, st, ep);
  return launch_nw_kind<0>(bm, bn, xq, sx, wq, sw, M, N, K, y, st, ep);
}

}  // namespace w8a8
