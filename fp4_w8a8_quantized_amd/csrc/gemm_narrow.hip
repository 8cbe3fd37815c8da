// W8A8 GEMM on narrow output tiles sized to the token count, the same result as the other
// GEMMs:
//   FP8   y = epilogue( s_x[m] s_w[n] sum_k dec(xq[m,k]) dec(wq[n,k]) )
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x[m]) s_w[n] )
// ("FP8 and FP4 inference, SmoothQuant and activation quantization", Scale granularity;
// "FP8 and INT8 Inference" §5 and the epilogue of §6-9).
//
// Below the ridge point the weights dominate the traffic ("Low-bit LLM Weights and
// Activations" §5): the kernel's time is the time to stream W from HBM once, plus what the
// CUs spend re-reading X from the L2. A workgroup of 4 or 8 waves owns BM token rows (16-128)
// against BN weight rows (16-128), a tile picked so that about one round of workgroups
// covers the output with the fewest bytes per CU (8 waves on the 64- and 128-row tiles):
//  - each LDS stage holds KB bytes of K (256-1024; 128 on the largest tiles) of every X and
//    W row of the tile. A stage is filled by direct-to-LDS loads that each read whole cache
//    lines of 1024 / KB rows, so the weight stream reaches HBM as runs of KB contiguous bytes
//    per row rather than one 128-byte line per row per K step;
//  - a ring of ST stages is issued ST - 1 stages ahead; one barrier per stage publishes it
//    and retires the one read before;
//  - the waves form a WM x WN x WK grid: wave (wm, wn, wk) owns a (BM / WM) x (BN / WN)
//    part of the tile as 16 x 16 subtiles and the K steps s = wk mod WK of every stage. With
//    WK > 1 (tiles too small for 4 waves) the waves' partial sums meet in LDS after the loop,
//    added in wk order;
//  - fragments: for K step s of a stage, lane l reads row l & 15 and the 16-byte chunks
//    8 s + g and 8 s + g + 4 (g = l >> 4) of both operands (16x16x128 FP8 MFMAs, or two
//    16x16x64 INT8 MFMAs); in LDS, chunk c of row r sits at slot c ^ swz(r), which keeps the
//    16 rows of a fragment read on distinct banks;
//  - the epilogue runs from registers.
// Workgroup ids are dealt round-robin over the 8 XCDs; they are remapped so that the row
// tiles that share a weight panel run on one XCD. Rows past M or N re-read the last valid
// row; their results are never stored.
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

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

// Slot of 16-byte chunk c of row r in a stage of KB-byte rows. With KB >= 256 the XOR of
// the row's low 4 bits puts the 16 rows of a fragment read on 16 distinct 16-byte bank
// groups; 128-byte rows pair up within 256 bytes, hence the shift.
template <int KB>
__device__ __forceinline__ int nw_slot(int r, int c) {
  if constexpr (KB >= 256) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

template <int KIND, int BM, int BN, int WK, int KB, int ST, bool OF8, int NWV>
__global__ void __launch_bounds__(64 * NWV)
gemm_narrow_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                   const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
                   int K, int kblocks, int ksteps, int tiles_m, void* __restrict__ yp, Epilogue ep) {
  constexpr int WMN = NWV / WK;
  constexpr int WM = (BM >= 32 && WMN >= 2) ? 2 : 1, WN = WMN / WM;
  constexpr int TM = BM / WM, TN = BN / WN;          // wave tile
  constexpr int SM = TM / 16, SN = TN / 16;          // 16 x 16 subtiles per wave
  static_assert(WK * WMN == NWV && SM >= 1 && SN >= 1 && SM * 16 * WM == BM && SN * 16 * WN == BN, "tile shape");
  constexpr int SPB = KB / 128;                      // K steps per stage
  static_assert(SPB % WK == 0, "every wave takes the same number of steps per stage");
  constexpr int RPL = 1024 / KB, LPR = KB / 16;      // rows per 1 KB load, lanes per row
  constexpr int XST = BM * KB, STAGE = (BM + BN) * KB;
  constexpr int NDX = BM / RPL, ND = (BM + BN) / RPL;   // 1 KB loads per stage
  static_assert(BM % RPL == 0 && BN % RPL == 0, "whole rows per load");
  constexpr int NQ = (ND + NWV - 1) / NWV;           // loads per wave per stage, at most
  constexpr int NDR = ND % NWV;                      // waves below NDR issue NQ, others NQ - 1
  constexpr int LA = NQ, LB = NDR == 0 ? NQ : NQ - 1;
  static_assert(ST >= 3 && LA * (ST - 2) < 64, "vmcnt holds at most 63");
  static_assert(ST * STAGE <= 160 * 1024, "LDS");
  typedef typename std::conditional<KIND == 1, i32x4, f32x4>::type acc_t;
  static_assert(WK == 1 || (WK - 1) * WMN * SN * SM * 64 * 16 <= ST * STAGE, "reduction area");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[ST * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wk = wave % WK, wmn = wave / WK;
  const int wm = wmn / WN, wn = wmn % WN;
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

  // The loads of stage kb (load d is issued by wave d % 4): lane l fills slot l % LPR of
  // tile row RPL d' + l / LPR of the X rows (d < NDX) or the W rows, reading the chunk that
  // the slot holds. The row's offset and the slot's chunk are fixed for the whole loop; the
  // stage's K offset goes into the scalar base. In a last, partial stage the chunks past K
  // re-read the row's last chunk instead; the steps they would feed are skipped.
  const int lrow = lane / LPR, lslot = lane % LPR;
  uint32_t vrow[NQ], vchunk[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int d = min(wave + NWV * q, ND - 1);
    const bool isx = d < NDX;
    const int r = RPL * (isx ? d : d - NDX) + lrow;
    const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
    vrow[q] = (uint32_t)row * (uint32_t)K;
    vchunk[q] = (uint32_t)nw_slot<KB>(r, lslot) << 4;
  }
  auto dma = [&](int kb, auto partial) {
    const uint32_t sb = lds0 + (kb % ST) * STAGE;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int d = wave + NWV * q;
      if (d < ND) {
        const bool isx = d < NDX;
        const uint32_t la = sb + (isx ? 0 : XST) + (isx ? d : d - NDX) * 1024;
        const uint8_t* base = isx ? xq : wq;
        if constexpr (decltype(partial)::value)
          nw_dma16(la, vrow[q] + (uint32_t)min(kb * KB + (int)vchunk[q], K - 16), base);
        else
          nw_dma16(la, vrow[q] + vchunk[q], base + (size_t)kb * KB);
      }
    }
  };
  const int kfull = ksteps / SPB;                    // stages holding SPB whole steps
  auto issue = [&](int kb) {
    if (kb < kfull) dma(kb, std::false_type{});
    else if (kb < kblocks) dma(kb, std::true_type{});
  };
  // Stage kb has landed for this wave once at most the loads of the stages after it that
  // were already issued remain: ST - 2 stages in the steady state, none near the end.
  auto wait_stage = [&](int kb) {
    if (kb + ST - 2 < kblocks) {
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

  // One stage's MFMAs: steps ss WK + wk for ss < NS (all SPB / WK of them but in a last,
  // partial stage).
  auto stage_mfma = [&](int kb, int NS) {
    const uint8_t* X = lds + (kb % ST) * STAGE;
    const uint8_t* W = X + XST;
#pragma unroll
    for (int ss = 0; ss < SPB / WK; ++ss) {
      if (ss >= NS) break;
      const int c0 = 8 * (ss * WK + wk) + g;
      i32x4 xl[SM], xh[SM], wl[SN], wh[SN];
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        const int row = wm * TM + 16 * i + fr;
        xl[i] = *reinterpret_cast<const i32x4*>(X + row * KB + (nw_slot<KB>(row, c0) << 4));
        xh[i] = *reinterpret_cast<const i32x4*>(X + row * KB + (nw_slot<KB>(row, c0 + 4) << 4));
      }
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int row = wn * TN + 16 * j + fr;
        wl[j] = *reinterpret_cast<const i32x4*>(W + row * KB + (nw_slot<KB>(row, c0) << 4));
        wh[j] = *reinterpret_cast<const i32x4*>(W + row * KB + (nw_slot<KB>(row, c0 + 4) << 4));
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
  };

  // Full stages in the loop; a last, partial stage (K not a multiple of KB) after it, so
  // that the loop's MFMAs carry no control flow between them.
  for (int kb = 0; kb < ST - 1; ++kb) issue(kb);
  for (int kb = 0; kb < kfull; ++kb) {
    wait_stage(kb);
    nw_barrier();                                    // stage kb visible; stage of kb - 1 free
    issue(kb + ST - 1);
    stage_mfma(kb, SPB / WK);
  }
  if (kfull < kblocks) {
    wait_stage(kfull);
    nw_barrier();
    const int rest = ksteps - kfull * SPB;           // 1 .. SPB - 1 steps
    stage_mfma(kfull, (rest - wk + WK - 1) / WK);
  }

  if constexpr (WK > 1) {
    // Partial sums of waves wk = 1 .. WK - 1 through LDS (the ring is free once every wave
    // has passed the barrier below), added by wave wk = 0 in wk order.
    nw_barrier();
    acc_t* red = reinterpret_cast<acc_t*>(lds);
    auto slot = [&](int k, int j, int i) { return ((((k - 1) * WMN + wmn) * SN + j) * SM + i) * 64 + lane; };
    if (wk > 0) {
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int i = 0; i < SM; ++i) red[slot(wk, j, i)] = acc[j][i];
    }
    __syncthreads();
    if (wk > 0) return;
    for (int k = 1; k < WK; ++k)
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int i = 0; i < SM; ++i) acc[j][i] += red[slot(k, j, i)];
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

template <int KIND, int BM, int BN, int WK, int KB, int ST, int NWV>
hipError_t launch_nw(const void* xq, const float* sx, const void* wq, const float* sw, int64_t M,
                     int64_t N, int64_t K, void* y, hipStream_t st, const Epilogue& ep) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles = tiles_m * (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)tiles), block(64 * NWV);
  const int kblocks = (int)((K + KB - 1) / KB), ksteps = (int)(K / 128);
  if (ep.out_fp8)
    hipLaunchKernelGGL((gemm_narrow_kernel<KIND, BM, BN, WK, KB, ST, true, NWV>), grid, block, 0, st, (const uint8_t*)xq, sx,
                       (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, kblocks, ksteps, tiles_m, y, ep);
  else
    hipLaunchKernelGGL((gemm_narrow_kernel<KIND, BM, BN, WK, KB, ST, false, NWV>), grid, block, 0, st, (const uint8_t*)xq, sx,
                       (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, kblocks, ksteps, tiles_m, y, ep);
  return hipGetLastError();
}

// The tiles, with the stage depth and wave count that measured best for each (FP8, K = 4096;
// LDS per workgroup in brackets, two workgroups share a CU up to 80 KB):
//   0  16 x 16,  4 waves splitting K 4 ways, 512-byte stages x 4  [64 KB]
//   1  16 x 32,  4 waves splitting K 2 ways, 512 x 3              [72 KB]
//   2  16 x 64,  4 waves, 256 x 4                                 [80 KB]
//   3  32 x 64,  4 waves, 512 x 3                                 [144 KB]
//   4-7  (16 | 32) x (64 | 128) on 128-byte steps, 4 waves
//   12  96 x 64, 8 waves, 256 x 3                                [120 KB]
//   8-11 (64 | 128) x (64 | 128), 8 waves: 8 waves issue twice the loads at once, which
//     measured 5-13% faster than 4 on these tiles (512 x 4096 18.4 -> 16.7 us, 48 x 14336
//     16.4 -> 14.9, 384 x 4096 x 14336 52.0 -> 46.4, 100 x 20000 29.0 -> 25.3); on the
//     32 x 64 tile they made no difference.
template <int KIND>
hipError_t launch_nw_cfg(int c, const void* xq, const float* sx, const void* wq, const float* sw,
                         int64_t M, int64_t N, int64_t K, void* y, hipStream_t st, const Epilogue& ep) {
  switch (c) {
    case 0: return launch_nw<KIND, 16, 16, 4, 512, 4, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 1: return launch_nw<KIND, 16, 32, 2, 512, 3, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 2: return launch_nw<KIND, 16, 64, 1, 256, 4, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 3: return launch_nw<KIND, 32, 64, 1, 512, 3, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 4: return launch_nw<KIND, 16, 64, 1, 128, 8, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 5: return launch_nw<KIND, 16, 128, 1, 128, 6, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 6: return launch_nw<KIND, 32, 64, 1, 128, 8, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 7: return launch_nw<KIND, 32, 128, 1, 128, 5, 4>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 8: return launch_nw<KIND, 64, 64, 1, 256, 4, 8>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 9: return launch_nw<KIND, 64, 128, 1, 128, 4, 8>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 10: return launch_nw<KIND, 128, 64, 1, 256, 3, 8>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 11: return launch_nw<KIND, 128, 128, 1, 128, 4, 8>(xq, sx, wq, sw, M, N, K, y, st, ep);
    case 12: return launch_nw<KIND, 96, 64, 1, 256, 3, 8>(xq, sx, wq, sw, M, N, K, y, st, ep);
    default: return hipErrorInvalidValue;
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Tile for M x N (-1: the kernel does not take the shape). The smallest tile whose
// workgroups fit one round of the CUs (two per CU for the tiles of up to 80 KB), as measured
// on MI355X (FP8, graph replay, against the kernels used before: the weight-streaming split-K
// kernel up to 32 tokens, the mid-size kernel above, the 128-byte-step narrow tiles on wide
// layers):
//   K = 4096:  8 x 4096 6.6 -> 5.6 us, 32 x 4096 9.2 -> 6.8, 64 x 4096 11.4 -> 8.7,
//              128 x 4096 12.9 -> 9.9, 16 x 6144 10.1 -> 7.5, 64 x 6144 13.6 -> 10.4,
//              100 x 6144 14.8 -> 11.5, 128 x 8192 16.9 -> 13.3, 8 x 14336 14.0 -> 12.8,
//              32 x 14336 15.2 -> 14.1, 200 x 4096 16.5 -> 15.9, 160 x 6144 18.4 -> 16.3,
//              384 x 6144 23.6 -> 23.0, 512 x 8192 26.8 -> 24.3;
//   K = 14336: 16 x 4096 20.4 -> 13.0 us, 32 x 4096 27.2 -> 16.9, 128 x 4096 35.9 -> 26.3,
//              192 x 4096 48.7 -> 45.9.
// Wider layers take 64 or 128 weight rows, 128 where 64 would need a second round; above
// 128 tokens, 64 x 64 tiles where one round of them covers the output, else 96 x 64, else
// 128 x 64 or 128 x 128. A CU streams its tile's rows at about the same rate whatever the
// tile, so the smallest tiles that fit one round win: 64 x 64 against 128 x 64 took
// 256 x 4096 from 15.8 to 11.9 us, 160 x 4096 15.4 -> 10.9, 256 x 2048 15.6 -> 11.3 and
// 256 x 4096 x 14336 45.5 -> 33.5; 96 x 64 against 128 x 64 took 384 x 4096 15.9 -> 13.7,
// 300 x 4096 15.6 -> 13.2 and 384 x 4096 x 14336 45.5 -> 39.0. The same holds at any token
// count: where one round of these tiles covers the output, the prefill kernels' 256-row tiles
// fill at most half the CUs, and the narrow tiles won on every such shape measured (1024 x 4096
// 29.1 -> 23.0 us, 1024 x 2048 28.6 -> 16.2, 2048 x 2048 28.0 -> 23.1, 900 x 1024 25.7 -> 10.7,
// 8192 x 512 28.0 -> 25.1, 1024 x 4096 x 14336 85.8 -> 68.4, 2048 x 1024 x 14336 81.6 -> 47.2).
int narrow_config(int64_t M, int64_t N) {
  if (M < 2 || N < 1) return -1;
  if (M <= 16) {
    if (cdiv(N, 16) <= 256) return 0;
    if (cdiv(N, 32) <= 512) return 1;
    return cdiv(N, 64) <= 256 ? 4 : 5;
  }
  if (M <= 32) {
    if (2 * cdiv(N, 32) <= 512) return 1;
    if (cdiv(N, 64) <= 256) return 3;
    return 7;
  }
  if (M <= 64) {
    if (4 * cdiv(N, 64) <= 256) return 2;
    if (2 * cdiv(N, 64) <= 256) return 3;
    return cdiv(N, 64) <= 256 ? 8 : 9;
  }
  if (M <= 128) {
    if (4 * cdiv(N, 64) <= 256) return 3;
    if (2 * cdiv(N, 64) <= 256) return 8;
    return cdiv(N, 64) <= 256 ? 10 : 11;
  }
  if (cdiv(M, 64) * cdiv(N, 64) <= 256) return 8;
  if (cdiv(M, 96) * cdiv(N, 64) <= 256) return 12;
  if (cdiv(M, 128) * cdiv(N, 64) <= 256) return 10;
  if (cdiv(M, 128) * cdiv(N, 128) <= 256) return 11;
  return -1;
}

bool use_gemm_narrow(int64_t M, int64_t N, int64_t K) {
  (void)K;
  return narrow_config(M, N) >= 0;
}

hipError_t launch_gemm_narrow(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                              const Epilogue& ep) {
  const int c = narrow_config(M, N);
  if (fmt == 1) return launch_nw_cfg<1>(c, xq, sx, wq, sw, M, N, K, y, st, ep);
  return launch_nw_cfg<0>(c, xq, sx, wq, sw, M, N, K, y, st, ep);
}

}  // namespace w8a8
