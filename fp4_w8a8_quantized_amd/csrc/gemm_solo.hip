// W8A8 GEMM on gfx950 with one wave per SIMD:
//   FP8   y = epilogue( s_x[m] s_w[n] sum_k dec(xq[m,k]) dec(wq[n,k]) )   (v_mfma 16x16x128 f8f6f4)
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x[m]) s_w[n] )   (two v_mfma_i32_16x16x64_i8 per
//         subtile and step on the same fragments; the INT8 form of the ping-pong kernel)
// with the scale factoring of "FP8 and FP4 inference, SmoothQuant and activation
// quantization" (Scale granularity) and the epilogue of "FP8 and INT8 Inference" §6-9.
//
// A 256-thread workgroup (4 waves, one per SIMD) computes a 256 x 128 tile; each wave owns
// 128 x 64 of it, 8 x 4 subtiles of 16 x 16, i.e. 32 MFMAs per 128-byte K step against 12
// fragment reads (24 KB per wave, 96 KB per step for the workgroup). The two-waves-per-SIMD
// kernel reads 128 KB per step for the same tile (64 x 64 wave tiles) and spends three
// barriers per step handing the matrix core between its wave groups.
//
// Pipeline, per K step s (LDS ring of three stages, stage s % 3 holds step s):
//  - the 32 MFMAs of step s run on fragments read during step s - 1;
//  - between them the wave reads step s + 1's fragments (the other register set) from
//    stage (s + 1) % 3, and issues its 12 direct-to-LDS loads of step s + 3 into stage
//    s % 3, whose fragments every wave finished reading before the last barrier;
//  - at the end of the step it waits for its loads of step s + 2 (its loads of step s + 3
//    may stay in flight) and for its fragment reads, then one barrier: step s + 2 is then
//    complete in LDS and stage (s + 1) % 3 is free for the next refill.
// The loop is unrolled by six so that the two fragment register sets swap roles without
// copies and every stage address is a constant. Every step reads and loads (past the end, re-fetches of the last step into a
// stage nobody reads again), so the MFMA sequence has no branches.
//
// Fragments: lane l reads row l & 15 and the 16-byte chunks g and g + 4 (g = l >> 4) of the
// 128-byte K step; both operands permute K the same way, so every dot product still covers
// the whole step. Rows sit 128 B apart with chunk c at slot c ^ ((row >> 1) & 7).
//
// Epilogue: scale, bias, activation, convert (bf16, or E4M3FN of clamp(v / s_out)) in
// registers, stage the tile through the freed LDS, write whole rows with 16-byte stores.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int kSoloBM = 256, kSoloBN = 128, kSoloThreads = 256;

__device__ __forceinline__ int so_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// One 16-byte direct global->LDS load per lane (lane l writes LDS bytes [m0 + 16 l, +16)),
// with the wait state gfx9 asks for between an SALU write of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void so_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate (gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int so_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void so_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef int sfrag_t __attribute__((ext_vector_type(8)));

template <int KIND, bool OF8>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
gemm_solo_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                 const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
                 int Kb, int ksteps, void* __restrict__ yp, int tiles_m, int vec_store, Epilogue ep) {
  constexpr int BM = kSoloBM, BN = kSoloBN;
  constexpr int WR = 128, WC = 64;                  // wave tile (2 x 2 waves)
  constexpr int SM = WR / 16, SN = WC / 16;         // 8 x 4 subtiles
  constexpr int T = SM * SN;                        // 32 MFMAs per step
  constexpr int XT = BM * 128, WT = BN * 128, STAGE = XT + WT;
  constexpr int NST = 3;
  constexpr int NX = BM / 32, NW = BN / 32;         // 1 KB loads per wave per step: 8 + 4
  constexpr int L = NX + NW;
  constexpr int NF = SM + SN;                       // fragments per step: 12
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NST * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // Tile order: as the two-waves-per-SIMD kernel (consecutive tiles on one XCD, at most 4
  // row blocks of X before the next W panel).
  int b = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  constexpr int GM = 4;
  const int tiles_n = nb / tiles_m;
  const int grp_m = b / (GM * tiles_n);
  const int rows_g = min(tiles_m - grp_m * GM, GM);
  const int rb = b - grp_m * GM * tiles_n;
  const int tm = grp_m * GM + rb % rows_g, tn = rb / rows_g;
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Load q of a step: X rows 8 (wave + 4 q) .. +7 (q < NX), then W rows 8 (wave + 4 (q - NX));
  // lane l fetches chunk (l & 7) ^ swizzle of row 8 d + (l >> 3). Rows past M or N re-read
  // the last valid row (their results are never stored).
  uint32_t voff[L];
#pragma unroll
  for (int q = 0; q < L; ++q) {
    const bool isx = q < NX;
    const int d = wave + 4 * (isx ? q : q - NX);
    const int r = 8 * d + (lane >> 3);
    const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
    voff[q] = (uint32_t)row * (uint32_t)Kb + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  auto dma_one = [&](int ks, int stage, int q) {
    const bool isx = q < NX;
    const int d = wave + 4 * (isx ? q : q - NX);
    so_dma16(lds0 + stage * STAGE + (isx ? 0 : XT) + d * 1024, voff[q], (isx ? xq : wq) + (size_t)ks * 128);
  };

  const int fr = lane & 15, g = lane >> 4;
  const int fo0 = so_off(fr, g), fo1 = so_off(fr, g + 4);
  // Fragment f of a step: f < SM is X rows wm WR + 16 f, else W rows wn WC + 16 (f - SM).
  auto frag_base = [&](int stage, int f) -> const uint8_t* {
    return lds + stage * STAGE + (f < SM ? (wm * WR + 16 * f) * 128 : XT + (wn * WC + 16 * (f - SM)) * 128);
  };
  auto read_half = [&](sfrag_t (&F)[NF], int stage, int h) {   // h = 2 f + half
    const int f = h >> 1;
    const i32x4 v = *reinterpret_cast<const i32x4*>(frag_base(stage, f) + ((h & 1) ? fo1 : fo0));
    if (h & 1) { F[f][4] = v[0]; F[f][5] = v[1]; F[f][6] = v[2]; F[f][7] = v[3]; }
    else { F[f][0] = v[0]; F[f][1] = v[1]; F[f][2] = v[2]; F[f][3] = v[3]; }
  };

  typedef typename std::conditional<KIND == 1, i32x4, f32x4>::type acc_t;
  acc_t acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = acc_t{};
  sfrag_t F0[NF], F1[NF];

  // One K step: MFMAs on `cur` (step s), reads of step s + 1 into `nxt`, loads of step
  // s + 3. Every step reads and loads, so the MFMA sequence has no branches: past the last
  // step the loads re-fetch the last step (into a stage nobody reads again) and the reads
  // fill a register set nobody uses; the stage bookkeeping depends on s only.
  auto step = [&](int s, sfrag_t (&cur)[NF], sfrag_t (&nxt)[NF], auto st_c) {
    constexpr int STC = decltype(st_c)::value;          // s % 3
    constexpr int stn = (STC + 1) % NST, std_ = STC;
    const int kl = min(s + 3, ksteps - 1);
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      const int i = tt % SM, j = tt / SM;
      if constexpr (KIND == 1) {
        // INT8: the fragment's two 16-byte chunks are the two 64-deep halves of the step.
        const sfrag_t& a = cur[SM + j];
        const sfrag_t& b = cur[i];
        acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{a[0], a[1], a[2], a[3]}, i32x4{b[0], b[1], b[2], b[3]},
                                                         acc[j][i], 0, 0, 0);
        acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{a[4], a[5], a[6], a[7]}, i32x4{b[4], b[5], b[6], b[7]},
                                                         acc[j][i], 0, 0, 0);
      } else {
        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur[SM + j], cur[i], acc[j][i], 0, 0, 0, 0, 0, 0);
      }
      if (tt < 2 * NF) read_half(nxt, stn, tt);
      if ((tt & 1) && (tt >> 1) < L) dma_one(kl, std_, tt >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(so_wait(L, 0));          // step s + 2 landed; s + 3 may fly
    so_barrier();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;

  // Prologue: steps 0, 1, 2 into stages 0, 1, 2 (the last step again where K is shorter);
  // once 0 and 1 have landed everywhere, the fragments of step 0, then a barrier so that no
  // wave refills stage 0 before all have read it.
#pragma unroll
  for (int p = 0; p < 3; ++p)
#pragma unroll
    for (int q = 0; q < L; ++q) dma_one(min(p, ksteps - 1), p, q);
  __builtin_amdgcn_s_waitcnt(so_wait(L, 15));
  so_barrier();
#pragma unroll
  for (int h = 0; h < 2 * NF; ++h) read_half(F0, 0, h);
  __builtin_amdgcn_s_waitcnt(so_wait(63, 0));
  so_barrier();

  // Unrolled by six (two register sets x three stages) so that every address is fixed.
  int s = 0;
  for (; s + 5 < ksteps; s += 6) {
    step(s, F0, F1, S0{});
    step(s + 1, F1, F0, S1{});
    step(s + 2, F0, F1, S2{});
    step(s + 3, F1, F0, S0{});
    step(s + 4, F0, F1, S1{});
    step(s + 5, F1, F0, S2{});
  }
  // The remaining 0-5 steps; s % 6 == 0 here, so step s + r uses stage r % 3.
  if (s < ksteps) step(s, F0, F1, S0{});
  if (s + 1 < ksteps) step(s + 1, F1, F0, S1{});
  if (s + 2 < ksteps) step(s + 2, F0, F1, S2{});
  if (s + 3 < ksteps) step(s + 3, F1, F0, S0{});
  if (s + 4 < ksteps) step(s + 4, F0, F1, S1{});
  __builtin_amdgcn_s_waitcnt(so_wait(0, 0));            // the re-fetches past the end
  so_barrier();

  // ---- epilogue. Every load has landed and every wave is past its last fragment read.
  float esm[SM], esn[SN][4];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) esn[j][r] = sw[min(n0 + wn * WC + 16 * j + 4 * g + r, N - 1)];
#pragma unroll
  for (int i = 0; i < SM; ++i) esm[i] = sx[min(m0 + wm * WR + 16 * i + fr, M - 1)];
  const bool has_bias = ep.bias != nullptr;
  constexpr int ES = OF8 ? 1 : 2;                      // output bytes per element
  constexpr int RS = BN * ES + 16;                     // padded rows: conflict-free column writes
  static_assert(BM * RS <= NST * STAGE, "output tile must fit in the pipeline LDS");
  // In the 16x16 result (A = W fragment, B = X fragment), lane l holds output row
  // m = 16 i + (l & 15) and the four consecutive columns 16 j + 4 (l >> 4) + r.
  epi_dispatch(ep.act, has_bias, [&](auto act_c, auto bias_c) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool BIAS = decltype(bias_c)::value;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int rl = wm * WR + 16 * i + fr;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int cl = wn * WC + 16 * j + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (KIND == 1) v[r] = mul_rn(mul_rn((float)acc[j][i][r], esm[i]), esn[j][r]);
          else v[r] = acc[j][i][r] * (esm[i] * esn[j][r]);
          if constexpr (BIAS) v[r] = add_rn(v[r], bf16_lo(ep.bias[min(n0 + cl + r, N - 1)]));
          v[r] = epi_act<ACT>(v[r]);
        }
        if constexpr (OF8) {
          *reinterpret_cast<uint32_t*>(lds + rl * RS + cl) =
              pack_e4m3x4(epi_requant<KIND == 1>(v[0], ep.s_out, ep.inv_s_out), epi_requant<KIND == 1>(v[1], ep.s_out, ep.inv_s_out),
                          epi_requant<KIND == 1>(v[2], ep.s_out, ep.inv_s_out), epi_requant<KIND == 1>(v[3], ep.s_out, ep.inv_s_out));
        } else {
          const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(lds + rl * RS + cl * 2) = o;
        }
      }
    }
  });
  __builtin_amdgcn_s_waitcnt(so_wait(63, 0));
  so_barrier();
  constexpr int EPC = 16 / ES;                         // output elements per 16-byte chunk
  constexpr int CPR = BN / EPC;                        // chunks per output row
  constexpr int ITERS = BM * CPR / kSoloThreads;       // chunks per thread: all reads, then stores
  static_assert(ITERS * kSoloThreads == BM * CPR, "whole chunks per thread");
  u32x4 ov[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int c = t + it * kSoloThreads;
    const int rl = c / CPR, ch = c - rl * CPR;
    ov[it] = *reinterpret_cast<const u32x4*>(lds + rl * RS + ch * 16);
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int c = t + it * kSoloThreads;
    const int rl = c / CPR, ch = c - rl * CPR;
    const int m = m0 + rl, n = n0 + ch * EPC;
    if (m >= M || n >= N) continue;
    const u32x4 v = ov[it];
    uint8_t* yr = reinterpret_cast<uint8_t*>(yp) + ((size_t)m * N + n) * ES;
    if (vec_store && n + EPC - 1 < N) {
      *reinterpret_cast<u32x4*>(yr) = v;
    } else {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if (n + e >= N) break;
        if constexpr (OF8) yr[e] = (uint8_t)((w4[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        else reinterpret_cast<uint16_t*>(yr)[e] = (uint16_t)((w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_solo(const void* xq, const float* sx, const void* wq, const float* sw,
                            int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                            const Epilogue& ep) {
  const int tiles_m = (int)((M + kSoloBM - 1) / kSoloBM);
  const int tiles_n = (int)((N + kSoloBN - 1) / kSoloBN);
  const int vec = ep.out_fp8 ? (N % 16) == 0 : (N % 8) == 0;
  auto go = [&](auto kind_c, auto of8_c) {
    hipLaunchKernelGGL((gemm_solo_kernel<decltype(kind_c)::value, decltype(of8_c)::value>),
                       dim3((unsigned)(tiles_m * tiles_n)), dim3(kSoloThreads), 0, st, (const uint8_t*)xq, sx,
                       (const uint8_t*)wq, sw, (int)M, (int)N, (int)K, (int)(K / 128), y, tiles_m, vec, ep);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if (fmt == 1) {
    if (ep.out_fp8) go(I1{}, std::true_type{});
    else go(I1{}, std::false_type{});
  } else {
    if (ep.out_fp8) go(I0{}, std::true_type{});
    else go(I0{}, std::false_type{});
  }
  return hipGetLastError();
}

}  // namespace w8a8
