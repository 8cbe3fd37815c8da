// W8A8 GEMM on gfx950 with two waves per SIMD taking turns ("ping-pong"):
//   FP8   y = epilogue( s_x[m] s_w[n] sum_k dec(xq[m,k]) dec(wq[n,k]) )   (v_mfma 16x16x128 f8f6f4)
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x[m]) s_w[n] ),  acc_i32 = sum_k xq wq
//         (two v_mfma_i32_16x16x64_i8 per subtile and step on the same 32-byte fragments;
//         SmoothQuant W8A8, each product of the dequantization rounded on its own, in that
//         order, so that outputs are exact functions of the codes)
// with the scale factoring of "FP8 and FP4 inference, SmoothQuant and activation
// quantization" (Scale granularity) and the epilogue of "FP8 and INT8 Inference" §6-9.
//
// Why two waves per SIMD. A wave issues in order: with one wave per SIMD, every LDS read
// and every direct-to-LDS load it issues sits between two MFMAs, and the CU's address
// unit (about 64 B per clock) and LDS latency hold back the matrix core. Here a 512-thread
// workgroup (8 waves, 2 per SIMD) computes a 256 x BN tile, BN in {128, 192, 224}; each
// wave owns 128 x 48 of it at BN = 192, else 64 x BN/2. Waves 0-3 (group A) and 4-7
// (group B) alternate between two
// phases separated by workgroup barriers:
//   LDS phase:  read this step's X and W fragments into registers
//   MFMA phase: SM x SN MFMAs on them
// so that while one wave of a SIMD issues memory instructions the other keeps the matrix
// core busy. Slot 2k: A reads step k, B computes step k-1; slot 2k+1: A computes step k,
// B reads step k.
//
// LDS: two stages of [256 x 128 B of X | BN x 128 B of W]. Group B reads a stage last,
// so group B refills it, but only once all four B waves are done reading it: the odd slot
// has a barrier in its middle (group A splits its MFMA phase around it). After that barrier
// each B wave issues half of its loads of step k+2 into the stage, waits for its loads of
// step k+1 (so the barrier that ends the slot publishes them to A), and issues the other
// half between the MFMAs of its next phase. The stage is next read by A two slots later.
// The last two steps load nothing and wait for all outstanding loads instead.
//
// Fragments: lane l reads row l & 15 and the 16-byte chunks g and g + 4 (g = l >> 4) of the
// 128-byte K step; both operands permute K the same way, so every dot product still covers
// the whole step. This assignment keeps the 8-wave fragment reads free of bank conflicts
// (about twice the throughput of chunks 2g, 2g + 1 on gfx950's LDS). Rows sit 128 B apart
// with chunk c at slot c ^ ((row >> 1) & 7).
//
// Epilogue: scale, bias, activation, convert (bf16, or E4M3FN of clamp(v / s_out)) in
// registers, stage the tile through the freed LDS, write whole rows with 16-byte stores.
//
// Block-scaled form (BLK; the DeepSeek-V3 recipe of "FP8 and INT8 Inference" §5: 1 x 128
// activation groups, 128 x 128 weight blocks, FP32 accumulation promoted at intervals):
//   y = bf16( sum_g s_x[m,g] s_w[n/128,g] sum_{k in g} dec(xq[m,k]) dec(wq[n,k]) )
// A K step is one 128-wide group, and each 16 x 16 subtile takes exactly one MFMA per step,
// so the MFMA (with a zero accumulator) yields the group's fp32 partial, which is promoted
// into the running sum with one FMA per element, times s_x[m,g] s_w[n/128,g]. The
// promotion of a subtile runs four MFMAs behind its product (the last four of a step
// during the next LDS phase), so it never waits on the matrix core. Group A, which issues
// no direct-to-LDS loads and may therefore use ordinary loads, fetches the 256 rows' s_x
// and the tile's s_w two steps ahead and publishes their products to a double-buffered
// 1 KB LDS area, laid out so that each lane reads its four rows with one 16-byte read.
// Tiles are 128 wide, one weight block, so every column of a tile shares s_w.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int kPPBM = 256;
constexpr int kPPThreads = 512;

__device__ __forceinline__ int pp_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// One 16-byte direct global->LDS load per lane (lane l writes LDS bytes [m0 + 16 l, +16)).
// M0 is written by the same inline assembly, with the one wait state gfx9 asks for
// between an SALU write of M0 and an LDS-DMA that reads it.
__device__ __forceinline__ void pp_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate (gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int pp_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void pp_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int KIND, int BN, bool OF8, bool BLK>
__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
gemm_pp_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
               const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
               int Kb, int ksteps, void* __restrict__ yp, int tiles_m, int vec_store, Epilogue ep) {
  constexpr int BM = kPPBM;
  static_assert(!BLK || (BN == 128 && !OF8 && KIND == 0), "block scales: FP8, 128-wide tiles (one weight block), bf16 out");
  typedef typename std::conditional<KIND == 1, i32x4, f32x4>::type acc_t;
  // Wave tiles: 128 x 48 at BN = 192 (2 x 4 waves); 64 x BN/2 otherwise (4 x 2 waves): at
  // BN = 128 that reads 8 fragments per step instead of 10 for the same 64 accumulators, and
  // at BN = 224 (64 x 112) 11 fragments for 28 MFMAs.
  constexpr int WAVES_M = (BN == 192) ? 2 : 4;
  constexpr int WR = BM / WAVES_M;            // rows per wave
  constexpr int SM = WR / 16;                 // 16-row subtiles
  constexpr int WC = BN * WAVES_M / 8;        // columns per wave
  constexpr int SN = WC / 16;
  static_assert(SN * 16 * (8 / WAVES_M) == BN, "tile width must give whole 16-column subtiles per wave");
  constexpr int XT = BM * 128, WT = BN * 128, STAGE = XT + WT;
  constexpr int XI = BM / 32, WI = BN / 32;   // 1 KB loads per group-B wave per step
  constexpr int DMA = XI + WI;
  constexpr int DC = DMA / 2;                 // of which issued during the MFMA phase
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];
  // Block scales s_x[m,g] s_w[n/128,g] of two steps (buffer g & 1): row r of the tile sits at
  // (r & ~63) + 4 (r & 15) + ((r >> 4) & 3), so lane l of a wave reads rows 16 i + (l & 15)
  // of its 64-row wave tile (i = 0..3) as one float4.
  __shared__ __attribute__((aligned(16))) float sxl[BLK ? 2 * BM : 4];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2, g4 = wave & 3;
  const int wm = WAVES_M == 4 ? g4 : (g4 & 1);
  const int wn = WAVES_M == 4 ? grp : grp * 2 + (g4 >> 1);
  // Workgroup ids are dealt round-robin over the 8 XCDs; remap so that consecutive tiles
  // run on one XCD and its L2. Consecutive tiles walk at most 4 row blocks of X, then the
  // next W panel, so that the 32 tiles an XCD holds at once share 4 X blocks and 8 W
  // panels (about 10 MB at K = 4096) rather than, in column-major order, all row blocks of
  // X and a few panels (33 MB at 8192 tokens).
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

  // Load d of a step (group B): d < XI fills X rows 8 (g4 + 4 d) .. +7, else W rows; lane l
  // fetches chunk (l & 7) ^ swizzle of row 8q + (l >> 3) into its slot. Rows past M or N
  // re-read the last valid row (their results are never stored).
  auto dma_one = [&](int ks, int stage, int d) {
    const uint32_t sbase = lds0 + stage * STAGE + g4 * 1024;
    const bool isx = d < XI;
    const int i = isx ? d : d - XI;
    const int r = 8 * (g4 + 4 * i) + (lane >> 3);
    const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
    const uint32_t vo = (uint32_t)row * (uint32_t)Kb + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    pp_dma16(sbase + (isx ? 0 : XT) + i * 4096, vo, (isx ? xq : wq) + (size_t)ks * 128);
  };

  const int fr = lane & 15, g = lane >> 4;
  const int fo0 = pp_off(fr, g), fo1 = pp_off(fr, g + 4);
  const int xrow0 = wm * WR, wrow0 = wn * WC;
  typedef int frag_t __attribute__((ext_vector_type(8)));
  auto frag = [&](const uint8_t* base) -> frag_t {
    const i32x4 a = *reinterpret_cast<const i32x4*>(base + fo0);
    const i32x4 c = *reinterpret_cast<const i32x4*>(base + fo1);
    return frag_t{a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
  };

  acc_t acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = acc_t{};
  frag_t xf[SM], wf[SN];

  constexpr int T = SM * SN;
  // Block-scaled state: the last PD group partials (ring indexed by subtile number) and the
  // scales of the step they belong to. Zero at the start, so that the first step's
  // promotion of "the previous step's tail" adds 0 * 0.
  constexpr int PD = 4;
  f32x4 pp[BLK ? PD : 1];
  float bscl[BLK ? SM : 1];
  if constexpr (BLK) {
#pragma unroll
    for (int p = 0; p < PD; ++p) pp[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < SM; ++i) bscl[i] = 0.f;
  }
  auto promote = [&](int tt) {                         // subtile tt's partial into its sum
    if constexpr (BLK) {
      const int ti = tt / SN, tj = tt % SN;
      acc[tj][ti] += pp[tt % PD] * bscl[ti];
    }
  };

  auto lds_phase = [&](int ks) {
    const uint8_t* X = lds + (ks & 1) * STAGE;
    const uint8_t* W = X + XT;
#pragma unroll
    for (int i = 0; i < SM; ++i) xf[i] = frag(X + (xrow0 + 16 * i) * 128);
#pragma unroll
    for (int j = 0; j < SN; ++j) wf[j] = frag(W + (wrow0 + 16 * j) * 128);
    if constexpr (BLK) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(sxl + (ks & 1) * BM + xrow0 + 4 * fr);
      // The previous step's last PD promotions, while the reads are in flight.
#pragma unroll
      for (int tt = T - PD; tt < T; ++tt) promote(tt);
      __builtin_amdgcn_s_waitcnt(pp_wait(63, 0));
#pragma unroll
      for (int i = 0; i < SM; ++i) bscl[i] = s4[i];
    } else {
      __builtin_amdgcn_s_waitcnt(pp_wait(63, 0));    // this wave's reads of the stage done
    }
  };
  // MFMA number tt of a step (row-major over the SM x SN subtiles). Block-scaled: the
  // product goes to the partial ring, after the promotion of the partial PD MFMAs back,
  // which held the same ring slot.
  auto mfma_one = [&](int tt) {
    const int i = tt / SN, j = tt % SN;
    if constexpr (BLK) {
      if (tt >= PD) promote(tt - PD);
      pp[tt % PD] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
    } else if constexpr (KIND == 1) {
      // INT8: the fragment's two 16-byte chunks are the two 64-deep halves of the step.
      acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{wf[j][0], wf[j][1], wf[j][2], wf[j][3]},
                                                       i32x4{xf[i][0], xf[i][1], xf[i][2], xf[i][3]}, acc[j][i], 0, 0, 0);
      acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{wf[j][4], wf[j][5], wf[j][6], wf[j][7]},
                                                       i32x4{xf[i][4], xf[i][5], xf[i][6], xf[i][7]}, acc[j][i], 0, 0, 0);
    } else {
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[j], xf[i], acc[j][i], 0, 0, 0, 0, 0, 0);
    }
  };
  // MFMAs number lo .. hi-1 of a step.
  auto mfma_range = [&](int lo, int hi) {
#pragma unroll
    for (int tt = lo; tt < hi; ++tt) {
      mfma_one(tt);
      if constexpr (BLK) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Group B's MFMA phase, with the last DC loads of step kd between the MFMAs.
  auto mfma_phase_loading = [&](int kd, int stage) {
#pragma unroll
    for (int tt = 0; tt < T; ++tt) {
      mfma_one(tt);
#pragma unroll
      for (int d = 0; d < DC; ++d)
        if (tt == (d * T) / DC) dma_one(kd, stage, DMA - DC + d);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Block scales: group A thread t (< 256) fetches row m0 + t's s_x and the tile's s_w two
  // steps ahead and publishes their product for the next step (ks + 1) during step ks.
  const int srow = min(m0 + (t & (BM - 1)), M - 1);
  const int spos = (t & (BM - 1) & ~63) + 4 * (t & 15) + ((t >> 4) & 3);
  const float* sxr = sx + (size_t)srow * ksteps;
  const float* swr = sw + (size_t)tn * ksteps;
  float sx_next = 0.f, sw_next = 0.f;
  auto publish = [&](int ks) {                         // group A: scales of step ks + 1
    if constexpr (BLK) {
      sxl[((ks + 1) & 1) * BM + spos] = sx_next * sw_next;
      const int k2 = min(ks + 2, ksteps - 1);
      sx_next = sxr[k2];
      sw_next = swr[k2];
    }
  };

  // The epilogue's scales are loaded up front, so that their latency hides behind the K
  // loop, except the column scales of the 224-wide tile, whose registers it cannot spare
  // during the loop (the bias is read in the epilogue).
  constexpr bool LATE_SN = (BN == 224);
  float esm[SM], esn[SN][4];
  const bool has_bias = !BLK && ep.bias != nullptr;
  auto load_esn = [&]() {
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) esn[j][r] = sw[min(n0 + wrow0 + 16 * j + 4 * g + r, N - 1)];
  };
  if constexpr (!BLK) {
    if constexpr (!LATE_SN) load_esn();
#pragma unroll
    for (int i = 0; i < SM; ++i) esm[i] = sx[min(m0 + xrow0 + 16 * i + fr, M - 1)];
  } else if (grp == 0) {
    // Scales of step 0 published before the first barrier; step 1's in registers.
    sxl[spos] = sxr[0] * swr[0];
    sx_next = sxr[min(1, ksteps - 1)];
    sw_next = swr[min(1, ksteps - 1)];
    __builtin_amdgcn_s_waitcnt(pp_wait(63, 0));
  }
  // Prologue: group B loads steps 0 and 1; step 0 landed and published. Past the last
  // step, loads re-fetch the last step into a stage nobody reads again (branch-free).
  if (grp == 1) {
#pragma unroll
    for (int d = 0; d < DMA; ++d) dma_one(0, 0, d);
#pragma unroll
    for (int d = 0; d < DMA; ++d) dma_one(min(1, ksteps - 1), 1, d);
    __builtin_amdgcn_s_waitcnt(pp_wait(DMA, 15));
  }
  pp_barrier();
  // Both groups pass 3 * ksteps + 1 barriers in the loop part.
  if (grp == 0) {
    for (int ks = 0; ks < ksteps; ++ks) {
      publish(ks);
      lds_phase(ks);                                   // slot 2k
      __builtin_amdgcn_sched_barrier(0);
      pp_barrier();
      mfma_range(0, T / 2);                            // slot 2k+1, first half
      __builtin_amdgcn_sched_barrier(0);
      pp_barrier();
      mfma_range(T / 2, T);                            // second half
      __builtin_amdgcn_sched_barrier(0);
      pp_barrier();
    }
    pp_barrier();
  } else {
    // Group B. The last two steps have nothing left to load: they wait for everything
    // outstanding instead (no re-fetch of the last step into a stage nobody reads).
    auto iter = [&](int ks, auto load_c) {
      constexpr bool LOAD = decltype(load_c)::value;
      lds_phase(ks);                                   // slot 2k+1, first half
      __builtin_amdgcn_sched_barrier(0);
      pp_barrier();                                    // no wave reads stage ks & 1 any more
      if constexpr (LOAD) {
#pragma unroll
        for (int d = 0; d < DMA - DC; ++d) dma_one(ks + 2, ks & 1, d);
        // Everything older than this slot's loads has landed: that is all of step k+1.
        __builtin_amdgcn_s_waitcnt(pp_wait(DMA - DC, 15));
      } else {
        __builtin_amdgcn_s_waitcnt(pp_wait(0, 15));
      }
      __builtin_amdgcn_sched_barrier(0);
      pp_barrier();
      if constexpr (LOAD) mfma_phase_loading(ks + 2, ks & 1);   // slot 2k+2
      else mfma_range(0, T);
      __builtin_amdgcn_sched_barrier(0);
      pp_barrier();
    };
    pp_barrier();                                      // slot 0
    int ks = 0;
    for (; ks + 2 < ksteps; ++ks) iter(ks, std::true_type{});
    for (; ks < ksteps; ++ks) iter(ks, std::false_type{});
  }

  if constexpr (BLK) {
#pragma unroll
    for (int tt = T - PD; tt < T; ++tt) promote(tt);   // the last step's tail
  }
  if constexpr (!BLK && LATE_SN) load_esn();

  // ---- epilogue. Every load has landed and every wave is past its last fragment read.
  constexpr int ES = OF8 ? 1 : 2;                      // output bytes per element
  constexpr bool SWZ = (BN == 256 && !OF8);
  constexpr int RS = SWZ ? 512 : BN * ES + 16;         // padded rows: conflict-free column writes
  static_assert(BM * RS <= 2 * STAGE, "output tile must fit in the pipeline LDS");
  auto opos = [&](int row, int byte) -> int {
    return SWZ ? row * RS + ((((byte >> 4) ^ (row & 15)) << 4) | (byte & 15)) : row * RS + byte;
  };
  __builtin_amdgcn_s_waitcnt(pp_wait(0, 0));
  pp_barrier();
  // In the 16x16 result (A = W fragment, B = X fragment), lane l holds output row
  // m = 16 i + (l & 15) and the four consecutive columns 16 j + 4 (l >> 4) + r.
  epi_dispatch(ep.act, has_bias, [&](auto act_c, auto bias_c) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool BIAS = decltype(bias_c)::value;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int rl = xrow0 + 16 * i + fr;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int cl = wrow0 + 16 * j + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (KIND == 1) v[r] = mul_rn(mul_rn((float)acc[j][i][r], esm[i]), esn[j][r]);
          else v[r] = BLK ? acc[j][i][r] : acc[j][i][r] * (esm[i] * esn[j][r]);
          if constexpr (BIAS) v[r] = add_rn(v[r], bf16_lo(ep.bias[min(n0 + cl + r, N - 1)]));
          v[r] = epi_act<ACT>(v[r]);
        }
        if constexpr (OF8) {
          *reinterpret_cast<uint32_t*>(lds + opos(rl, cl)) =
              pack_e4m3x4(epi_requant<KIND == 1>(v[0], ep.s_out, ep.inv_s_out), epi_requant<KIND == 1>(v[1], ep.s_out, ep.inv_s_out),
                          epi_requant<KIND == 1>(v[2], ep.s_out, ep.inv_s_out), epi_requant<KIND == 1>(v[3], ep.s_out, ep.inv_s_out));
        } else {
          const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(lds + opos(rl, cl * 2)) = o;
        }
      }
    }
  });
  __builtin_amdgcn_s_waitcnt(pp_wait(63, 0));
  pp_barrier();
  constexpr int EPC = 16 / ES;                         // output elements per 16-byte chunk
  constexpr int CPR = BN / EPC;                        // chunks per output row
  // Every thread moves ITERS chunks: all LDS reads first, then all global stores.
  constexpr int ITERS = BM * CPR / kPPThreads;
  static_assert(ITERS * kPPThreads == BM * CPR, "whole chunks per thread");
  u32x4 ov[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int c = t + it * kPPThreads;
    const int rl = c / CPR, ch = c - rl * CPR;
    ov[it] = *reinterpret_cast<const u32x4*>(lds + opos(rl, ch * 16));
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int c = t + it * kPPThreads;
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

template <int KIND, int BN, bool OF8, bool BLK = false>
hipError_t launch_pp(const void* xq, const float* sx, const void* wq, const float* sw, int64_t M,
                     int64_t N, int64_t K, void* y, hipStream_t st, const Epilogue& ep) {
  const int tiles_m = (int)((M + kPPBM - 1) / kPPBM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int vec = OF8 ? (N % 16) == 0 : (N % 8) == 0;
  hipLaunchKernelGGL((gemm_pp_kernel<KIND, BN, OF8, BLK>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kPPThreads), 0, st, (const uint8_t*)xq, sx, (const uint8_t*)wq, sw,
                     (int)M, (int)N, (int)K, (int)(K / 128), y, tiles_m, vec, ep);
  return hipGetLastError();
}

}  // namespace

// Tile width: the one whose waves of workgroups over the 256 CUs cost least, weighting
// each width by its measured steady-state MFMA efficiency (0.83 at 224, 0.80 at 192, 0.66
// at 128 on MI355X: a wider tile spends a smaller share of each step on loads, fragment
// reads and barriers). 224 wins where it removes a partial wave, as for 2048 x 28672
// (1024 tiles, four full waves, against 1200 tiles of 192).
hipError_t launch_gemm_pp(const void* xq, const float* sx, const void* wq, const float* sw,
                          int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                          const Epilogue& ep) {
  const int64_t tm = (M + kPPBM - 1) / kPPBM;
  auto cost = [&](int64_t bn, int64_t per_tile) { return ((tm * ((N + bn - 1) / bn) + 255) / 256) * per_tile; };
  const int64_t c224 = cost(224, 270), c192 = cost(192, 240), c128 = cost(128, 194);
  const int bn = (c224 < c192 && c224 < c128) ? 224 : (c192 <= c128 ? 192 : 128);
  // 128-wide tiles in up to two rounds over the CUs: the one-wave-per-SIMD kernel, which
  // reads a quarter fewer fragment bytes per MFMA (2048 x 4096 x 4096: 34.7 -> 32.6 us;
  // 2048 x 4096 x 14336: 102.5 -> 93.4 us; 4096 x 4096 x 4096: 64.7 -> 62.1 us). At four
  // rounds (8192 x 4096 x 14336) it measured 3% slower.
  if (bn == 128 && tm * ((N + 127) / 128) <= 512)
    return launch_gemm_solo(xq, sx, wq, sw, M, N, K, fmt, y, st, ep);
  auto go = [&](auto kind_c) {
    constexpr int KD = decltype(kind_c)::value;
    if (ep.out_fp8) {
      if (bn == 224) return launch_pp<KD, 224, true>(xq, sx, wq, sw, M, N, K, y, st, ep);
      return bn == 192 ? launch_pp<KD, 192, true>(xq, sx, wq, sw, M, N, K, y, st, ep)
                       : launch_pp<KD, 128, true>(xq, sx, wq, sw, M, N, K, y, st, ep);
    }
    if (bn == 224) return launch_pp<KD, 224, false>(xq, sx, wq, sw, M, N, K, y, st, ep);
    return bn == 192 ? launch_pp<KD, 192, false>(xq, sx, wq, sw, M, N, K, y, st, ep)
                     : launch_pp<KD, 128, false>(xq, sx, wq, sw, M, N, K, y, st, ep);
  };
  return fmt == 1 ? go(std::integral_constant<int, 1>{}) : go(std::integral_constant<int, 0>{});
}

// Block-scaled FP8 (s_x [M, K/128], s_w [ceil(N/128), K/128]): 256 x 128 tiles, bf16 out.
hipError_t launch_gemm_blockscaled(const void* xq, const float* sx, const void* wq,
                                   const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                   hipStream_t st) {
  return launch_pp<0, 128, false, true>(xq, sx, wq, sw, M, N, K, y, st, Epilogue{});
}

}  // namespace w8a8
