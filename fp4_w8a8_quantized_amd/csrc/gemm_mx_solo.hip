// MXFP4 x MXFP4 GEMM on gfx950 with one wave per SIMD and 256 x 256 tiles:
//   y = bf16( sum_b 2^(ex[m,b]-127) 2^(ew[n,b]-127) sum_{k in b} dec4(xq) dec4(wq) )
// for OCP MXFP4 operands (E2M1 elements, one E8M0 scale per 32 along K; "Low-bit LLM Weights
// and Activations" §2.4). The E8M0 scales go straight into the scale operands of
// v_mfma_scale_f32_32x32x64_f8f6f4.
//
// A 256-thread workgroup (4 waves, one per SIMD) computes a 256 x 256 tile; each wave owns
// 128 x 128 of it, 4 x 4 subtiles of 32 x 32 with their accumulators in AGPRs, i.e. 64 MFMAs
// per K step of 256 elements (128 bytes of codes per row) against 32 fragment reads. Per
// MFMA that is half the LDS bytes and half the L2 bytes of the two-waves-per-SIMD kernel's
// 256 x 128 tiles with 64 x 64 wave tiles.
//
// LDS: two stages of [X codes 256 x 128 B | W codes 256 x 128 B | X scales 256 x 8 B |
// W scales 256 x 8 B], 68 KB each, filled by direct-to-LDS loads (16-byte loads for the
// codes, 4-byte loads for the scales).
//
// The fragments are not double-buffered (the accumulators take all 256 AGPRs): the MFMAs
// of a step run in four quarters q = 0..3 (the 64-element slice q of every subtile), and
// the registers of quarter q are refilled with the next step's quarter q as soon as they
// are free. Per K step s (stage s % 2 holds step s):
//   quarter 0: MFMAs of q = 0; read step s's quarter 3 (its registers were freed by the
//     previous step's quarter 3); then wait for every outstanding load and fragment read
//     and one barrier: every wave is done with stage s % 2 and step s + 1 is complete in
//     stage (s + 1) % 2;
//   quarter 1: MFMAs of q = 1; read step s + 1's quarter 0 and scale words; issue the loads
//     of step s + 2 into stage s % 2;
//   quarters 2, 3: MFMAs; read step s + 1's quarters 1, 2.
// Every step loads (past the last step, re-fetches of the last step into a stage nobody
// reads again), so the MFMA sequence has no branches.
//
// Fragments: lane l reads row l & 31 and, for quarter q, the 16-byte chunk 2q + h
// (h = l >> 5), which holds the 32-element block whose scale byte the lane supplies. Rows sit
// 128 B apart with chunk c at slot c ^ ((row >> 1) & 7). Rows past M or N re-read the last
// valid row; their results are never stored.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int kMsBM = 256, kMsBN = 256, kMsThreads = 256;

__device__ __forceinline__ int ms_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Direct global->LDS loads of 16 and 4 bytes per lane (lane l writes LDS bytes
// [m0 + 16 l, +16) or [m0 + 4 l, +4)), with the wait state gfx9 asks for between an SALU
// write of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void ms_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}
__device__ __forceinline__ void ms_dma4(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate (gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int ms_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void ms_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef int ms_i32x8 __attribute__((ext_vector_type(8)));

__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
gemm_mx_solo_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ sx,
                    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ sw, int M, int N,
                    int Kb, int ksteps, uint16_t* __restrict__ y, int tiles_m, int vec_store) {
  constexpr int BM = kMsBM, BN = kMsBN;
  constexpr int WR = 128, WC = 128;                 // wave tile (2 x 2 waves)
  constexpr int SM = WR / 32, SN = WC / 32;         // 4 x 4 subtiles of 32 x 32
  constexpr int XT = BM * 128, WT = BN * 128, SXT = BM * 8, SWT = BN * 8;
  constexpr int STAGE = XT + WT + SXT + SWT;
  constexpr int NC = (BM + BN) / 32;                // 16-byte-per-lane code loads per wave per step
  constexpr int NS = (BM + BN) / 128;               // 4-byte-per-lane scale loads per wave per step
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // Tile order: consecutive tiles on one XCD, at most 4 row blocks of X before the next
  // W panel (as the other tiled kernels).
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
  const int S = ksteps * 8;                          // scale bytes per row
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Code load c (< NC): X rows 8 (wave + 4 c) .. +7 for c < NC / 2, else W rows
  // 8 (wave + 4 (c - NC / 2)); lane l fetches chunk (l & 7) ^ swizzle of row 8 d + (l >> 3).
  // Scale load e (< NS): X scale rows 32 (wave + 4 e) .. +31 for e < NS / 2, else W; lane l
  // fetches bytes 4 (l & 1) .. +3 of the step's 8 scale bytes of row 32 d + (l >> 1).
  uint32_t cvo[NC], svo[NS];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const bool isx = c < NC / 2;
    const int d = wave + 4 * (isx ? c : c - NC / 2);
    const int r = 8 * d + (lane >> 3);
    const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
    cvo[c] = (uint32_t)row * (uint32_t)Kb + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int e = 0; e < NS; ++e) {
    const bool isx = e < NS / 2;
    const int d = wave + 4 * (isx ? e : e - NS / 2);
    const int r = 32 * d + (lane >> 1);
    const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
    svo[e] = (uint32_t)row * (uint32_t)S + 4 * (lane & 1);
  }
  auto dma_code = [&](int ks, int stage, int c) {
    const bool isx = c < NC / 2;
    const int d = wave + 4 * (isx ? c : c - NC / 2);
    ms_dma16(lds0 + stage * STAGE + (isx ? 0 : XT) + d * 1024, cvo[c], (isx ? xq : wq) + (size_t)ks * 128);
  };
  auto dma_scale = [&](int ks, int stage, int e) {
    const bool isx = e < NS / 2;
    const int d = wave + 4 * (isx ? e : e - NS / 2);
    ms_dma4(lds0 + stage * STAGE + XT + WT + (isx ? 0 : SXT) + d * 256, svo[e], (isx ? sx : sw) + (size_t)ks * 8);
  };
  constexpr int NL = NC + NS;                        // loads per wave per step
  auto dma_one = [&](int ks, int stage, int u) {
    if (u < NC) dma_code(ks, stage, u);
    else dma_scale(ks, stage, u - NC);
  };

  const int fr = lane & 31, h = lane >> 5;
  int fo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) fo[q] = ms_off(fr, 2 * q + h);
  i32x4 xf[SM][4], wf[SN][4];                        // quarter q of each subtile row / column
  auto read_quarter = [&](int stage, int q, int part) {   // part 0: X, 1: W (4 reads each)
    const uint8_t* base = lds + stage * STAGE;
    if (part == 0) {
#pragma unroll
      for (int i = 0; i < SM; ++i) xf[i][q] = *reinterpret_cast<const i32x4*>(base + (wm * WR + 32 * i) * 128 + fo[q]);
    } else {
#pragma unroll
      for (int j = 0; j < SN; ++j) wf[j][q] = *reinterpret_cast<const i32x4*>(base + XT + (wn * WC + 32 * j) * 128 + fo[q]);
    }
  };
  // The step's 8 scale bytes of the lane's row in each subtile row (X) and column (W).
  auto read_scales = [&](int stage, u32x2 (&scx)[SM], u32x2 (&scw)[SN]) {
    const uint8_t* base = lds + stage * STAGE + XT + WT;
#pragma unroll
    for (int i = 0; i < SM; ++i) scx[i] = *reinterpret_cast<const u32x2*>(base + (wm * WR + 32 * i + fr) * 8);
#pragma unroll
    for (int j = 0; j < SN; ++j) scw[j] = *reinterpret_cast<const u32x2*>(base + SXT + (wn * WC + 32 * j + fr) * 8);
  };

  f32x16 acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = f32x16{};

  // The 16 MFMAs of quarter q, with `extra(u)` issued after MFMA u (reads and loads).
  auto quarter = [&](int q, const u32x2 (&scx)[SM], const u32x2 (&scw)[SN], auto&& extra) {
    const int blk = 2 * q + h;                       // the lane's 32-element block of the step
    int ex[SM], ew[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) ex[i] = (int)((((blk < 4) ? scx[i].x : scx[i].y) >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
    for (int j = 0; j < SN; ++j) ew[j] = (int)((((blk < 4) ? scw[j].x : scw[j].y) >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
    for (int u = 0; u < SM * SN; ++u) {
      const int i = u / SN, j = u % SN;
      const ms_i32x8 a = {wf[j][q][0], wf[j][q][1], wf[j][q][2], wf[j][q][3], 0, 0, 0, 0};
      const ms_i32x8 bb = {xf[i][q][0], xf[i][q][1], xf[i][q][2], xf[i][q][3], 0, 0, 0, 0};
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, acc[j][i], 4, 4, 0, ew[j], 0, ex[i]);
      extra(u);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One K step on scale words (cur), reading the next step's words into (nxt). P = s % 2.
  auto step = [&](int s, u32x2 (&cx)[SM], u32x2 (&cw)[SN], u32x2 (&nx)[SM], u32x2 (&nw)[SN], auto p_c) {
    constexpr int P = decltype(p_c)::value, Q = 1 - P;
    const int kl = min(s + 2, ksteps - 1);
    quarter(0, cx, cw, [&](int u) {                  // this step's quarter 3
      if (u == 2) read_quarter(P, 3, 0);
      if (u == 6) read_quarter(P, 3, 1);
    });
    __builtin_amdgcn_s_waitcnt(ms_wait(0, 0));
    ms_barrier();
    quarter(1, cx, cw, [&](int u) {                  // next step's quarter 0, scales, loads
      if (u == 0) read_quarter(Q, 0, 0);
      if (u == 2) read_quarter(Q, 0, 1);
      if (u == 4) read_scales(Q, nx, nw);
      if (u < 16) {                                  // NL = 20 loads over the 16 MFMAs
        dma_one(kl, P, u);
        if (u < NL - 16) dma_one(kl, P, 16 + u);
      }
    });
    quarter(2, cx, cw, [&](int u) {
      if (u == 0) read_quarter(Q, 1, 0);
      if (u == 4) read_quarter(Q, 1, 1);
    });
    quarter(3, cx, cw, [&](int u) {
      if (u == 0) read_quarter(Q, 2, 0);
      if (u == 4) read_quarter(Q, 2, 1);
    });
  };
  static_assert(NL >= 16 && NL <= 32, "loads are spread over the 16 MFMAs of quarter 1");

  // Prologue: steps 0 and 1 into stages 0 and 1; once step 0 has landed everywhere, its
  // quarters 0-2 and scale words.
  u32x2 scx0[SM], scw0[SN], scx1[SM], scw1[SN];
#pragma unroll
  for (int u = 0; u < NL; ++u) dma_one(0, 0, u);
#pragma unroll
  for (int u = 0; u < NL; ++u) dma_one(min(1, ksteps - 1), 1, u);
  __builtin_amdgcn_s_waitcnt(ms_wait(NL, 15));
  ms_barrier();
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    read_quarter(0, q, 0);
    read_quarter(0, q, 1);
  }
  read_scales(0, scx0, scw0);

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  int s = 0;
  for (; s + 1 < ksteps; s += 2) {
    step(s, scx0, scw0, scx1, scw1, P0{});
    step(s + 1, scx1, scw1, scx0, scw0, P1{});
  }
  if (s < ksteps) step(s, scx0, scw0, scx1, scw1, P0{});
  __builtin_amdgcn_s_waitcnt(ms_wait(0, 0));           // the re-fetches past the end
  ms_barrier();

  // ---- epilogue: bf16 tile staged through the freed LDS, whole 16-byte row chunks out.
  constexpr int RS = BN * 2 + 16;                      // padded rows
  static_assert(BM * RS <= 2 * STAGE, "output tile must fit in the pipeline LDS");
  // In the 32x32 result (A = W fragment, B = X fragment), lane l holds output row
  // m = 32 i + (l & 31) and the columns 32 j + 8 q + 4 (l >> 5) + r, q, r in 0..3.
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int rl = wm * WR + 32 * i + fr;
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = wn * WC + 32 * j + 8 * q + 4 * h;
        const f32x16 a = acc[j][i];
        const u32x2 o = {pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
        *reinterpret_cast<u32x2*>(lds + rl * RS + cl * 2) = o;
      }
  }
  __builtin_amdgcn_s_waitcnt(ms_wait(63, 0));
  ms_barrier();
  constexpr int CPR = BN / 8;                          // 16-byte chunks per output row
  constexpr int ITERS = BM * CPR / kMsThreads;         // 32, in two halves
  static_assert(ITERS % 2 == 0, "");
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 ov[ITERS / 2];
#pragma unroll
    for (int it = 0; it < ITERS / 2; ++it) {
      const int c = t + (half * ITERS / 2 + it) * kMsThreads;
      const int rl = c / CPR, ch = c - rl * CPR;
      ov[it] = *reinterpret_cast<const u32x4*>(lds + rl * RS + ch * 16);
    }
#pragma unroll
    for (int it = 0; it < ITERS / 2; ++it) {
      const int c = t + (half * ITERS / 2 + it) * kMsThreads;
      const int rl = c / CPR, ch = c - rl * CPR;
      const int m = m0 + rl, n = n0 + ch * 8;
      if (m >= M || n >= N) continue;
      uint16_t* yr = y + (size_t)m * N + n;
      if (vec_store && n + 7 < N) {
        *reinterpret_cast<u32x4*>(yr) = ov[it];
      } else {
        const uint32_t w4[4] = {ov[it].x, ov[it].y, ov[it].z, ov[it].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (n + e >= N) break;
          yr[e] = (uint16_t)((w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mx_solo(const void* xq, const uint8_t* sx, const void* wq, const uint8_t* sw,
                               int64_t M, int64_t N, int64_t K, void* y, hipStream_t st) {
  const int tiles_m = (int)((M + kMsBM - 1) / kMsBM);
  const int tiles_n = (int)((N + kMsBN - 1) / kMsBN);
  hipLaunchKernelGGL(gemm_mx_solo_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kMsThreads), 0, st,
                     (const uint8_t*)xq, sx, (const uint8_t*)wq, sw, (int)M, (int)N, (int)(K / 2),
                     (int)(K / 256), (uint16_t*)y, tiles_m, (int)((N % 8) == 0));
  return hipGetLastError();
}

}  // namespace w8a8
