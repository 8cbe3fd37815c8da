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
// LDS: two code stages of [X codes 256 x 128 B | W codes 256 x 128 B] (64 KB each), filled
// by 16-byte direct-to-LDS loads, and the E8M0 scales. With one wave per SIMD a wave whose
// load cannot issue cannot issue its MFMAs either, and the cost of a load grows with the
// cache lines it touches: a 4-byte-per-lane scale load touches 32 rows' lines for 256 bytes,
// as many lines as four code loads. So when K is a multiple of 512 (SC2) the scales of two
// steps are fetched at once, 16 bytes per row and lane, into two scale stages of
// [X 256 x 16 B | W 256 x 16 B]: four times fewer scale loads (measured: 4300 -> 3000 cycles
// per K step at 8192^3 together with the spread code loads below). Otherwise the step's 8
// scale bytes per row ride in the code stage, two lanes per row.
//
// The fragments are not double-buffered (the accumulators take all 256 AGPRs): the MFMAs
// of a step run in four quarters q = 0..3 (the 64-element slice q of every subtile), and
// the registers of quarter q are refilled with the next step's quarter q as soon as they
// are free. Per K step s (code stage s % 2 holds step s):
//   quarter 0: MFMAs of q = 0; read step s's quarter 3 (its registers were freed by the
//     previous step's quarter 3); then wait for every outstanding load and fragment read
//     and one barrier: every wave is done with code stage s % 2 and step s + 1 is complete;
//   quarter 1: MFMAs of q = 1; read step s + 1's quarter 0 and scale words; the scale
//     loads (SC2: of steps s + 2 and s + 3, in even steps);
//   quarters 1 and 2: the 16 code loads of step s + 2 into code stage s % 2, one after
//     every other MFMA;
//   quarters 2, 3: read step s + 1's quarters 1, 2.
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

template <bool SC2>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
gemm_mx_solo_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ sx,
                    const uint8_t* __restrict__ wq, const uint8_t* __restrict__ sw, int M, int N,
                    int Kb, int ksteps, uint16_t* __restrict__ y, int tiles_m, int vec_store) {
  constexpr int BM = kMsBM, BN = kMsBN;
  constexpr int WR = 128, WC = 128;                 // wave tile (2 x 2 waves)
  constexpr int SM = WR / 32, SN = WC / 32;         // 4 x 4 subtiles of 32 x 32
  constexpr int XT = BM * 128, WT = BN * 128;
  // Per-step scales in the code stage (8 bytes per row), or SC2 scale stages of two steps.
  constexpr int SXT = SC2 ? 0 : BM * 8, SWT = SC2 ? 0 : BN * 8;
  constexpr int STAGE = XT + WT + SXT + SWT;
  constexpr int SC_BASE = 2 * STAGE, SC_STAGE = (BM + BN) * 16;
  constexpr int NC = (BM + BN) / 32;                // 16-byte-per-lane code loads per wave per step
  constexpr int NS = SC2 ? 2 : (BM + BN) / 128;     // scale loads per wave per (even, SC2) step
  static_assert(NC == 16 && NS <= 4, "loads per step assume 256 x 256 tiles");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SC2 ? SC_BASE + 2 * SC_STAGE : 2 * STAGE];

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
  // Scale load e (< NS), SC2: e = 0 X, 1 W rows 64 wave + l, 16 bytes (steps 2j and 2j + 1)
  // per lane; otherwise: X scale rows 32 (wave + 4 e) .. +31 for e < NS / 2, else W; lane l
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
    if constexpr (SC2) {
      const int r = 64 * wave + lane;
      const int row = e == 0 ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
      svo[e] = (uint32_t)row * (uint32_t)S;
    } else {
      const bool isx = e < NS / 2;
      const int d = wave + 4 * (isx ? e : e - NS / 2);
      const int r = 32 * d + (lane >> 1);
      const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
      svo[e] = (uint32_t)row * (uint32_t)S + 4 * (lane & 1);
    }
  }
  auto dma_code = [&](int ks, int stage, int c) {
    const bool isx = c < NC / 2;
    const int d = wave + 4 * (isx ? c : c - NC / 2);
    ms_dma16(lds0 + stage * STAGE + (isx ? 0 : XT) + d * 1024, cvo[c], (isx ? xq : wq) + (size_t)ks * 128);
  };
  // Scale load e of step ks into code stage `stage`; SC2: of steps ks and ks + 1 (ks even)
  // into scale stage `stage`.
  auto dma_scale = [&](int ks, int stage, int e) {
    if constexpr (SC2) {
      ms_dma16(lds0 + SC_BASE + stage * SC_STAGE + e * (BM * 16) + wave * 1024, svo[e],
               (e == 0 ? sx : sw) + (size_t)ks * 8);
    } else {
      const bool isx = e < NS / 2;
      const int d = wave + 4 * (isx ? e : e - NS / 2);
      ms_dma4(lds0 + stage * STAGE + XT + WT + (isx ? 0 : SXT) + d * 256, svo[e], (isx ? sx : sw) + (size_t)ks * 8);
    }
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
  // The 8 scale bytes of step ks for the lane's row in each subtile row (X) and column (W).
  auto read_scales = [&](int ks, int stage, u32x2 (&scx)[SM], u32x2 (&scw)[SN]) {
    const uint8_t* bx;
    int rs;
    if constexpr (SC2) {
      bx = lds + SC_BASE + ((ks >> 1) & 1) * SC_STAGE + (ks & 1) * 8;
      rs = 16;
    } else {
      bx = lds + stage * STAGE + XT + WT;
      rs = 8;
    }
    const uint8_t* bw = bx + (SC2 ? BM * 16 : SXT);
#pragma unroll
    for (int i = 0; i < SM; ++i) scx[i] = *reinterpret_cast<const u32x2*>(bx + (wm * WR + 32 * i + fr) * rs);
#pragma unroll
    for (int j = 0; j < SN; ++j) scw[j] = *reinterpret_cast<const u32x2*>(bw + (wn * WC + 32 * j + fr) * rs);
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
      if (u == 4) read_scales(s + 1, Q, nx, nw);
      if (!(u & 1)) dma_code(kl, P, u >> 1);
      if constexpr (SC2) {                           // even steps: steps s + 2, s + 3 (clamped)
        if (P == 0 && (u & 1) && (u >> 1) < NS) dma_scale(min(s + 2, ksteps - 2), ((s + 2) >> 1) & 1, u >> 1);
      } else {
        if ((u & 1) && (u >> 1) < NS) dma_scale(kl, P, u >> 1);
      }
    });
    quarter(2, cx, cw, [&](int u) {
      if (u == 0) read_quarter(Q, 1, 0);
      if (u == 4) read_quarter(Q, 1, 1);
      if (!(u & 1)) dma_code(kl, P, 8 + (u >> 1));
    });
    quarter(3, cx, cw, [&](int u) {
      if (u == 0) read_quarter(Q, 2, 0);
      if (u == 4) read_quarter(Q, 2, 1);
    });
  };

  // Prologue: steps 0 and 1 into stages 0 and 1 (and the scales of step 0, SC2: of steps
  // 0 and 1); once step 0 has landed everywhere, its quarters 0-2 and scale words.
  u32x2 scx0[SM], scw0[SN], scx1[SM], scw1[SN];
#pragma unroll
  for (int c = 0; c < NC; ++c) dma_code(0, 0, c);
#pragma unroll
  for (int e = 0; e < NS; ++e) dma_scale(0, 0, e);
#pragma unroll
  for (int c = 0; c < NC; ++c) dma_code(min(1, ksteps - 1), 1, c);
  if constexpr (!SC2) {
#pragma unroll
    for (int e = 0; e < NS; ++e) dma_scale(min(1, ksteps - 1), 1, e);
    __builtin_amdgcn_s_waitcnt(ms_wait(NC + NS, 15));
  } else {
    __builtin_amdgcn_s_waitcnt(ms_wait(NC, 15));
  }
  ms_barrier();
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    read_quarter(0, q, 0);
    read_quarter(0, q, 1);
  }
  read_scales(0, 0, scx0, scw0);

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
  static_assert(BM * RS <= (int)sizeof(lds), "output tile must fit in the pipeline LDS");
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
  // Paired scale loads need 16-byte aligned rows of scales: K / 32 a multiple of 16.
  auto kern = (K % 512 == 0) ? gemm_mx_solo_kernel<true> : gemm_mx_solo_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles_m * tiles_n)), dim3(kMsThreads), 0, st,
                     (const uint8_t*)xq, sx, (const uint8_t*)wq, sw, (int)M, (int)N, (int)(K / 2),
                     (int)(K / 256), (uint16_t*)y, tiles_m, (int)((N % 8) == 0));
  return hipGetLastError();
}

}  // namespace w8a8
