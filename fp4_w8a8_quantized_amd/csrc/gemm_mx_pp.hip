// MXFP4 x MXFP4 GEMM on gfx950 with two waves per SIMD taking turns ("ping-pong"), on
// 32 x 32 MFMAs whose operands are 16 bytes per lane:
//   y = bf16( sum_b 2^(ex[m,b]-127) 2^(ew[n,b]-127) sum_{k in b} dec4(xq) dec4(wq) )
// for OCP MXFP4 operands (E2M1 elements, one E8M0 scale per 32 along K; "Low-bit LLM
// Weights and Activations" §2.4). The E8M0 scales go straight into the scale operands of
// v_mfma_scale_f32_32x32x64_f8f6f4, so scaling costs no vector work. It takes the shapes
// whose 256 x 256 tiles would not fill a round of the CUs (the one-wave-per-SIMD kernel,
// gemm_mx_solo.hip, takes the rest).
//
// Schedule: as the FP8 ping-pong kernel. A 512-thread workgroup computes a 256 x 128 tile;
// waves 0-3 (group A) and 4-7 (group B) alternate an LDS phase (fragments and scales of a
// K step into registers) and an MFMA phase; each wave owns a 64 x 64 block of 2 x 2
// subtiles of 32 x 32, with four 64-deep MFMAs per subtile per K step of 256 elements
// (128 bytes of codes per row). Group B refills the code stages with direct-to-LDS loads
// (its waits are counted by hand); group A, whose loads the compiler tracks, brings the
// E8M0 scales of each step into a small LDS area of the stage one step ahead.
//
// Fragments: lane l reads row l & 31 and the 16-byte chunks h, h+2, h+4, h+6 (h = l >> 5);
// chunk 2q + h is the lane's 16 bytes for the q-th MFMA of the step: the 32-element block
// 2q + h, whose scale byte the lane supplies.
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int kMxBM = 256, kMxBN = 128, kMxThreads = 512;

__device__ __forceinline__ int mx_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// One 16-byte direct global->LDS load per lane (lane l writes LDS bytes [m0 + 16 l, +16)),
// with the wait state gfx9 asks for between an SALU write of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void mx_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate (gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int mx_wait(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void mx_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__global__ void __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
gemm_mx_pp_kernel(const uint8_t* __restrict__ xq, const uint8_t* __restrict__ sx,
                  const uint8_t* __restrict__ wq, const uint8_t* __restrict__ sw, int M, int N,
                  int Kb, int ksteps, uint16_t* __restrict__ y, int tiles_m, int vec_store) {
  constexpr int BM = kMxBM, BN = kMxBN;
  constexpr int SM = 2, SN = BN / 64;               // 32 x 32 subtiles per wave (64 x BN/2)
  constexpr int XT = BM * 128, WT = BN * 128;       // code bytes of a stage
  constexpr int SCX = BM * 8, SCW = BN * 8;         // scale bytes of a stage
  constexpr int STAGE = XT + WT + SCX + SCW;
  constexpr int XI = BM / 32, WI = BN / 32;         // 1 KB loads per group-B wave per step
  constexpr int DMA = XI + WI, DC = DMA / 2;        // of which issued during the MFMA phase
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2, g4 = wave & 3;
  const int wm = g4, wn = grp;
  // Workgroup ids are dealt round-robin over the 8 XCDs; remap so that consecutive tiles
  // run on one XCD and its L2, walking at most 4 row blocks of X before the next W panel.
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

  // Group B: load d of a step fills X rows 8 (g4 + 4 d) .. +7 (d < XI), else W rows; lane l
  // fetches chunk (l & 7) ^ swizzle of row 8q + (l >> 3). Rows past M or N re-read the last
  // valid row (their results are never stored).
  auto dma_one = [&](int ks, int stage, int d) {
    const uint32_t sbase = lds0 + stage * STAGE + g4 * 1024;
    const bool isx = d < XI;
    const int i = isx ? d : d - XI;
    const int r = 8 * (g4 + 4 * i) + (lane >> 3);
    const int row = isx ? min(m0 + r, M - 1) : min(n0 + r, N - 1);
    const uint32_t vo = (uint32_t)row * (uint32_t)Kb + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
    mx_dma16(sbase + (isx ? 0 : XT) + i * 4096, vo, (isx ? xq : wq) + (size_t)ks * 128);
  };

  // Group A: thread ta keeps X scale row ta and (ta < 128) W scale row ta of one step.
  const int ta = t & 255;
  const uint8_t* sxr = sx + (size_t)min(m0 + ta, M - 1) * S;
  const uint8_t* swr = sw + (size_t)min(n0 + (ta & 127), N - 1) * S;
  u32x2 scx = {0u, 0u}, scw = {0u, 0u};
  auto load_sc = [&](int ks) {
    scx = *reinterpret_cast<const u32x2*>(sxr + (size_t)ks * 8);
    scw = *reinterpret_cast<const u32x2*>(swr + (size_t)ks * 8);
  };
  auto store_sc = [&](int stage) {
    uint8_t* base = lds + stage * STAGE + XT + WT;
    *reinterpret_cast<u32x2*>(base + ta * 8) = scx;
    if (ta < 128) *reinterpret_cast<u32x2*>(base + SCX + ta * 8) = scw;
  };

  const int fr = lane & 31, h = lane >> 5;
  const int xrow0 = wm * 64, wrow0 = wn * (BN / 2);
  int fo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) fo[q] = mx_off(fr, 2 * q + h);

  f32x16 acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = f32x16{};
  i32x4 xf[SM][4], wf[SN][4];
  int ex[SM][4], ew[SN][4];                          // scale byte per subtile and MFMA

  auto lds_phase = [&](int ks) {
    const uint8_t* X = lds + (ks & 1) * STAGE;
    const uint8_t* W = X + XT;
    const uint8_t* SC = W + WT;
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) xf[i][q] = *reinterpret_cast<const i32x4*>(X + (xrow0 + 32 * i) * 128 + fo[q]);
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) wf[j][q] = *reinterpret_cast<const i32x4*>(W + (wrow0 + 32 * j) * 128 + fo[q]);
    u32x2 sxv[SM], swv[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) sxv[i] = *reinterpret_cast<const u32x2*>(SC + (xrow0 + 32 * i + fr) * 8);
#pragma unroll
    for (int j = 0; j < SN; ++j) swv[j] = *reinterpret_cast<const u32x2*>(SC + SCX + (wrow0 + 32 * j + fr) * 8);
    __builtin_amdgcn_s_waitcnt(mx_wait(63, 0));    // this wave's reads of the stage done
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int blk = 2 * q + h;
#pragma unroll
      for (int i = 0; i < SM; ++i) ex[i][q] = (int)((((blk < 4) ? sxv[i].x : sxv[i].y) >> (8 * (blk & 3))) & 0xFFu);
#pragma unroll
      for (int j = 0; j < SN; ++j) ew[j][q] = (int)((((blk < 4) ? swv[j].x : swv[j].y) >> (8 * (blk & 3))) & 0xFFu);
    }
  };
  constexpr int T = SM * SN * 4;                     // MFMAs per wave per step
  // MFMA number u = (i * SN + j) * 4 + q. FP4 operands occupy the low 16 bytes.
  auto mfma_one = [&](int u) {
    const int q = u & 3, j = (u >> 2) % SN, i = (u >> 2) / SN;
    const i32x8_t a = {wf[j][q][0], wf[j][q][1], wf[j][q][2], wf[j][q][3], 0, 0, 0, 0};
    const i32x8_t bb = {xf[i][q][0], xf[i][q][1], xf[i][q][2], xf[i][q][3], 0, 0, 0, 0};
    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, acc[j][i], 4, 4, 0, ew[j][q], 0, ex[i][q]);
  };
  auto mfma_range = [&](int lo, int hi) {
#pragma unroll
    for (int u = 0; u < T; ++u)
      if (u >= lo && u < hi) mfma_one(u);
  };
  auto mfma_phase_loading = [&](int kd, int stage) {
#pragma unroll
    for (int u = 0; u < T; ++u) {
      mfma_one(u);
#pragma unroll
      for (int d = 0; d < DC; ++d)
        if (u == (d * T) / DC) dma_one(kd, stage, DMA - DC + d);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: B loads the codes of steps 0 and 1; A stores step 0's scales and holds step
  // 1's; step 0 is published by the barrier.
  if (grp == 1) {
#pragma unroll
    for (int d = 0; d < DMA; ++d) dma_one(0, 0, d);
#pragma unroll
    for (int d = 0; d < DMA; ++d) dma_one(min(1, ksteps - 1), 1, d);
    __builtin_amdgcn_s_waitcnt(mx_wait(DMA, 15));
  } else {
    load_sc(0);
    store_sc(0);
    if (ksteps > 1) load_sc(1);
    __builtin_amdgcn_s_waitcnt(mx_wait(63, 0));
  }
  mx_barrier();
  // Both groups pass 3 * ksteps + 1 barriers in the loop part.
  if (grp == 0) {
    for (int ks = 0; ks < ksteps; ++ks) {
      if (ks + 1 < ksteps) {                         // scales one step ahead
        store_sc((ks + 1) & 1);
        if (ks + 2 < ksteps) load_sc(ks + 2);
      }
      lds_phase(ks);                                 // slot 2k (waits for the store too)
      __builtin_amdgcn_sched_barrier(0);
      mx_barrier();
      mfma_range(0, T / 2);                          // slot 2k+1, first half
      __builtin_amdgcn_sched_barrier(0);
      mx_barrier();
      mfma_range(T / 2, T);                          // second half
      __builtin_amdgcn_sched_barrier(0);
      mx_barrier();
    }
    mx_barrier();
  } else {
    auto iter = [&](int ks, auto load_c) {
      constexpr bool LOAD = decltype(load_c)::value;
      lds_phase(ks);                                 // slot 2k+1, first half
      __builtin_amdgcn_sched_barrier(0);
      mx_barrier();                                  // no wave reads stage ks & 1 any more
      if constexpr (LOAD) {
#pragma unroll
        for (int d = 0; d < DMA - DC; ++d) dma_one(ks + 2, ks & 1, d);
        __builtin_amdgcn_s_waitcnt(mx_wait(DMA - DC, 15));   // all of step k+1 landed
      } else {
        __builtin_amdgcn_s_waitcnt(mx_wait(0, 15));
      }
      __builtin_amdgcn_sched_barrier(0);
      mx_barrier();
      if constexpr (LOAD) mfma_phase_loading(ks + 2, ks & 1);   // slot 2k+2
      else mfma_range(0, T);
      __builtin_amdgcn_sched_barrier(0);
      mx_barrier();
    };
    mx_barrier();                                    // slot 0
    int ks = 0;
    for (; ks + 2 < ksteps; ++ks) iter(ks, std::true_type{});
    for (; ks < ksteps; ++ks) iter(ks, std::false_type{});
  }

  // ---- epilogue
  __builtin_amdgcn_s_waitcnt(mx_wait(0, 0));
  mx_barrier();
  {
    constexpr int RS = BN * 2 + 16;                    // padded rows
    static_assert(BM * RS <= 2 * STAGE, "output tile must fit in the pipeline LDS");
    // In the 32x32 result (A = W fragment, B = X fragment), lane l holds output row
    // m = 32 i + (l & 31) and the columns 32 j + 8 q + 4 (l >> 5) + r, q, r in 0..3.
  #pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int rl = xrow0 + 32 * i + fr;
  #pragma unroll
      for (int j = 0; j < SN; ++j)
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = wrow0 + 32 * j + 8 * q + 4 * h;
          const f32x16 a = acc[j][i];
          const u32x2 o = {pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
          *reinterpret_cast<u32x2*>(lds + rl * RS + cl * 2) = o;
        }
    }
    __builtin_amdgcn_s_waitcnt(mx_wait(63, 0));
    mx_barrier();
    constexpr int CPR = BN / 8;                        // 16-byte chunks per output row
    constexpr int ITERS = BM * CPR / kMxThreads;
    u32x4 ov[ITERS];
  #pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int c = t + it * kMxThreads;
      const int rl = c / CPR, ch = c - rl * CPR;
      ov[it] = *reinterpret_cast<const u32x4*>(lds + rl * RS + ch * 16);
    }
  #pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int c = t + it * kMxThreads;
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

// MXFP4: 256 x 256 tiles on one wave per SIMD (gemm_mx_solo.hip) once they fill a round of
// the CUs (8192^3: 365 -> 293 us; 4096^3: 52 -> 42 us; 4096 x 18432 x 7168: 364 -> 316 us);
// below that the 256 x 128 tiles of this kernel (2048 x 4096 x 4096: 27 against 37 us).
hipError_t launch_gemm_mxfp4(const void* xq, const uint8_t* sx, const void* wq, const uint8_t* sw,
                             int64_t M, int64_t N, int64_t K, void* y, hipStream_t st) {
  if (((M + 255) / 256) * ((N + 255) / 256) >= 256)
    return launch_gemm_mx_solo(xq, sx, wq, sw, M, N, K, y, st);
  const int tiles_m = (int)((M + kMxBM - 1) / kMxBM);
  const int tiles_n = (int)((N + kMxBN - 1) / kMxBN);
  hipLaunchKernelGGL(gemm_mx_pp_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(kMxThreads), 0, st,
                     (const uint8_t*)xq, sx, (const uint8_t*)wq, sw, (int)M, (int)N, (int)(K / 2),
                     (int)(K / 256), (uint16_t*)y, tiles_m, (int)((N % 8) == 0));
  return hipGetLastError();
}

}  // namespace w8a8
