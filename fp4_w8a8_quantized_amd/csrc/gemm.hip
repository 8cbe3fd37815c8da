// The tiled GEMM for INT8 (SmoothQuant W8A8) on gfx950 matrix cores, and the GEMM
// dispatch (few tokens: gemm_skinny.hip; FP8 and block-scaled FP8: gemm_pp.hip; MXFP4:
// gemm_mx_pp.hip).
//
//   INT8   y = bf16( fp32(fp32(acc_i32) s_x[m]) s_w[n] )        v_mfma_i32_32x32x32_i8
//
// The scales are applied after the low-precision reduction, which the scale-factoring
// identity diag(s_X)(X_q W_q^T)diag(s_W) allows ("FP8 and FP4 inference, SmoothQuant and
// activation quantization", Scale granularity; "FP8 and INT8 Inference" §6-9, the GEMM
// epilogue; "Low-bit LLM Weights and Activations" §3.4). INT8 uses the 32x32 MFMA shape,
// which runs at twice the rate of its 16x16 form on gfx950.
//
// One 256-thread workgroup (4 waves, 2 x 2) computes a 256 x BN output tile:
//  - K advances 128 bytes (128 elements) per step. The X
//    [256 x 128 B] and W [BN x 128 B] slices of a step land in an LDS stage by direct
//    global->LDS loads (no register staging). STAGES buffers give the loads STAGES-1
//    steps to land.
//  - LDS rows are 128 B; 16-byte chunk c of row r sits at slot c ^ ((r >> 1) & 7), which
//    keeps fragment reads free of bank conflicts on the 64-bank LDS.
//  - Fragments are double-buffered in registers: while step k's MFMAs run, the wave reads
//    step k+1's fragments, so MFMAs never wait on LDS after a step boundary. One barrier
//    per step publishes the next stage and retires the one just read.
//  - The A operand of every MFMA is a W fragment and B an X fragment, so each lane's
//    accumulators are runs of four consecutive output columns of one row.
//  - The epilogue scales and converts in registers, stages the bf16 tile through the
//    now-free LDS, and writes whole rows with 16-byte stores.
//  - Workgroup ids are remapped so that consecutive tiles (which share a W panel) land
//    on the same XCD and its L2 (ids are dealt round-robin over the 8 XCDs).
#include "common.h"
#include "internal.h"

namespace w8a8 {

constexpr int kBM = 256;
constexpr int kThreads = 256;

// Byte offset of chunk `chunk` of LDS tile row `row`.
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// One 16-byte direct global->LDS load per lane: lane l writes LDS bytes
// [lds_addr + 16 l, +16) (M0 holds the wave's LDS address) from gbase + voff. Issued as
// inline assembly so that the compiler does not serialize it against unrelated LDS reads;
// completion is tracked by hand with vmcnt waits before the barrier that publishes a stage.
// gfx9 wants one wait state between an SALU write of M0 and an LDS-DMA that reads it; the
// compiler cannot see inside the asm to insert it, so the s_nop does.
__device__ __forceinline__ void lds_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int BN, int STAGES, bool OF8>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
gemm_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
            const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
            int Kb, int ksteps, void* __restrict__ yp, int tiles_m, int vec_store, Epilogue ep) {
  constexpr int SUB = 32;                     // MFMA output tile edge
  constexpr int SM = 128 / SUB;               // X subtiles per wave (128 rows)
  constexpr int SN = (BN / 2) / SUB;          // W subtiles per wave (BN/2 rows)
  static_assert(SN * SUB * 2 == BN, "tile width must split into whole subtiles");
  constexpr int XT = kBM * 128, WT = BN * 128, STAGE = XT + WT;
  constexpr int XI = kBM / 32, WI = BN / 32;  // 1 KB DMA instructions per wave per step
  constexpr int DMA_PER_STEP = XI + WI;
  constexpr int FR = 16;                      // fragment registers per subtile
  typedef int frag_t __attribute__((ext_vector_type(FR)));
  typedef i32x16 acc_t;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[STAGES * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  int b = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int tm = b % tiles_m, tn = b / tiles_m;
  const int m0 = tm * kBM, n0 = tn * BN;

  // DMA map: instruction i of wave w fills tile rows 8q..8q+7 (q = w + 4 i); lane l
  // writes slot (l & 7) of row 8q + (l >> 3), which holds chunk (l & 7) ^ ((row >> 1) & 7).
  // Rows past M or N re-read the last valid row (their results are never stored).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  uint32_t xoff[XI], woff[WI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int r = 8 * (wave + 4 * i) + (lane >> 3);
    xoff[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)Kb + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int r = 8 * (wave + 4 * i) + (lane >> 3);
    woff[i] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)Kb + (((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  // DMA instructions [first, first + count) of a step, X rows first, then W rows.
  auto dma_part = [&](int ks, int stage, int first, int count) {
    const uint8_t* xb = xq + (size_t)ks * 128;
    const uint8_t* wb = wq + (size_t)ks * 128;
    const uint32_t sbase = lds0 + stage * STAGE + wave * 1024;
#pragma unroll
    for (int i = 0; i < XI; ++i)
      if (i >= first && i < first + count) lds_dma16(sbase + i * 4096, xoff[i], xb);
#pragma unroll
    for (int i = 0; i < WI; ++i)
      if (XI + i >= first && XI + i < first + count) lds_dma16(sbase + XT + i * 4096, woff[i], wb);
  };
  auto dma = [&](int ks, int stage) { dma_part(ks, stage, 0, DMA_PER_STEP); };

  // Fragment map: lane reads row (lane & 31), chunks h, h+2, h+4, h+6 (h = lane >> 5);
  // chunk 2q + h feeds the q-th of the four 32-deep MFMAs of the step.
  const int fr = lane & 31;
  const int g = lane >> 5;
  int fo[FR / 4];
#pragma unroll
  for (int c = 0; c < FR / 4; ++c) fo[c] = tile_off(fr, 2 * c + g);
  const int xrow0 = wm * 128, wrow0 = wn * (BN / 2);
  auto frag = [&](const uint8_t* base) -> frag_t {
    frag_t f;
#pragma unroll
    for (int c = 0; c < FR / 4; ++c) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(base + fo[c]);
      f[4 * c + 0] = v[0]; f[4 * c + 1] = v[1]; f[4 * c + 2] = v[2]; f[4 * c + 3] = v[3];
    }
    return f;
  };

  acc_t acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = acc_t{};

  // ---- prologue: stages 0..STAGES-1 in flight, stage 0 published, F(0) in registers
  frag_t xf[SM], wf0[SN], wf1[SN];
#pragma unroll
  for (int s = 0; s < STAGES; ++s) dma(min(s, ksteps - 1), s);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((STAGES - 1) * DMA_PER_STEP, 15));
  lds_barrier();
#pragma unroll
  for (int i = 0; i < SM; ++i) xf[i] = frag(lds + (xrow0 + SUB * i) * 128);
#pragma unroll
  for (int j = 0; j < SN; ++j) wf0[j] = frag(lds + XT + (wrow0 + SUB * j) * 128);

  // ---- one K step, branch-free: near the end the loads re-fetch the last step into the
  // stage just retired and the next-fragment reads see a stale stage; neither is used.
  // The loads of step ks+STAGES go out in groups between the MFMA rows of the first half
  // of the step, so the CU's address unit (about 1 KB per 16 cycles, shared by the four
  // waves) works behind the matrix cores instead of holding back their issue.
  constexpr int DMA_SLOTS = SM / 2;
  constexpr int DPS = (DMA_PER_STEP + DMA_SLOTS - 1) / DMA_SLOTS;
  auto step = [&](int ks, frag_t (&wcur)[SN], frag_t (&wnxt)[SN]) {
    // Own loads of step ks+1 landed (later steps may still be in flight), own fragment
    // reads of step ks done; then the barrier makes stage ks+1 visible to every wave and
    // guarantees that stage ks (read during the previous step) is free.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((STAGES - 2) * DMA_PER_STEP, 0));
    lds_barrier();
    const int kdma = min(ks + STAGES, ksteps - 1);
    const uint8_t* X = lds + ((ks + 1) % STAGES) * STAGE;
    const uint8_t* W = X + XT;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
#pragma unroll
      for (int j = 0; j < SN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const i32x4 a = {wcur[j][4 * q], wcur[j][4 * q + 1], wcur[j][4 * q + 2], wcur[j][4 * q + 3]};
          const i32x4 bb = {xf[i][4 * q], xf[i][4 * q + 1], xf[i][4 * q + 2], xf[i][4 * q + 3]};
          acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bb, acc[j][i], 0, 0, 0);
        }
      }
      xf[i] = frag(X + (xrow0 + SUB * i) * 128);
      if (i < SN) wnxt[i] = frag(W + (wrow0 + SUB * i) * 128);
      if (i < DMA_SLOTS) dma_part(kdma, ks % STAGES, i * DPS, DPS);
    }
#pragma unroll
    for (int j = SM; j < SN; ++j) wnxt[j] = frag(W + (wrow0 + SUB * j) * 128);
  };
  int ks = 0;
  for (; ks + 1 < ksteps; ks += 2) {
    step(ks, wf0, wf1);
    step(ks + 1, wf1, wf0);
  }
  if (ks < ksteps) step(ks, wf0, wf1);

  // ---- epilogue: dequantize, add the bias, activate and convert in registers (bf16, or
  // E4M3FN codes of clamp(v / s_out) when OF8), stage the tile through LDS (free once every
  // in-flight load has landed and every wave left the loop), then write whole rows with
  // 16-byte stores. Row stride is padded by 16 B (conflict-free writes down a column); a
  // bf16 tile at BN = 256 does not fit with padding, so its chunks are XOR-swizzled.
  constexpr int ES = OF8 ? 1 : 2;              // output bytes per element
  constexpr bool SWZ = (BN == 256 && !OF8);
  constexpr int RS = SWZ ? 512 : BN * ES + 16;
  static_assert(kBM * RS <= STAGES * STAGE, "output tile must fit in the pipeline LDS");
  auto opos = [&](int row, int byte) -> int {
    return SWZ ? row * RS + ((((byte >> 4) ^ (row & 15)) << 4) | (byte & 15)) : row * RS + byte;
  };
  // The per-row and per-column scales (and biases) this lane needs are loaded in one
  // batch, so their latencies overlap, before the first epilogue barrier.
  constexpr int NG = 4;                       // runs of 4 columns per lane per subtile
  float esm[SM], esn[SN][NG][4], ebias[SN][NG][4];
  const bool has_bias = ep.bias != nullptr;
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = min(n0 + wrow0 + SUB * j + 8 * q + 4 * g + r, N - 1);
        esn[j][q][r] = sw[n];
        ebias[j][q][r] = has_bias ? bf16_lo(ep.bias[n]) : 0.f;
      }
#pragma unroll
  for (int i = 0; i < SM; ++i) esm[i] = sx[min(m0 + xrow0 + SUB * i + fr, M - 1)];
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  lds_barrier();
  // Bias and activation are checked at run time: one copy of the element loop keeps the
  // widest tile within its registers.
  {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int rl = xrow0 + SUB * i + fr;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const int cl = wrow0 + SUB * j + 8 * q + 4 * g;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[r] = mul_rn(mul_rn((float)acc[j][i][4 * q + r], esm[i]), esn[j][q][r]);
            if (has_bias) v[r] = add_rn(v[r], ebias[j][q][r]);
            v[r] = epi_activate(v[r], ep.act);
          }
          if constexpr (OF8) {
            *reinterpret_cast<uint32_t*>(lds + opos(rl, cl)) =
                pack_e4m3x4(epi_requant<true>(v[0], ep.s_out, ep.inv_s_out), epi_requant<true>(v[1], ep.s_out, ep.inv_s_out),
                            epi_requant<true>(v[2], ep.s_out, ep.inv_s_out), epi_requant<true>(v[3], ep.s_out, ep.inv_s_out));
          } else {
            const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2*>(lds + opos(rl, cl * 2)) = o;
          }
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  lds_barrier();
  constexpr int EPC = 16 / ES;                 // output elements per 16-byte chunk
  constexpr int CPR = BN / EPC;                // 16-byte chunks per output row
  for (int c = t; c < kBM * CPR; c += kThreads) {
    const int rl = c / CPR, ch = c - rl * CPR;
    const int m = m0 + rl, n = n0 + ch * EPC;
    if (m >= M || n >= N) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(lds + opos(rl, ch * 16));
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

// Tile width along N: among the widths a variant supports, the one that fills the 256
// CUs with the fewest workgroup waves (work per wave grows with BN); ties go wider.
static int pick_bn(int64_t M, int64_t N, const int* cands, int nc) {
  const int64_t tm = (M + kBM - 1) / kBM;
  int best = cands[nc - 1];
  int64_t best_cost = INT64_MAX;
  for (int i = 0; i < nc; ++i) {
    const int c = cands[i];
    const int64_t tiles = tm * ((N + c - 1) / c);
    const int64_t cost = ((tiles + 255) / 256) * c;
    if (cost < best_cost) { best_cost = cost; best = c; }
  }
  return best;
}

template <int BN, int STAGES, bool OF8>
static hipError_t launch_bn(hipStream_t st, const void* xq, const float* sx, const void* wq,
                            const float* sw, int64_t M, int64_t N, int64_t Kb, void* y,
                            const Epilogue& ep = Epilogue{}) {
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int ksteps = (int)(Kb / 128);
  // 16-byte row stores need 16-byte aligned rows: N % 8 == 0 for bf16, N % 16 for bytes.
  const int vec = OF8 ? (N % 16) == 0 : (N % 8) == 0;
  hipLaunchKernelGGL((gemm_kernel<BN, STAGES, OF8>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kThreads), 0, st, (const uint8_t*)xq, sx, (const uint8_t*)wq, sw,
                     (int)M, (int)N, (int)Kb, ksteps, y, tiles_m, vec, ep);
  return hipGetLastError();
}

// Tile widths: the 32x32 MFMA tiles need multiples of 64.
template <bool OF8>
static hipError_t launch_int8(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, void* y, hipStream_t st,
                              const Epilogue& ep) {
  static const int c[3] = {256, 192, 128};
  switch (pick_bn(M, N, c, 3)) {
    case 256: return launch_bn<256, 2, OF8>(st, xq, sx, wq, sw, M, N, K, y, ep);
    case 192: return launch_bn<192, 2, OF8>(st, xq, sx, wq, sw, M, N, K, y, ep);
    default: return launch_bn<128, 3, OF8>(st, xq, sx, wq, sw, M, N, K, y, ep);
  }
}

// Few tokens: the weight-streaming kernel; FP8 otherwise: the two-waves-per-SIMD kernel;
// INT8: the tiled kernel of this file.
hipError_t launch_gemm(const void* xq, const float* sx, const void* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                       const Epilogue& ep) {
  if (use_skinny(M, N)) return launch_gemm_skinny(xq, sx, wq, sw, M, N, K, fmt, y, st, ep);
  if (fmt == 0) return launch_gemm_pp(xq, sx, wq, sw, M, N, K, y, st, ep);
  if (ep.out_fp8) return launch_int8<true>(xq, sx, wq, sw, M, N, K, y, st, ep);
  return launch_int8<false>(xq, sx, wq, sw, M, N, K, y, st, ep);
}

}  // namespace w8a8
