// Low-precision GEMMs with fused scale epilogues on gfx950 matrix cores.
//
//   FP8    y = bf16( s_x[m] s_w[n] sum_k dec(xq) dec(wq) )      v_mfma_f32_16x16x128_f8f6f4
//   INT8   y = bf16( fp32(fp32(acc_i32) s_x[m]) s_w[n] )        v_mfma_i32_16x16x64_i8
//   BLOCK  y = bf16( sum_g s_x[m,g] s_w[n/128,g] partial_g )    fp32 partial per 128-K group
//   MXFP4  y = bf16( sum_b 2^ex 2^ew sum dec4 dec4 )            v_mfma_scale_f32_16x16x128_f8f6f4
//
// The scales are applied after the low-precision reduction, which the scale-factoring
// identity diag(s_X)(X_q W_q^T)diag(s_W) allows ("FP8 and FP4 inference, SmoothQuant and
// activation quantization", Scale granularity; "FP8 and INT8 Inference" §6-9 epilogue;
// "Low-bit LLM Weights and Activations" §3.4). The block-scaled variant promotes each
// 128-wide K group's fp32 partial into the running fp32 sum ("FP8 and INT8 Inference" §5,
// What DeepSeek did); MXFP4 lets the matrix core apply the E8M0 block scales
// ("Low-bit LLM Weights and Activations" §2.4).
//
// Structure (one 256-thread workgroup = 4 waves per output tile of 256 x BN):
//  - K advances 128 bytes per step (128 FP8/INT8 or 256 FP4 elements); X [256 x 128 B]
//    and W [BN x 128 B] stage through a double-buffered LDS tile (global -> VGPR -> LDS),
//    the next step's global loads in flight while the current step runs on the MFMAs.
//  - LDS rows are 128 B; 16-byte chunk c of row r sits at chunk slot c ^ (r & 7), so the
//    fragment reads (16 rows x 32 B per instruction) are bank-conflict free.
//  - The waves form a 2 x 2 grid: each owns 128 rows of X and BN/2 rows of W. The MFMA
//    A operand is a W fragment and B an X fragment, so each lane's four accumulators are
//    four consecutive output columns of one row: the epilogue stores 8 contiguous bytes.
//  - Workgroup ids are remapped so that consecutive tiles land on the same XCD (ids are
//    dealt round-robin over the 8 XCDs) and tiles sharing a W panel share an L2.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {

enum Kind : int { KIND_FP8 = 0, KIND_INT8 = 1, KIND_BLOCK = 2, KIND_MXFP4 = 3 };

constexpr int kBM = 256;
constexpr int kThreads = 256;

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <int BN, int KIND>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
gemm_kernel(const uint8_t* __restrict__ xq, const void* __restrict__ sxp,
            const uint8_t* __restrict__ wq, const void* __restrict__ swp, int M, int N,
            int Kb, int ksteps, uint16_t* __restrict__ y, int tiles_m, int vec_store) {
  constexpr int SM = 8;                 // 16-row X subtiles per wave (128 rows)
  constexpr int SN = BN / 32;           // 16-row W subtiles per wave (BN/2 rows)
  constexpr int XCH = kBM / 32;         // 16-byte X chunks per thread per step
  constexpr int WCH = BN / 32;          // 16-byte W chunks per thread per step
  constexpr int XT = kBM * 128, WT = BN * 128;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (XT + WT)];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  int b = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int tm = b % tiles_m, tn = b / tiles_m;
  const int m0 = tm * kBM, n0 = tn * BN;

  // Global -> LDS staging map: thread t moves chunk (t & 7) of rows (t >> 3) + 32 i.
  const int lrow = t >> 3, lch = t & 7;
  uint32_t xo[XCH], wo[WCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) xo[i] = (uint32_t)min(m0 + lrow + 32 * i, M - 1) * (uint32_t)Kb + lch * 16;
#pragma unroll
  for (int i = 0; i < WCH; ++i) wo[i] = (uint32_t)min(n0 + lrow + 32 * i, N - 1) * (uint32_t)Kb + lch * 16;
  const int st_off = lds_off(lrow, lch);   // row lrow + 32 i has the same (row & 7)

  // Fragment map: lane reads row (lane & 15) of a 16-row subtile, chunks 2g and 2g + 1.
  const int fr = lane & 15, g = lane >> 4;
  const int fo0 = fr * 128 + (((2 * g) ^ (fr & 7)) << 4);
  const int fo1 = fr * 128 + (((2 * g + 1) ^ (fr & 7)) << 4);
  const int xrow0 = wm * 128, wrow0 = wn * (BN / 2);

  typedef typename std::conditional<KIND == KIND_INT8, i32x4, f32x4>::type acc_t;
  acc_t acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = acc_t{0, 0, 0, 0};

  // Per-lane scale state of the block-scaled and MXFP4 variants.
  const int G = ksteps;                    // one scale column per K step
  int srow[SM];
#pragma unroll
  for (int i = 0; i < SM; ++i) srow[i] = min(m0 + xrow0 + 16 * i + fr, M - 1);
  int swrow[SN];
#pragma unroll
  for (int j = 0; j < SN; ++j) swrow[j] = min(n0 + wrow0 + 16 * j + fr, N - 1);

  u32x4 xs[XCH], ws[WCH];
  auto gload = [&](int ks) {
    const uint32_t kof = (uint32_t)ks * 128u;
#pragma unroll
    for (int i = 0; i < XCH; ++i) xs[i] = *reinterpret_cast<const u32x4*>(xq + xo[i] + kof);
#pragma unroll
    for (int i = 0; i < WCH; ++i) ws[i] = *reinterpret_cast<const u32x4*>(wq + wo[i] + kof);
  };
  auto sstore = [&](int buf) {
    uint8_t* X = lds + buf * (XT + WT);
    uint8_t* W = X + XT;
#pragma unroll
    for (int i = 0; i < XCH; ++i) *reinterpret_cast<u32x4*>(X + st_off + i * 4096) = xs[i];
#pragma unroll
    for (int i = 0; i < WCH; ++i) *reinterpret_cast<u32x4*>(W + st_off + i * 4096) = ws[i];
  };
  auto frag = [&](const uint8_t* base) -> i32x8 {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(base + fo0);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(base + fo1);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < ksteps) gload(ks + 1);

    // scales for this K step (block-scaled: fp32 per row group / W block; MXFP4: the two
    // E8M0 bytes of this lane's blocks 2g and 2g + 1)
    float sxv[SM], swv[SN];
    uint32_t sxe[SM], swe[SN];
    if (KIND == KIND_BLOCK) {
      const float* sx = reinterpret_cast<const float*>(sxp);
      const float* sw = reinterpret_cast<const float*>(swp);
#pragma unroll
      for (int i = 0; i < SM; ++i) sxv[i] = sx[(size_t)srow[i] * G + ks];
#pragma unroll
      for (int j = 0; j < SN; ++j) swv[j] = sw[(size_t)(min(n0 + wrow0 + 16 * j, N - 1) >> 7) * G + ks];
    }
    if (KIND == KIND_MXFP4) {
      const uint8_t* sx = reinterpret_cast<const uint8_t*>(sxp);
      const uint8_t* sw = reinterpret_cast<const uint8_t*>(swp);
      const int S = ksteps * 8;            // E8M0 bytes per row
#pragma unroll
      for (int i = 0; i < SM; ++i)
        sxe[i] = *reinterpret_cast<const uint16_t*>(sx + (size_t)srow[i] * S + ks * 8 + 2 * g);
#pragma unroll
      for (int j = 0; j < SN; ++j)
        swe[j] = *reinterpret_cast<const uint16_t*>(sw + (size_t)swrow[j] * S + ks * 8 + 2 * g);
    }

    const uint8_t* X = lds + cur * (XT + WT);
    const uint8_t* W = X + XT;
    i32x8 xf[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) xf[i] = frag(X + (xrow0 + 16 * i) * 128);
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const i32x8 wf = frag(W + (wrow0 + 16 * j) * 128);
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        if constexpr (KIND == KIND_FP8) {
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[i], acc[j][i], 0, 0, 0, 0, 0, 0);
        } else if constexpr (KIND == KIND_INT8) {
          const i32x4 wl = __builtin_shufflevector(wf, wf, 0, 1, 2, 3);
          const i32x4 wh = __builtin_shufflevector(wf, wf, 4, 5, 6, 7);
          const i32x4 xl = __builtin_shufflevector(xf[i], xf[i], 0, 1, 2, 3);
          const i32x4 xh = __builtin_shufflevector(xf[i], xf[i], 4, 5, 6, 7);
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl, xl, acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wh, xh, acc[j][i], 0, 0, 0);
        } else if constexpr (KIND == KIND_BLOCK) {
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf[i], zero, 0, 0, 0, 0, 0, 0);
          const float sc = sxv[i] * swv[j];
          acc[j][i] += p * sc;
        } else {
          // FP4 operands use the low 16 bytes of each fragment register group.
          const i32x8 wf2 = __builtin_shufflevector(wf, wf, 4, 5, 6, 7, 0, 1, 2, 3);
          const i32x8 xf2 = __builtin_shufflevector(xf[i], xf[i], 4, 5, 6, 7, 0, 1, 2, 3);
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf, xf[i], acc[j][i], 4, 4, 0, (int)(swe[j] & 0xFFu), 0, (int)(sxe[i] & 0xFFu));
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf2, xf2, acc[j][i], 4, 4, 0, (int)(swe[j] >> 8), 0, (int)(sxe[i] >> 8));
        }
      }
    }

    if (ks + 1 < ksteps) sstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds rows m = m0 + xrow0 + 16 i + (lane & 15), columns
  // n = n0 + wrow0 + 16 j + 4 (lane >> 4) + {0..3}.
  const float* sxf = reinterpret_cast<const float*>(sxp);
  const float* swf = reinterpret_cast<const float*>(swp);
#pragma unroll
  for (int j = 0; j < SN; ++j) {
    const int n = n0 + wrow0 + 16 * j + 4 * g;
    float swr[4] = {1.f, 1.f, 1.f, 1.f};
    if (KIND == KIND_FP8 || KIND == KIND_INT8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) swr[r] = swf[min(n + r, N - 1)];
    }
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int m = m0 + xrow0 + 16 * i + fr;
      if (m >= M) continue;
      float v[4];
      if constexpr (KIND == KIND_FP8) {
        const float sm = sxf[m];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[j][i][r] * (sm * swr[r]);
      } else if constexpr (KIND == KIND_INT8) {
        const float sm = sxf[m];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = __fmul_rn(__fmul_rn((float)acc[j][i][r], sm), swr[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[j][i][r];
      }
      uint16_t* yr = y + (size_t)m * N;
      if (vec_store && n + 3 < N) {
        u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *reinterpret_cast<u32x2*>(yr + n) = o;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) yr[n + r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xFFFFu);
      }
    }
  }
}

// Tile width along N: among the widths a kernel variant supports, the one that fills the
// 256 CUs with the fewest workgroup waves (work per wave grows with BN); ties go to the
// wider tile. The block-scaled variant keeps a second fp32 partial per accumulator and
// the MXFP4 variant two scale registers per subtile, so they stop at narrower tiles to
// stay within the register file without spilling.
static int pick_bn(int64_t M, int64_t N, int max_bn) {
  const int cands[4] = {256, 224, 192, 128};
  const int64_t tm = (M + kBM - 1) / kBM;
  int best = 128;
  int64_t best_cost = INT64_MAX;
  for (int c : cands) {
    if (c > max_bn) continue;
    const int64_t tiles = tm * ((N + c - 1) / c);
    const int64_t cost = ((tiles + 255) / 256) * c;
    if (cost < best_cost) { best_cost = cost; best = c; }
  }
  return best;
}

template <int BN, int KIND>
static void launch_bn(dim3 grid, hipStream_t st, const void* xq, const void* sx, const void* wq,
                      const void* sw, int64_t M, int64_t N, int64_t Kb, int ksteps, void* y,
                      int tiles_m, int vec) {
  hipLaunchKernelGGL((gemm_kernel<BN, KIND>), grid, dim3(kThreads), 0, st, (const uint8_t*)xq,
                     sx, (const uint8_t*)wq, sw, (int)M, (int)N, (int)Kb, ksteps, (uint16_t*)y,
                     tiles_m, vec);
}

template <int KIND>
static hipError_t launch_kind(const void* xq, const void* sx, const void* wq, const void* sw,
                              int64_t M, int64_t N, int64_t Kb, void* y, hipStream_t st) {
  constexpr int kMaxBN = KIND == KIND_BLOCK ? 128 : (KIND == KIND_MXFP4 ? 224 : 256);
  const int bn = pick_bn(M, N, kMaxBN);
  const int tiles_m = (int)((M + kBM - 1) / kBM);
  const int tiles_n = (int)((N + bn - 1) / bn);
  const int ksteps = (int)(Kb / 128);
  const int vec = (N % 4) == 0;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  if constexpr (kMaxBN >= 256) {
    if (bn == 256) { launch_bn<256, KIND>(grid, st, xq, sx, wq, sw, M, N, Kb, ksteps, y, tiles_m, vec); return hipGetLastError(); }
  }
  if constexpr (kMaxBN >= 224) {
    if (bn == 224) { launch_bn<224, KIND>(grid, st, xq, sx, wq, sw, M, N, Kb, ksteps, y, tiles_m, vec); return hipGetLastError(); }
    if (bn == 192) { launch_bn<192, KIND>(grid, st, xq, sx, wq, sw, M, N, Kb, ksteps, y, tiles_m, vec); return hipGetLastError(); }
  }
  launch_bn<128, KIND>(grid, st, xq, sx, wq, sw, M, N, Kb, ksteps, y, tiles_m, vec);
  return hipGetLastError();
}

hipError_t launch_gemm(const void* xq, const float* sx, const void* wq, const float* sw,
                       int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st) {
  if (fmt == 1) return launch_kind<KIND_INT8>(xq, sx, wq, sw, M, N, K, y, st);
  return launch_kind<KIND_FP8>(xq, sx, wq, sw, M, N, K, y, st);
}

hipError_t launch_gemm_blockscaled(const void* xq, const float* sx, const void* wq,
                                   const float* sw, int64_t M, int64_t N, int64_t K, void* y,
                                   hipStream_t st) {
  return launch_kind<KIND_BLOCK>(xq, sx, wq, sw, M, N, K, y, st);
}

hipError_t launch_gemm_mxfp4(const void* xq, const uint8_t* sx, const void* wq,
                             const uint8_t* sw, int64_t M, int64_t N, int64_t K, void* y,
                             hipStream_t st) {
  return launch_kind<KIND_MXFP4>(xq, sx, wq, sw, M, N, K / 2, y, st);
}

}  // namespace w8a8
