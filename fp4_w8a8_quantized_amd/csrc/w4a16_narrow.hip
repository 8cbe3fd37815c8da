// W4A16 GEMM for 9-128 tokens on gfx950: y = X W^T with bf16 X and symmetric INT4 weights,
// one fp16 scale per row and group of 128 along K ("Low-bit LLM Weights and Activations"
// §2.3 for the format, §3.3 for dequantizing the weights next to a 16-bit matrix product).
// Per group, four 16x16x32 bf16 MFMAs from zero sum the exact products of the activations and
// the codes plus 136 (a bias that makes the conversion to bf16 a few integer instructions),
// four more sum the activations; the partial minus 136 times that sum, times the group's
// scale, is added to the running sum.
//
// Below the ridge point the time is the time to stream the codes from HBM once, plus what the
// CUs spend re-reading X from the L2. A workgroup of 4 waves owns BM token rows (16 or 32)
// against BN weight rows (16-64), a tile whose workgroups fit one round of the CUs (two per
// CU for the 16-row tiles):
//  - each LDS stage holds 4 groups (512 elements of K) of every row of the tile: 1 KB of X
//    per token row, 256 bytes of codes per weight row and the 8 bytes of the row's four
//    scales. Direct-to-LDS loads fill it with whole cache lines per row (one X row or four
//    code rows per 1 KB load; the scales 4 bytes per lane), so the code stream reaches HBM
//    as 256-byte runs per row;
//  - a ring of ST stages is issued ST - 1 stages ahead; one barrier per stage publishes it
//    and retires the one read before;
//  - the 4 waves form a WM x WN x WK grid: wave (wm, wn, wk) owns a (BM / WM) x (BN / WN)
//    part of the tile as 16 x 16 subtiles and the groups q = wk mod WK of every stage; with
//    WK > 1 the waves' partial sums meet in LDS after the loop, added in wk order;
//  - fragments: for group q, lane l takes row l & 15 and the 32 elements 32 (l >> 4) ..
//    +31 of the group (16 bytes of codes, converted to four bf16x8 of 136 + code in
//    registers; the same elements of X in four 16-byte reads); in LDS, chunk c of row r
//    sits at slot c ^ (r & 15), which keeps the 16 rows of a fragment read on distinct
//    banks.
// Rows past M or N re-read the last valid row; their results are never stored. Needs K a
// multiple of 512 (whole stages, and 4-byte-aligned scale pairs).
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kW4nGroups = 4;                        // groups of 128 per stage
constexpr int kW4nXRow = kW4nGroups * 128 * 2;       // bytes of one token row per stage (1 KB)
constexpr int kW4nWRow = kW4nGroups * 64;            // code bytes of one weight row per stage
constexpr int kW4nSRow = kW4nGroups * 2;             // scale bytes of one weight row per stage

// One 16-byte (4-byte) direct global->LDS load per lane: lane l writes LDS bytes
// [m0 + 16 l, +16) ([m0 + 4 l, +4)), with the wait state gfx9 asks for between an SALU write
// of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void w4n_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}
__device__ __forceinline__ void w4n_dma4(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate waiting for vmcnt <= vm only (gfx9 encoding).
constexpr int w4n_wait(int vm) { return (vm & 15) | (7 << 4) | (15 << 8) | (((vm >> 4) & 3) << 14); }

__device__ __forceinline__ void w4n_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Eight 4-bit two's-complement codes n (element 2i in the low nibble of byte i) as eight bf16
// of 136 + n, exactly: n + 8 = n ^ 8 is the unsigned nibble u, and the bf16 pattern
// 0x4300 | u is 128 + u (one unit in the last place at 128). That is 1.5 integer
// instructions per element against 3.5 for a conversion through fp32; the bias comes off
// each group's sum as 136 times the group's sum of X.
__device__ __forceinline__ bf16x8 w4n_codes_to_bf16_biased(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;   // u0 u2 u4 u6 | u1 u3 u5 u7
  u32x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[i] = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | ((4u + i) << 16) | (uint32_t)i) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, p);
}

template <int BM, int BN, int WK, int ST, int XR>
__global__ void __launch_bounds__(256)
gemm_w4a16_narrow_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ wq,
                         const uint8_t* __restrict__ sc, int M, int N, int K, int groups, int kblocks,
                         int tiles_m, uint16_t* __restrict__ y) {
  constexpr int WMN = 4 / WK;
  constexpr int WM = (BM >= 32 && WMN >= 2) ? 2 : 1, WN = WMN / WM;
  constexpr int TM = BM / WM, TN = BN / WN;          // wave tile
  constexpr int SM = TM / 16, SN = TN / 16;          // 16 x 16 subtiles per wave
  static_assert(WK * WMN == 4 && SM >= 1 && SN >= 1 && SM * 16 * WM == BM && SN * 16 * WN == BN, "tile shape");
  // XR token rows of X are staged per tile: BM, or 8 of a 16-row tile when M <= 8, whose
  // fragment rows 8-15 then read rows 0-7 again (their outputs are never stored).
  static_assert(XR == BM || (XR == 8 && BM == 16), "staged X rows");
  static_assert(kW4nGroups % WK == 0, "every wave takes the same number of groups per stage");
  constexpr int SROWS = BN < 32 ? 32 : BN;           // scale rows per stage (32 per 4-byte load)
  constexpr int XST = XR * kW4nXRow, WST = BN * kW4nWRow, SST = SROWS * kW4nSRow;
  constexpr int STAGE = XST + WST + SST;
  constexpr int NDX = XR, NDW = BN / 4, NDS = SROWS / 32;
  constexpr int ND = NDX + NDW + NDS;                // loads per stage
  constexpr int NQ = (ND + 3) / 4;                   // loads per wave per stage, at most
  constexpr int NDR = ND % 4;                        // waves below NDR issue NQ, others NQ - 1
  constexpr int LA = NQ, LB = NDR == 0 ? NQ : NQ - 1;
  static_assert(ST >= 3 && LA * (ST - 2) < 64, "vmcnt holds at most 63");
  static_assert(ST * STAGE <= 160 * 1024, "LDS");
  static_assert(WK == 1 || (WK - 1) * WMN * SN * SM * 64 * 16 <= ST * STAGE, "reduction area");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[ST * STAGE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wk = wave % WK, wmn = wave / WK;
  const int wm = wmn / WN, wn = wmn % WN;
  const int fr = lane & 15, g = lane >> 4;

  // Logical workgroup id: the row tiles of a weight panel share an XCD and its L2.
  int b = blockIdx.x;
  const int nb = gridDim.x;
  if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
  const int tm = b % tiles_m, tn = b / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // Per load slot q of this wave: the lane's byte offset within the stage's block of its
  // operand (fixed over the loop), and the LDS offset of the load within a stage.
  const uint32_t rowx = (uint32_t)K * 2u, roww = (uint32_t)K / 2u, rows_ = (uint32_t)groups * 2u;
  uint32_t voff[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int d = min(wave + 4 * q, ND - 1);
    if (d < NDX) {                                   // token row d, 1 KB
      voff[q] = (uint32_t)min(m0 + d, M - 1) * rowx + (uint32_t)((lane ^ (d & 15)) << 4);
    } else if (d < NDX + NDW) {                      // code rows 4 dd .. 4 dd + 3, 256 bytes each
      const int r = 4 * (d - NDX) + (lane >> 4);
      voff[q] = (uint32_t)min(n0 + r, N - 1) * roww + (uint32_t)(((lane & 15) ^ (r & 15)) << 4);
    } else {                                         // scale rows 32 ds .. +31, 8 bytes each
      const int r = 32 * (d - NDX - NDW) + (lane >> 1);
      voff[q] = (uint32_t)min(n0 + r, N - 1) * rows_ + (uint32_t)((lane & 1) << 2);
    }
  }
  auto dma = [&](int kb) {
    const uint32_t sb = lds0 + (kb % ST) * STAGE;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int d = wave + 4 * q;
      if (d < NDX) w4n_dma16(sb + d * 1024, voff[q], x + (size_t)kb * kW4nXRow);
      else if (d < NDX + NDW) w4n_dma16(sb + XST + (d - NDX) * 1024, voff[q], wq + (size_t)kb * kW4nWRow);
      else if (d < ND) w4n_dma4(sb + XST + WST + (d - NDX - NDW) * 256, voff[q], sc + (size_t)kb * kW4nSRow);
    }
  };
  // Stage kb has landed for this wave once at most the loads of the stages after it that
  // were already issued remain: ST - 2 stages in the steady state, none near the end.
  auto wait_stage = [&](int kb) {
    if (kb + ST - 2 < kblocks) {
      if (wave < NDR || NDR == 0) __builtin_amdgcn_s_waitcnt(w4n_wait(LA * (ST - 2)));
      else __builtin_amdgcn_s_waitcnt(w4n_wait(LB * (ST - 2)));
    } else {
      __builtin_amdgcn_s_waitcnt(w4n_wait(0));
    }
  };

  f32x4 acc[SN][SM];
#pragma unroll
  for (int j = 0; j < SN; ++j)
#pragma unroll
    for (int i = 0; i < SM; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < ST - 1 && kb < kblocks; ++kb) dma(kb);
  for (int kb = 0; kb < kblocks; ++kb) {
    wait_stage(kb);
    w4n_barrier();                                   // stage kb visible; stage of kb - 1 free
    if (kb + ST - 1 < kblocks) dma(kb + ST - 1);
    const uint8_t* X = lds + (kb % ST) * STAGE;
    const uint8_t* W = X + XST;
    const uint8_t* S = W + WST;
    // The four scales (one per group of the stage) of the lane's output rows 4 g + r.
    float s4[SN][4][kW4nGroups];
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(S + (wn * TN + 16 * j + 4 * g + r) * kW4nSRow);
        s4[j][r][0] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x & 0xFFFFu));
        s4[j][r][1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.x >> 16));
        s4[j][r][2] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y & 0xFFFFu));
        s4[j][r][3] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v.y >> 16));
      }
#pragma unroll
    for (int qq = 0; qq < kW4nGroups / WK; ++qq) {
      const int q = qq * WK + wk;
      bf16x8 xf[SM][4];
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        const int row = (wm * TM + 16 * i + fr) % XR;
#pragma unroll
        for (int p = 0; p < 4; ++p)
          xf[i][p] = *reinterpret_cast<const bf16x8*>(X + row * kW4nXRow + (((16 * q + 4 * g + p) ^ (row & 15)) << 4));
      }
      // 136 times the group's sum of each token row's X (the same in every output row).
      f32x4 xb[SM];
#pragma unroll
      for (int i = 0; i < SM; ++i) {
        f32x4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 4; ++p)
          xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}),
                                                       xf[i][p], xs, 0, 0, 0);
        xb[i] = xs * 136.0f;
      }
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int row = wn * TN + 16 * j + fr;
        const u32x4 cw = *reinterpret_cast<const u32x4*>(W + row * kW4nWRow + (((4 * q + g) ^ (row & 15)) << 4));
        const bf16x8 wf[4] = {w4n_codes_to_bf16_biased(cw.x), w4n_codes_to_bf16_biased(cw.y),
                              w4n_codes_to_bf16_biased(cw.z), w4n_codes_to_bf16_biased(cw.w)};
#pragma unroll
        for (int i = 0; i < SM; ++i) {
          f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < 4; ++p) part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[p], xf[i][p], part, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][i][r] = __builtin_fmaf(part[r] - xb[i][r], s4[j][r][q], acc[j][i][r]);
        }
      }
    }
  }

  if constexpr (WK > 1) {
    // Partial sums of waves wk = 1 .. WK - 1 through LDS (free once every wave has passed
    // the barrier below), added by wave wk = 0 in wk order.
    w4n_barrier();
    f32x4* red = reinterpret_cast<f32x4*>(lds);
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

  // Lane l holds token row m0 + wm TM + 16 i + (l & 15) and the four consecutive outputs
  // n0 + wn TN + 16 j + 4 (l >> 4) + r.
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int m = m0 + wm * TM + 16 * i + fr;
    if (m >= M) continue;
    uint16_t* yr = y + (size_t)m * N;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int n = n0 + wn * TN + 16 * j + 4 * g;
      if (n >= N) continue;
      const uint32_t o[2] = {pack_bf16x2(acc[j][i][0], acc[j][i][1]), pack_bf16x2(acc[j][i][2], acc[j][i][3])};
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

template <int BM, int BN, int WK, int ST, int XR = BM>
hipError_t launch_w4n(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N, int64_t K,
                      void* y, hipStream_t st) {
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles = tiles_m * (int)((N + BN - 1) / BN);
  if (XR < BM && M > XR) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_w4a16_narrow_kernel<BM, BN, WK, ST, XR>), dim3((unsigned)tiles), dim3(256), 0, st,
                     (const uint8_t*)x, (const uint8_t*)wq, (const uint8_t*)sc, (int)M, (int)N, (int)K,
                     (int)(K / 128), (int)(K / 512), tiles_m, (uint16_t*)y);
  return hipGetLastError();
}

int64_t w4n_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Tile for M x N (-1: the kernel does not take the shape), as measured on MI355X (K = 4096,
// graph replay, against the kernels used before: the decode kernel whose waves split K, and
// the LDS-staged kernel above 16-32 tokens):
//   9-16 tokens on 8193-16384 outputs: 16 x 32 (8 x 14336 14.0 -> 12.5 us, 16 x 14336
//     16.0 -> 12.8); up to 8 tokens the same tile stages only 8 rows of X (8 x 14336 12.0 ->
//     11.5 us, 4 x 14336 11.8 -> 11.5);
//   17-32 tokens: 16 x 16 up to 4096 outputs (32 x 4096 11.0 -> 8.8 us), 16 x 32 up to
//     8192 (24 x 6144 16.8 -> 12.1), 32 x 64 up to 16384 (32 x 14336 25.6 -> 19.6);
//   33-64 tokens: 16 x 32 where one round of them (two per CU) covers the output (64 x 4096
//     17.5 -> 12.6 us, 48 x 4096 17.2 -> 12.3);
//   65-128 tokens: 32 x 64 where one round covers the output (128 x 4096 20.1 -> 18.9 us).
// On wider layers above 32 tokens the LDS-staged kernel stays faster (64 x 14336: 30.4
// against 36.7 us here).
//   2-16 tokens on 4097-8192 outputs: 16 x 16 (K split over the 4 waves; 8 staged X rows
//     up to 8 tokens): 8 x 8192 10.4 -> 8.7 us, 16 x 8192 12.7 -> 9.6.
// Up to 16 tokens on narrower layers the decode kernel stays faster (8 x 4096: 6.1 against
// 7.0 us): its 8 waves per workgroup hide the load latency that this kernel's stages expose.
int w4a16_narrow_config(int64_t M, int64_t N, int64_t K) {
  if (M < 2 || M > 128 || N < 1 || K % 512 != 0) return -1;
  if (M <= 16) {
    if (N > 8192) return w4n_cdiv(N, 32) <= 512 ? (M <= 8 ? 4 : 1) : -1;
    if (N > 4096) return M <= 8 ? 5 : 0;
    return -1;
  }
  if (M <= 32) {
    if (2 * w4n_cdiv(N, 16) <= 512) return 0;
    if (2 * w4n_cdiv(N, 32) <= 512) return 1;
    return w4n_cdiv(N, 64) <= 256 ? 2 : -1;
  }
  if (M <= 64) return w4n_cdiv(M, 16) * w4n_cdiv(N, 32) <= 512 ? 1 : -1;
  return w4n_cdiv(M, 32) * w4n_cdiv(N, 64) <= 256 ? 2 : -1;
}

bool use_w4a16_narrow(int64_t M, int64_t N, int64_t K) { return w4a16_narrow_config(M, N, K) >= 0; }

hipError_t launch_gemm_w4a16_narrow(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                                    int64_t K, void* y, hipStream_t st) {
  switch (w4a16_narrow_config(M, N, K)) {
    case 0: return launch_w4n<16, 16, 4, 3>(x, wq, sc, M, N, K, y, st);
    case 1: return launch_w4n<16, 32, 2, 3>(x, wq, sc, M, N, K, y, st);
    case 2: return launch_w4n<32, 64, 1, 3>(x, wq, sc, M, N, K, y, st);
    case 4: return launch_w4n<16, 32, 2, 3, 8>(x, wq, sc, M, N, K, y, st);
    case 5: return launch_w4n<16, 16, 4, 3, 8>(x, wq, sc, M, N, K, y, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w8a8
