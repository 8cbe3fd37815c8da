// W4A16 GEMM for more than 32 tokens (16 on wide layers) on gfx950: y = X W^T with bf16 X and symmetric INT4
// weights, one fp16 scale per row and group of 128 along K ("Low-bit LLM Weights and
// Activations" §2.3 for the format, §3.3 for dequantizing the weights next to a 16-bit
// matrix product). Same arithmetic as the decode kernel of w4a16.hip: per group, the exact
// bf16 products of codes and activations are summed by four 16x16x32 bf16 MFMAs from zero,
// and that fp32 partial, times the group's scale, is added to the running sum.
//
// The decode kernel's waves split K and load their X fragments from L2 for every MFMA;
// beyond a few tokens that X traffic bounds it (about 125 TFLOP/s at every token count).
// Here a workgroup owns RX = 32, 64 or 128 token rows and RW = 16, 32 or 64 weight rows and
// stages one group (128 elements) of both per K step in LDS by direct-to-LDS loads:
//  - X (256 bytes per row and step) through a ring of 4 stages (6 at 32 rows), issued
//    three (five) steps ahead;
//  - the codes (64 bytes per row and step) and the 16-byte chunk of scales holding the
//    step's group (8 groups, one chunk per weight row) through a ring of up to 16 slots
//    (as many as LDS holds) issued a ring ahead, before the X of the same iteration, so
//    that one hand-counted wait per step covers all three;
//  - the 4 waves tile the workgroup as WN x (4 / WN): wave (wn, wm) owns 16 NWW weight rows
//    against RX WN / 4 token rows, so each wave converts only its own codes to bf16;
//  - one barrier per step publishes the step's stage and slots and retires those read
//    before.
// Rows past M or N re-read the last valid row; their results are never stored. Needs K a
// multiple of 1024 (whole 16-byte scale chunks per row).
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));


// X ring stages by token rows per workgroup: as deep as LDS allows next to the code and
// scale ring (4 stages measured 4-10% faster than 3 at 64 and 128 rows).
constexpr int w4_xstages(int rx) { return rx == 32 ? 6 : 4; }
constexpr int kXRowBytes = 256;                       // one group of one token row (bf16)
constexpr int kWRowBytes = 64;                        // one group of one weight row (int4)

// LDS byte offsets of 16-byte chunk c of a row, swizzled so that the 16 rows one fragment
// read touches fall on distinct banks.
__device__ __forceinline__ int w4_xoff(int row, int c) { return row * kXRowBytes + ((c ^ (row & 15)) << 4); }
__device__ __forceinline__ int w4_woff(int row, int c) { return row * kWRowBytes + ((c ^ ((row >> 2) & 3)) << 4); }

// One 16-byte direct global->LDS load per lane (lane l writes LDS bytes [m0 + 16 l, +16)),
// with the wait state gfx9 asks for between an SALU write of M0 and an LDS-DMA reading it.
__device__ __forceinline__ void w4_dma16(uint32_t lds_addr, uint32_t voff, const uint8_t* gbase) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory");
}

// s_waitcnt immediate waiting for vmcnt <= vm only (gfx9 encoding).
constexpr int w4_wait(int vm) { return (vm & 15) | (7 << 4) | (15 << 8) | (((vm >> 4) & 3) << 14); }

// Eight 4-bit two's-complement codes (element 2i in the low nibble of byte i) as eight
// bf16. The values are small integers, so the high half of their fp32 form is exact.
__device__ __forceinline__ bf16x8 w4_codes_to_bf16(uint32_t w) {
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = __float_as_uint((float)((int)(w << (28 - 4 * e)) >> 28));
  u32x4 p;
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_perm(h[2 * i + 1], h[2 * i], 0x07060302u);
  return __builtin_bit_cast(bf16x8, p);
}

template <int RX, int WN, int NWW>
__global__ void __launch_bounds__(256)
gemm_w4a16_mid_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ wq,
                      const uint8_t* __restrict__ sc, int M, int N, int K, int groups,
                      uint16_t* __restrict__ y) {
  constexpr int XS = w4_xstages(RX);                 // X ring stages
  constexpr int WM = 4 / WN;                         // waves along M
  constexpr int MW = RX / 16 / WM;                   // 16-row token subtiles per wave
  constexpr int RW = 16 * NWW * WN;                  // weight rows per workgroup
  constexpr int XSTAGE = RX * kXRowBytes, WSLOT = RW * kWRowBytes, SSLOT = 1024;
  constexpr int WSFIT = (160 * 1024 - XS * XSTAGE) / (WSLOT + SSLOT);
  constexpr int WS = WSFIT < 16 ? WSFIT : 16;        // code / scale ring slots
  constexpr int NDX = XSTAGE / 1024, NDW = WSLOT / 1024;   // 1 KB loads per step
  constexpr int SWAVE = 3;                           // the wave that loads the scale chunks
  constexpr int LMIN = NDX / 4;                      // loads per wave per step, at least
  static_assert(RW <= 64, "one scale chunk per lane");
  static_assert(MW >= 1 && WS >= XS, "shape");
  static_assert(XS * XSTAGE + WS * (WSLOT + SSLOT) <= 160 * 1024, "LDS");
  static_assert(LMIN * (XS - 2) < 64, "vmcnt holds at most 63");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[XS * XSTAGE + WS * (WSLOT + SSLOT)];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave % WN, wm = wave / WN;
  const int n0 = blockIdx.x * RW, m0 = blockIdx.y * RX;
  const int fr = lane & 15, g = lane >> 4;
  const int ksteps = groups;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  const uint32_t wlds0 = lds0 + XS * XSTAGE, slds0 = wlds0 + WS * WSLOT;

  // The loads of step ks. X: load d carries rows 4 d .. 4 d + 3 (lane l: row 4 d + (l >> 4),
  // LDS chunk l & 15). Codes: load d carries rows 16 d .. 16 d + 15 (lane l: row
  // 16 d + (l >> 2), LDS chunk l & 3). Scales: lane l fetches the chunk of weight row n0 + l
  // that holds group ks. Steps past the last re-fetch the last step into a stage or slot
  // that is never read again.
  auto dma_x = [&](int ks) {
    const uint8_t* xb = x + (size_t)min(ks, ksteps - 1) * kXRowBytes;
#pragma unroll
    for (int d = wave; d < NDX; d += 4) {
      const int r = 4 * d + (lane >> 4);
      const uint32_t vo = (uint32_t)min(m0 + r, M - 1) * (uint32_t)(2 * K) + (((lane & 15) ^ (r & 15)) << 4);
      w4_dma16(lds0 + (ks % XS) * XSTAGE + d * 1024, vo, xb);
    }
  };
  auto dma_w = [&](int ks) {
    const int kc = min(ks, ksteps - 1);
    const uint8_t* wb = wq + (size_t)kc * kWRowBytes;
    for (int d = wave; d < NDW; d += 4) {
      const int r = 16 * d + (lane >> 2);
      const uint32_t vo = (uint32_t)min(n0 + r, N - 1) * (uint32_t)(K / 2) + (((lane & 3) ^ ((r >> 2) & 3)) << 4);
      w4_dma16(wlds0 + (ks % WS) * WSLOT + d * 1024, vo, wb);
    }
    if (wave == SWAVE) {
      const uint32_t vo = (uint32_t)min(n0 + lane, N - 1) * (uint32_t)(2 * groups);
      w4_dma16(slds0 + (ks % WS) * SSLOT, vo, sc + (size_t)(kc >> 3) * 16);
    }
  };

  f32x4 acc[NWW][MW];
#pragma unroll
  for (int j = 0; j < NWW; ++j)
#pragma unroll
    for (int i = 0; i < MW; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue: codes and scales of steps 0 .. WS - 2, with the X of steps 0 .. XS - 2
  // after those of steps WS - XS .. WS - 2, in the order the loop keeps.
  for (int j = 1 - WS; j < 0; ++j) {
    dma_w(j + WS - 1);
    if (j + XS - 1 >= 0) dma_x(j + XS - 1);
  }
  for (int ks = 0; ks < ksteps; ++ks) {
    // The X of step ks was issued XS - 1 iterations ago, after its codes and scales,
    // and every later iteration issued at least LMIN loads from this wave: once at most
    // LMIN (XS - 2) remain, all three have landed for this wave; after the barrier,
    // for every wave, and every wave is done with step ks - 1's stage and slots.
    __builtin_amdgcn_s_waitcnt(w4_wait(LMIN * (XS - 2)));
    asm volatile("s_barrier" ::: "memory");
    dma_w(ks + WS - 1);
    dma_x(ks + XS - 1);
    const uint8_t* X = lds + (ks % XS) * XSTAGE;
    const uint8_t* W = lds + XS * XSTAGE + (ks % WS) * WSLOT;
    const uint8_t* S = lds + XS * XSTAGE + WS * WSLOT + (ks % WS) * SSLOT;
    // Lane (fr, g) covers K elements 32 g .. 32 g + 31 of the group: MFMA p takes 32 g + 8 p
    // .. + 7 of its weight row (code word p of its 16-byte chunk g) and of its token row
    // (X chunk 4 g + p).
    u32x4 xv[MW][4];
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const int row = 16 * (wm * MW + i) + fr;
#pragma unroll
      for (int p = 0; p < 4; ++p) xv[i][p] = *reinterpret_cast<const u32x4*>(X + w4_xoff(row, 4 * g + p));
    }
#pragma unroll
    for (int j = 0; j < NWW; ++j) {
      const int wrow = 16 * (wn * NWW + j);
      const u32x4 wc = *reinterpret_cast<const u32x4*>(W + w4_woff(wrow + fr, g));
      float s[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        s[r] = (float)*reinterpret_cast<const _Float16*>(S + 16 * (wrow + 4 * g + r) + 2 * (ks & 7));
      bf16x8 wf[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) wf[p] = w4_codes_to_bf16(wc[p]);
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < 4; ++p)
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[p], __builtin_bit_cast(bf16x8, xv[i][p]), part, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][i][r] = __builtin_fmaf(part[r], s[r], acc[j][i][r]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(w4_wait(0));           // the re-fetches past the end

  // Lane l holds token row m0 + 16 (wm MW + i) + (l & 15) and the four consecutive outputs
  // n0 + 16 (wn NWW + j) + 4 (l >> 4) + r.
#pragma unroll
  for (int i = 0; i < MW; ++i) {
    const int m = m0 + 16 * (wm * MW + i) + fr;
    if (m >= M) continue;
    uint16_t* yr = y + (size_t)m * N;
#pragma unroll
    for (int j = 0; j < NWW; ++j) {
      const int n = n0 + 16 * (wn * NWW + j) + 4 * g;
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

template <int RX, int WN, int NWW>
hipError_t launch_w4mid_cfg(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                            int64_t K, void* y, hipStream_t st) {
  constexpr int RW = 16 * NWW * WN;
  const dim3 grid((unsigned)((N + RW - 1) / RW), (unsigned)((M + RX - 1) / RX));
  hipLaunchKernelGGL((gemm_w4a16_mid_kernel<RX, WN, NWW>), grid, dim3(256), 0, st, (const uint8_t*)x,
                     (const uint8_t*)wq, (const uint8_t*)sc, (int)M, (int)N, (int)K, (int)(K / 128),
                     (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

// Up to 32 tokens on layers of up to 8192 outputs the decode kernel, which splits K over
// its waves, measured faster (4096 outputs, 32 tokens: 11.5 against 17.5 us).
bool use_w4a16_mid(int64_t M, int64_t N, int64_t K) {
  return (M > 32 || (M > 16 && N > 8192)) && K % 1024 == 0 && (M + 31) / 32 <= 65535 && N > 0;
}

// Launch shapes (token rows RX x weight rows RW per workgroup) and the choice among them.
// Measured at K = 4096, a step of a workgroup takes about (RX + 2 RW) x 5 ns, whatever the
// shape (a weight row costs two token rows: its codes come from HBM and are converted by
// the waves), so take the fewest rounds of workgroups over the 256 CUs times that, the
// later (taller) shape on a tie.
struct W4Shape { int rx, rw; };
static constexpr W4Shape kW4Shapes[] = {{32, 32}, {32, 64}, {64, 16}, {64, 32},
                                        {64, 64}, {128, 32}, {128, 64}};

static int w4a16_mid_shape(int64_t M, int64_t N) {
  int best = 0;
  int64_t best_cost = INT64_MAX;
  for (int i = 0; i < (int)(sizeof(kW4Shapes) / sizeof(kW4Shapes[0])); ++i) {
    const W4Shape& c = kW4Shapes[i];
    const int64_t wg = ((M + c.rx - 1) / c.rx) * ((N + c.rw - 1) / c.rw);
    const int64_t cost = ((wg + 255) / 256) * (c.rx + 2 * c.rw);
    if (cost <= best_cost) { best_cost = cost; best = i; }
  }
  return best;
}

hipError_t launch_gemm_w4a16_mid(const void* x, const void* wq, const uint16_t* sc, int64_t M,
                                 int64_t N, int64_t K, void* y, hipStream_t st) {
  switch (w4a16_mid_shape(M, N)) {
    case 0: return launch_w4mid_cfg<32, 2, 1>(x, wq, sc, M, N, K, y, st);
    case 1: return launch_w4mid_cfg<32, 2, 2>(x, wq, sc, M, N, K, y, st);
    case 2: return launch_w4mid_cfg<64, 1, 1>(x, wq, sc, M, N, K, y, st);
    case 3: return launch_w4mid_cfg<64, 2, 1>(x, wq, sc, M, N, K, y, st);
    case 4: return launch_w4mid_cfg<64, 2, 2>(x, wq, sc, M, N, K, y, st);
    case 5: return launch_w4mid_cfg<128, 2, 1>(x, wq, sc, M, N, K, y, st);
    default: return launch_w4mid_cfg<128, 2, 2>(x, wq, sc, M, N, K, y, st);
  }
}

}  // namespace w8a8
