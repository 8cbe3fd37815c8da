// W4A16 on gfx950: symmetric INT4 weights with one fp16 scale per group of 128 along K,
// and the weight-only decode GEMM y = X W^T with bf16 activations ("Low-bit LLM Weights and
// Activations" §2.3: q in [-7, 7], S = max|x| / 7 per group; §3.3: unpack and dequantize
// the weights next to a 16-bit matrix product; weight traffic is the only gain, so this is
// a decode kernel).
//
// Quantization: four lanes per group (32 elements each); S = fp16(fp32(amax) / 7) (1 for an
// all-zero group, 65504 where fp16 overflows); q = clamp(rint(x / S), -7, 7) with the IEEE
// quotient; codes are 4-bit two's complement, element 2i in the low nibble.
//
// GEMM: organised like the few-token FP8 kernel, around streaming W once at HBM rate. A
// workgroup owns 16 NW weight rows; its WPB waves split the K groups (wave w: groups w,
// w + WPB, ...). Per group a lane reads 16 bytes of its row (32 codes, K offsets 32 g + 0..31
// of the group for lane group g = lane >> 4), converts them to bf16 pairs of 136 + code with
// the biased conversion below (seven integer instructions per eight codes; the exact
// conversion through fp32 took about 28 and measured 2-4% slower) and feeds four 16x16x32
// bf16 MFMAs; X supplies the same K offsets, re-paired to the codes' pairs, and four more
// MFMAs against ones give 136 times its sum, which comes off the group's partial. S is kept
// outside the group's sum: the group's fp32 partial is multiplied by S[n, group] and
// accumulated, which keeps every product exact (S q would need up to 14 significant bits).
// The waves' sums meet in LDS. M above 128 is processed in slices of 128 rows (each re-reads
// W).
//
// GEMV (one token, K a multiple of 2048 up to 16384): the weight stream in whole rows. A
// 16-byte-per-lane load of the tile kernel above covers 16 rows x 64 bytes, half a cache line
// per row. Here each wave reads whole weight rows, a kilobyte of one row per load (8 full
// lines); each lane keeps its K / 64 elements of X in registers for the whole kernel,
// dequantizes its 32 codes per load with the biased conversion and takes the products
// with v_dot2 (two bf16 products accumulated in fp32 per instruction); the row's sum is reduced
// across the wave with DPP moves. The vector unit's work is a large part of the time on wide
// layers: the conversion at seven instructions per eight codes (one three-input bitwise op
// per pair) instead of eleven took 14336 x 4096 from 8.6 to 7.8 us. From two tokens on, the
// MFMA kernel above is faster (the dot products grow with the tokens while the MFMA's are
// free up to 16).
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kG = 128;                 // group size along K
constexpr int kGB = kG / 2;             // code bytes per row and group

// ----------------------------------------------------------------------- quantization
__global__ __launch_bounds__(256) void quant_int4_kernel(const u32x4* __restrict__ x, int64_t nthr,
                                                         uint32_t* __restrict__ q,
                                                         uint16_t* __restrict__ sc) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 32 elements per thread
  const bool live = c < nthr;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = live ? __builtin_nontemporal_load(x + 4 * c + i) : u32x4{0u, 0u, 0u, 0u};
  float amax = fmaxf(fmaxf(chunk_absmax(v[0]), chunk_absmax(v[1])), fmaxf(chunk_absmax(v[2]), chunk_absmax(v[3])));
  amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
  amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
  if (!live) return;
  _Float16 s16 = (_Float16)(amax / 7.0f);                      // IEEE division, then RNE to fp16
  if (__builtin_isinf((float)s16)) s16 = (_Float16)65504.0f;
  if ((float)s16 == 0.f) s16 = (_Float16)1.0f;
  const float s = (float)s16;
  const float rcp = 1.0f / s;                                  // s in [2^-24, 65504]: exact quotient
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __builtin_rintf(div_static(bf16_lo(w[e]), s, rcp));
      const float hi = __builtin_rintf(div_static(bf16_hi(w[e]), s, rcp));
      const int ql = (int)fminf(fmaxf(lo, -7.f), 7.f), qh = (int)fminf(fmaxf(hi, -7.f), 7.f);
      out[i] |= ((uint32_t)(ql & 15) | ((uint32_t)(qh & 15) << 4)) << (8 * e);
    }
  }
  reinterpret_cast<u32x4*>(q)[c] = u32x4{out[0], out[1], out[2], out[3]};
  if ((threadIdx.x & 3) == 0) sc[c >> 2] = __builtin_bit_cast(uint16_t, s16);
}

// ------------------------------------------------------------------------------- GEMM
// Eight 4-bit two's-complement codes n (one word, element 2i in the low nibble of byte i) as
// four bf16 pairs of 136 + n, exactly, pair k (k < 4) being (136 + n_k, 136 + n_{k+4}), whose
// nibbles sit 16 bits apart in the word. With n + 8 = n ^ 8 (the unsigned nibble u), the bf16
// pattern 0x4300 | u is 128 + u; every product x (136 + n) is exact in fp32, and the bias
// comes off each sum as 136 sum x. For a nibble c = n mod 16, c ^ 8 = n + 8, so the pair is
// ((w >> 4k) & 0x000F000F) ^ 0x43084308: one three-input bitwise instruction (v_bitop3_b32)
// and one shift for k > 0, seven instructions a word. The two masks are handed over in
// registers (m, kc): as literals they would not fit one instruction. The partner operand pairs
// x_k with x_{k+4}.
__device__ __forceinline__ void int4x8_to_bf16_biased_k4(uint32_t w, uint32_t m, uint32_t kc,
                                                         uint32_t (&p)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) p[k] = ((w >> (4 * k)) & m) ^ kc;
}

// A constant in a vector register that the compiler cannot fold back into an instruction.
__device__ __forceinline__ uint32_t vreg_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

template <int MT, int WPB, int NW>
__global__ void __launch_bounds__(WPB * 64)
gemm_w4a16_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
                  const uint16_t* __restrict__ sc, int M, int N, int K, int groups,
                  uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) f32x4 red[WPB][NW][MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * NW;
  const int64_t kb = K / 2;

  const uint8_t* wrow[NW];
  const uint16_t* srow[NW][4];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    wrow[j] = wq + (int64_t)min(n0 + 16 * j + fr, N - 1) * kb + 16 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r) srow[j][r] = sc + (int64_t)min(n0 + 16 * j + 4 * g + r, N - 1) * groups;
  }
  const uint16_t* xrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) xrow[i] = x + (int64_t)min(16 * i + fr, M - 1) * K + 32 * g;

  f32x4 acc[NW][MT];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Groups of this wave: gi = wave + WPB * s for s < cnt. Weights, scales and X of the next
  // group are loaded while this one is multiplied. (Two or four groups ahead measured slower:
  // 6.5 and 7.0 against 5.9 us at 8 x 4096 x 4096.)
  const int cnt = (groups - wave + WPB - 1) / WPB;
  u32x4 wn[NW];
  float sn[NW][4];
  u32x4 xn[MT][4];
  auto load = [&](int s) {
    const int gi = wave + WPB * s;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      wn[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[j] + (int64_t)gi * kGB));
#pragma unroll
      for (int r = 0; r < 4; ++r) sn[j][r] = (float)__builtin_bit_cast(_Float16, srow[j][r][gi]);
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xn[i][q] = *reinterpret_cast<const u32x4*>(xrow[i] + (int64_t)gi * kG + 8 * q);
  };
  const uint32_t m4 = vreg_const(0x000F000Fu), kc4 = vreg_const(0x43084308u);
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  if (cnt > 0) load(0);
  for (int s = 0; s < cnt; ++s) {
    u32x4 wc[NW];
    float scur[NW][4];
    u32x4 xv[MT][4];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      wc[j] = wn[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) scur[j][r] = sn[j][r];
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[i][q] = xn[i][q];
    if (s + 1 < cnt) load(s + 1);
    // X re-paired to the codes' pairs (x_k, x_{k+4}) of each 8-element word, and 136 times
    // each token's sum over the group (MFMAs against ones: the same in every output row).
    u32x4 xp[MT][4];
    f32x4 xb[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      f32x4 xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = xv[i][q];
        xp[i][q] = u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                         __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
        xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, v), xs, 0, 0, 0);
      }
      xb[i] = xs * 136.0f;
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const uint32_t ww[4] = {wc[j].x, wc[j].y, wc[j].z, wc[j].w};
      bf16x8 wf[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t pk[4];
        int4x8_to_bf16_biased_k4(ww[q], m4, kc4, pk);
        wf[q] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[q], __builtin_bit_cast(bf16x8, xp[i][q]), part, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][i][r] = __builtin_fmaf(part[r] - xb[i][r], scur[j][r], acc[j][i][r]);
      }
    }
  }

  // Partial sums of the waves meet in LDS. Lane l holds output row m = 16 i + (l & 15) and
  // the four consecutive columns n0 + 16 j + 4 (l >> 4) + r.
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) red[wave][j][i][lane] = acc[j][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < NW * MT * 64; idx += WPB * 64) {
    const int j = idx / (MT * 64), i = (idx >> 6) % MT, l = idx & 63;
    f32x4 v = red[0][j][i][l];
#pragma unroll
    for (int w = 1; w < WPB; ++w) v += red[w][j][i][l];
    const int m = 16 * i + (l & 15), n = n0 + 16 * j + 4 * (l >> 4);
    if (m >= M || n >= N) continue;
    uint16_t* yr = y + (int64_t)m * N;
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

template <int MT, int WPB, int NW>
hipError_t launch_w4a16_cfg(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                            int64_t K, void* y, hipStream_t st) {
  const int blocks = (int)((N + 16 * NW - 1) / (16 * NW));
  hipLaunchKernelGGL((gemm_w4a16_kernel<MT, WPB, NW>), dim3((unsigned)blocks), dim3(WPB * 64), 0, st,
                     (const uint16_t*)x, (const uint8_t*)wq, sc, (int)M, (int)N, (int)K, (int)(K / kG),
                     (uint16_t*)y);
  return hipGetLastError();
}

// Launch shape by token count (MT 16-row subtiles) and layer width, for M <= 128.
hipError_t launch_w4a16_slice(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                              int64_t K, void* y, hipStream_t st) {
  const bool wide = N > 8192;
  if (M <= 16) return wide ? launch_w4a16_cfg<1, 8, 2>(x, wq, sc, M, N, K, y, st)
                           : launch_w4a16_cfg<1, 8, 1>(x, wq, sc, M, N, K, y, st);
  if (M <= 32) return launch_w4a16_cfg<2, 8, 1>(x, wq, sc, M, N, K, y, st);
  if (M <= 64) return launch_w4a16_cfg<4, 4, 1>(x, wq, sc, M, N, K, y, st);
  return launch_w4a16_cfg<8, 4, 1>(x, wq, sc, M, N, K, y, st);
}


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kGvChunk = 2048;          // K elements per load of a whole wave (one kilobyte of codes)

// Wave w of the grid takes weight rows w, w + W, ... (W waves in all), one row in flight: L
// loads of 16 bytes per lane (chunk 64 t + l of the row, K offsets 32 (64 t + l) .. +31). (Two
// rows in flight measured slower: 4.8 against 4.5 us at 4096 rows, 8.7 against 8.5 at 14336.)
template <int L>
__global__ void __launch_bounds__(256)
gemm_w4a16_gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ wq,
                       const uint16_t* __restrict__ sc, int N, int K, int groups,
                       uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), GW = gridDim.x * 4;
  const int cnt = gw < N ? (N - 1 - gw) / GW + 1 : 0;
  const int64_t kb = K / 2;
  u32x4 wb[L];
  uint16_t sb[L];
  auto load = [&](int i) {
    const int n = gw + GW * i;
    const u32x4* wr = reinterpret_cast<const u32x4*>(wq + (int64_t)n * kb);
#pragma unroll
    for (int t = 0; t < L; ++t) {
      wb[t] = __builtin_nontemporal_load(wr + 64 * t + lane);
      sb[t] = sc[(int64_t)n * groups + ((64 * t + lane) >> 2)];
    }
  };
  if (cnt > 0) load(0);
  // X once per workgroup into LDS (its four waves need the same values), then each lane's
  // chunks and 136 times their sums (the conversion's bias).
  __shared__ u32x4 xl[256 * L];
#pragma unroll
  for (int t = 0; t < L; ++t) xl[256 * t + threadIdx.x] = reinterpret_cast<const u32x4*>(x)[256 * t + threadIdx.x];
  __syncthreads();
  uint32_t xw[L][16];
  float xb[L];
#pragma unroll
  for (int t = 0; t < L; ++t) {
    const u32x4* xp = xl + 4 * (64 * t + lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // Eight bf16 of X, (x0 x1) (x2 x3) (x4 x5) (x6 x7) as words, to the conversion's
      // pairs (x0 x4) (x1 x5) (x2 x6) (x3 x7).
      const u32x4 v = xp[q];
      xw[t][4 * q] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
      xw[t][4 * q + 1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
      xw[t][4 * q + 2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
      xw[t][4 * q + 3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
    }
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += __uint_as_float(xw[t][e] << 16) + __uint_as_float(xw[t][e] & 0xFFFF0000u);
    xb[t] = 136.0f * sum;
  }
  const uint32_t m4 = vreg_const(0x000F000Fu), kc4 = vreg_const(0x43084308u);
  for (int i = 0; i < cnt; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < L; ++t) {
      const uint32_t w4[4] = {wb[t].x, wb[t].y, wb[t].z, wb[t].w};
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t pk[4];
        int4x8_to_bf16_biased_k4(w4[j], m4, kc4, pk);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]),
                                              __builtin_bit_cast(bf16x2, xw[t][4 * j + e]), d, false);
      }
      acc = __builtin_fmaf(d - xb[t], (float)__builtin_bit_cast(_Float16, sb[t]), acc);
    }
    if (i + 1 < cnt) load(i + 1);
    acc = wave_sum_dpp(acc);
    if (lane == 63) y[gw + GW * i] = (uint16_t)(pack_bf16x2(acc, 0.f) & 0xFFFFu);
  }
}

template <int L>
hipError_t launch_w4a16_gemv(const void* x, const void* wq, const uint16_t* sc, int64_t N, int64_t K,
                             void* y, hipStream_t st) {
  // About two rows per wave, at most 1024 workgroups (measured at 4096 and 14336 rows; one
  // row per wave, or 4096 workgroups, measured slower).
  const int64_t want = (N + 7) / 8;
  const int blocks = (int)(want < 1 ? 1 : (want > 1024 ? 1024 : want));
  hipLaunchKernelGGL((gemm_w4a16_gemv_kernel<L>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint16_t*)x, (const uint8_t*)wq, sc, (int)N, (int)K, (int)(K / kG),
                     (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_int4(const void* w, int64_t N, int64_t K, void* q, uint16_t* sc,
                                hipStream_t st) {
  const int64_t nthr = N * K / 32;
  hipLaunchKernelGGL(quant_int4_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const u32x4*>(w), nthr, reinterpret_cast<uint32_t*>(q), sc);
  return hipGetLastError();
}

bool use_w4a16_gemv(int64_t M, int64_t N, int64_t K) {
  return M == 1 && K % kGvChunk == 0 && K / kGvChunk <= 8 && N >= 1 && N <= INT32_MAX;
}

hipError_t launch_gemm_w4a16(const void* x, const void* wq, const uint16_t* sc, int64_t M, int64_t N,
                             int64_t K, void* y, hipStream_t st) {
  if (use_w4a16_gemv(M, N, K)) {
    switch (K / kGvChunk) {
      case 1: return launch_w4a16_gemv<1>(x, wq, sc, N, K, y, st);
      case 2: return launch_w4a16_gemv<2>(x, wq, sc, N, K, y, st);
      case 3: return launch_w4a16_gemv<3>(x, wq, sc, N, K, y, st);
      case 4: return launch_w4a16_gemv<4>(x, wq, sc, N, K, y, st);
      case 5: return launch_w4a16_gemv<5>(x, wq, sc, N, K, y, st);
      case 6: return launch_w4a16_gemv<6>(x, wq, sc, N, K, y, st);
      case 7: return launch_w4a16_gemv<7>(x, wq, sc, N, K, y, st);
      default: return launch_w4a16_gemv<8>(x, wq, sc, N, K, y, st);
    }
  }
  if (use_w4a16_narrow(M, N, K)) return launch_gemm_w4a16_narrow(x, wq, sc, M, N, K, y, st);
  if (use_w4a16_mid(M, N, K)) return launch_gemm_w4a16_mid(x, wq, sc, M, N, K, y, st);
  for (int64_t m0 = 0; m0 < M; m0 += 128) {
    const int64_t mr = M - m0 < 128 ? M - m0 : 128;
    const hipError_t e = launch_w4a16_slice(reinterpret_cast<const uint16_t*>(x) + m0 * K, wq, sc, mr,
                                            N, K, reinterpret_cast<uint16_t*>(y) + m0 * N, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace w8a8
