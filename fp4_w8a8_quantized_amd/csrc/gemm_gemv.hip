// One-token W8A8 GEMM (decode at batch 1) on gfx950: the same result as the other kernels,
//   FP8   y = epilogue( s_x s_w[n] sum_k dec(xq[k]) dec(wq[n,k]) )
//   INT8  y = epilogue( fp32(fp32(acc_i32) s_x) s_w[n] ),  acc_i32 = sum_k xq wq
// for a single row of X, where the time is the time to stream W once ("FP8 and INT8
// Inference", arithmetic intensity and the decode regime).
//
// The tiled few-token kernels load 16 weight rows x 64 bytes per 16-byte-per-lane load, half a
// cache line per row, so that each lane group feeds its own MFMA row. With one token there is
// nothing for the matrix core to do that the vector unit cannot, so here each wave streams
// whole weight rows: a kilobyte of one row per load (8 full lines), all K / 1024 loads of a
// row in flight at once, one row after another (rows w, w + W, ... for wave w of W).
//  - X (K bytes) is read once per workgroup into LDS; each lane then keeps the 16 bytes of
//    every load slot it covers in registers for the whole kernel (FP8: as bf16 pairs).
//  - FP8: the weight codes go to bf16 pairs (v_cvt_scalef32_pk_bf16_fp8 with scale 1, exact:
//    E4M3 values are bf16 values) and v_dot2 takes two products per instruction into fp32
//    (each product of two E4M3 values is exact in fp32). INT8: v_dot4 takes four byte
//    products into the exact int32 sum, so INT8 results are bit-identical to the tiled
//    kernels'.
//  - The row's sum over the wave's lanes is a DPP reduction into lane 63, which applies the
//    epilogue of the other kernels (scales, bias, activation, bf16 or E4M3 output) and writes
//    the output element.
#include "common.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kGmChunk = 1024;          // K bytes per load of a whole wave

// FUSED: the kernel also quantizes X. Every workgroup reads the bf16 row (2K bytes) and
// encodes it into its LDS copy exactly as the per-token quantizer does (row amax, one IEEE
// division for the scale, the same per-element encode); workgroup 0 also stores the codes
// and the scale. That replaces the quantizer's launch in a one-token linear layer.
template <int L, bool FUSED>
__global__ void __launch_bounds__(256)
gemm_gemv_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                 const uint8_t* __restrict__ wq, const float* __restrict__ sw, int N, int K,
                 int kind, void* __restrict__ yp, Epilogue ep, const uint16_t* __restrict__ xbf,
                 uint8_t* __restrict__ xq_out, float* __restrict__ sx_out) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), GW = gridDim.x * 4;
  const int cnt = gw < N ? (N - 1 - gw) / GW + 1 : 0;
  u32x4 wb[L];
  auto load = [&](int i) {
    const u32x4* wr = reinterpret_cast<const u32x4*>(wq + (int64_t)(gw + GW * i) * K);
#pragma unroll
    for (int t = 0; t < L; ++t) wb[t] = __builtin_nontemporal_load(wr + 64 * t + lane);
  };
  if (cnt > 0) load(0);

  __shared__ u32x4 xl[64 * L];
  float sxv;
  if constexpr (FUSED) {
    // The row's 16-byte chunks of bf16 (128 L of them) stay in registers from the amax to the
    // encode: chunk threadIdx.x + 256 i is element i of xraw.
    constexpr int XC = (L + 1) / 2;
    const u32x4* xr = reinterpret_cast<const u32x4*>(xbf);
    const int nchunk = K >> 3;
    u32x4 xraw[XC];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = threadIdx.x + 256 * i;
      xraw[i] = c < nchunk ? xr[c] : u32x4{0u, 0u, 0u, 0u};
      amax = fmaxf(amax, chunk_absmax(xraw[i]));
    }
    amax = wave_max(amax);
    __shared__ float red[4];
    if (lane == 0) red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax_scale(amax, kind == 1 ? 127.0f : 448.0f);
    const bool finite = __builtin_isfinite(s);
    const float rcp = 1.0f / s;
    u32x2* xl2 = reinterpret_cast<u32x2*>(xl);
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = threadIdx.x + 256 * i;
      if (c >= nchunk) break;
      const u32x4 v = xraw[i];
      float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                    bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = finite ? div_by_scale(f[e], s, rcp) : f[e] / s;
      u32x2 o;
      if (kind == 1) {
        o.x = int8_code(f[0]) | (int8_code(f[1]) << 8) | (int8_code(f[2]) << 16) | (int8_code(f[3]) << 24);
        o.y = int8_code(f[4]) | (int8_code(f[5]) << 8) | (int8_code(f[6]) << 16) | (int8_code(f[7]) << 24);
      } else {
        o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
        o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
      }
      xl2[c] = o;
      if (blockIdx.x == 0) reinterpret_cast<u32x2*>(xq_out)[c] = o;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) sx_out[0] = s;
    sxv = s;
  } else {
    for (int c = threadIdx.x; c < 64 * L; c += 256) xl[c] = reinterpret_cast<const u32x4*>(xq)[c];
    sxv = sx[0];
  }
  __syncthreads();
  // The lane's X bytes of load slot t: bf16 pairs (FP8) or the raw words (INT8).
  uint32_t xv[L][8];
#pragma unroll
  for (int t = 0; t < L; ++t) {
    const u32x4 v = xl[64 * t + lane];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (kind == 0) {
        xv[t][2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[j], 1.0f, false));
        xv[t][2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[j], 1.0f, true));
      } else {
        xv[t][2 * j] = w4[j];
        xv[t][2 * j + 1] = 0u;
      }
    }
  }

  for (int i = 0; i < cnt; ++i) {
    float accf = 0.f;
    int acci = 0;
    if (kind == 0) {
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const uint32_t w4[4] = {wb[t].x, wb[t].y, wb[t].z, wb[t].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[j], 1.0f, false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4[j], 1.0f, true);
          accf = __builtin_amdgcn_fdot2_f32_bf16(lo, __builtin_bit_cast(bf16x2, xv[t][2 * j]), accf, false);
          accf = __builtin_amdgcn_fdot2_f32_bf16(hi, __builtin_bit_cast(bf16x2, xv[t][2 * j + 1]), accf, false);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < L; ++t) {
        const uint32_t w4[4] = {wb[t].x, wb[t].y, wb[t].z, wb[t].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) acci = __builtin_amdgcn_sdot4((int)w4[j], (int)xv[t][2 * j], acci, false);
      }
    }
    if (i + 1 < cnt) load(i + 1);
    if (kind == 0) accf = wave_sum_dpp(accf);
    else acci = wave_sum_dpp(acci);
    if (lane == 63) {
      const int n = gw + GW * i;
      const float swn = sw[n];
      float v = kind == 0 ? accf * (sxv * swn) : mul_rn(mul_rn((float)acci, sxv), swn);
      if (ep.bias) v = add_rn(v, bf16_lo(ep.bias[n]));
      v = epi_activate(v, ep.act);
      if (ep.out_fp8) {
        const float q = kind == 0 ? epi_requant<false>(v, ep.s_out, ep.inv_s_out)
                                  : epi_requant<true>(v, ep.s_out, ep.inv_s_out);
        reinterpret_cast<uint8_t*>(yp)[n] = (uint8_t)(pack_e4m3x4(q, 0.f, 0.f, 0.f) & 0xFFu);
      } else {
        reinterpret_cast<uint16_t*>(yp)[n] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
      }
    }
  }
}

// Workgroups: about 1.5 rows per wave (six per workgroup), but no more than fit on the chip
// at once (the register count grows with K). Measured at K = 4096: 4096 rows best at 768
// workgroups (5.0 us against 5.6 at 512), 14336 rows at 2048 (11.0 against 11.4 at 1024);
// K = 14336 (two waves per SIMD) at the 512 that fit.
template <int L, bool FUSED>
int gemv_blocks(int64_t N) {
  static int resident = 0;                         // per CU x CUs, the same on every call
  if (resident == 0) {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_gemv_kernel<L, FUSED>, 256, 0) != hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 1024;
    resident = per_cu > 0 && cus > 0 ? per_cu * cus : 1024;
  }
  const int64_t want = (N + 5) / 6;
  return (int)(want < 1 ? 1 : (want > resident ? resident : want));
}

template <int L>
hipError_t launch_l(const void* xq, const float* sx, const void* wq, const float* sw, int64_t N,
                    int64_t K, int fmt, void* y, hipStream_t st, const Epilogue& ep) {
  const int blocks = gemv_blocks<L, false>(N);
  hipLaunchKernelGGL((gemm_gemv_kernel<L, false>), dim3((unsigned)blocks), dim3(256), 0, st, (const uint8_t*)xq, sx,
                     (const uint8_t*)wq, sw, (int)N, (int)K, fmt, y, ep, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

template <int L>
hipError_t launch_fused_l(const void* xbf, const void* wq, const float* sw, int64_t N, int64_t K, int fmt,
                          void* xq, float* sx, void* y, hipStream_t st) {
  const int blocks = gemv_blocks<L, true>(N);
  hipLaunchKernelGGL((gemm_gemv_kernel<L, true>), dim3((unsigned)blocks), dim3(256), 0, st, nullptr, nullptr,
                     (const uint8_t*)wq, sw, (int)N, (int)K, fmt, y, Epilogue{}, (const uint16_t*)xbf,
                     (uint8_t*)xq, sx);
  return hipGetLastError();
}

}  // namespace

bool use_gemm_gemv(int64_t M, int64_t N, int64_t K) {
  return M == 1 && K % kGmChunk == 0 && K / kGmChunk >= 1 && K / kGmChunk <= 16 && N >= 1;
}

hipError_t launch_gemm_gemv(const void* xq, const float* sx, const void* wq, const float* sw, int64_t N,
                            int64_t K, int fmt, void* y, hipStream_t st, const Epilogue& ep) {
  switch (K / kGmChunk) {
    case 1: return launch_l<1>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 2: return launch_l<2>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 3: return launch_l<3>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 4: return launch_l<4>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 5: return launch_l<5>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 6: return launch_l<6>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 7: return launch_l<7>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 8: return launch_l<8>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 9: return launch_l<9>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 10: return launch_l<10>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 11: return launch_l<11>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 12: return launch_l<12>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 13: return launch_l<13>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 14: return launch_l<14>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    case 15: return launch_l<15>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
    default: return launch_l<16>(xq, sx, wq, sw, N, K, fmt, y, st, ep);
  }
}

hipError_t launch_linear_gemv(const void* xbf, const void* wq, const float* sw, int64_t N, int64_t K, int fmt,
                              void* xq, float* sx, void* y, hipStream_t st) {
  switch (K / kGmChunk) {
    case 1: return launch_fused_l<1>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 2: return launch_fused_l<2>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 3: return launch_fused_l<3>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 4: return launch_fused_l<4>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 5: return launch_fused_l<5>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 6: return launch_fused_l<6>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 7: return launch_fused_l<7>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 8: return launch_fused_l<8>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 9: return launch_fused_l<9>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 10: return launch_fused_l<10>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 11: return launch_fused_l<11>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 12: return launch_fused_l<12>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 13: return launch_fused_l<13>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 14: return launch_fused_l<14>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    case 15: return launch_fused_l<15>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
    default: return launch_fused_l<16>(xbf, wq, sw, N, K, fmt, xq, sx, y, st);
  }
}

}  // namespace w8a8
