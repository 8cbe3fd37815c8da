// Few-token W8A8 GEMM (one token, where K does not suit the vector kernel) on gfx950: the same
// result as the tiled GEMM,
// y = bf16( s_x[m] s_w[n] sum_k dec(xq) dec(wq) ) for FP8 and
// y = bf16( fp32(fp32(acc_i32) s_x[m]) s_w[n] ) for INT8, but organised around streaming
// the weights once at HBM rate.
//
// Below the machine's ridge point the contraction does 2M flops per weight byte, so the
// time is the time to read W ("FP8 and INT8 Inference", arithmetic intensity and the
// decode regime; "FP8 and FP4 inference, SmoothQuant and activation quantization", the
// roofline of batch size). The kernel therefore spreads W over as many CUs and as many
// loads in flight as possible:
//  - one workgroup per 16 NW weight rows (NW = 1 at N = 4096: 256 workgroups, one per
//    CU; wider layers take 32 rows so that X is re-read fewer times);
//  - its WPB waves split K: wave w takes K steps w, w + WPB, ...; each wave keeps the
//    weights of the next 4 steps (2 KB each) and the X fragments of the next step in
//    flight while it computes;
//  - the contraction itself still runs on the matrix cores, with M padded to 16-row
//    subtiles (the matrix core is far faster than HBM here);
//  - the waves' partial sums meet in LDS, and the workgroup applies the scales.
//
// Operand layout. A 16x16x128 FP8 MFMA (or two 16x16x64 INT8 MFMAs) takes, for lane l,
// row l & 15 and 32 bytes of the 128-byte K step. Any assignment of K bytes to lanes
// gives the same sum as long as W and X use the same one, so lane group g = l >> 4 takes
// bytes [16g, 16g+16) and [64+16g, 64+16g+16): each 16-byte load instruction then reads
// one contiguous 64-byte half-row per row. INT8 sums are exact in any order, so the INT8
// result is bit-identical to the two-waves-per-SIMD kernel's.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace w8a8 {

template <int KIND, int MT, int WPB, int NW, bool OF8>
__global__ void __launch_bounds__(WPB * 64)
gemm_skinny_kernel(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                   const uint8_t* __restrict__ wq, const float* __restrict__ sw, int M, int N,
                   int K, int ksteps, void* __restrict__ yp, Epilogue ep) {
  typedef typename std::conditional<KIND == 1, i32x4, f32x4>::type acc_t;
  __shared__ __attribute__((aligned(16))) acc_t red[WPB][NW][MT][64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * NW;
  const uint8_t* wrowj[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) wrowj[j] = wq + (size_t)min(n0 + 16 * j + fr, N - 1) * K + 16 * g;
  const uint8_t* xrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) xrow[i] = xq + (size_t)min(16 * i + fr, M - 1) * K + 16 * g;

  acc_t acc[NW][MT];
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[j][i] = acc_t{};

  // K steps of this wave: ks = wave + WPB * s for s < cnt. The weights of a chunk of CH
  // steps are loaded a chunk ahead (two register buffers), the X fragments one step ahead,
  // so no MFMA waits on a load issued just before it. Loads past the last step re-read
  // the last step (in bounds; their products are never accumulated).
  const int cnt = (ksteps - wave + WPB - 1) / WPB;
  constexpr int CH = (4 / NW) > 2 ? (4 / NW) : 2;   // steps per weight chunk
  auto kofs = [&](int s) -> size_t { return (size_t)(wave + WPB * min(s, cnt - 1)) * 128; };
  auto load_w = [&](int s0, u32x4 (&lo)[CH][NW], u32x4 (&hi)[CH][NW]) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const uint8_t* p = wrowj[j] + kofs(s0 + c);
      lo[c][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      hi[c][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 64));
    }
  };
  auto load_x = [&](int s, u32x4 (&lo)[MT], u32x4 (&hi)[MT]) {
    const size_t kb = kofs(s);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      lo[i] = *reinterpret_cast<const u32x4*>(xrow[i] + kb);
      hi[i] = *reinterpret_cast<const u32x4*>(xrow[i] + kb + 64);
    }
  };
  auto mfma = [&](const u32x4 (&wlj)[NW], const u32x4 (&whj)[NW], const u32x4 (&xl)[MT], const u32x4 (&xh)[MT]) {
#pragma unroll
    for (int j = 0; j < NW; ++j)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const u32x4 wl = wlj[j], wh = whj[j];
      if constexpr (KIND == 1) {
        acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, wl), __builtin_bit_cast(i32x4, xl[i]), acc[j][i], 0, 0, 0);
        acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, wh), __builtin_bit_cast(i32x4, xh[i]), acc[j][i], 0, 0, 0);
      } else {
        const i32x8 a = {(int)wl.x, (int)wl.y, (int)wl.z, (int)wl.w, (int)wh.x, (int)wh.y, (int)wh.z, (int)wh.w};
        const i32x8 b = {(int)xl[i].x, (int)xl[i].y, (int)xl[i].z, (int)xl[i].w,
                         (int)xh[i].x, (int)xh[i].y, (int)xh[i].z, (int)xh[i].w};
        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j][i], 0, 0, 0, 0, 0, 0);
      }
    }
  };
  // One chunk: prefetch the next chunk's weights, then run CH steps with X one ahead.
  u32x4 xl0[MT], xh0[MT], xl1[MT], xh1[MT];
  auto chunk = [&](int s0, const u32x4 (&wl)[CH][NW], const u32x4 (&wh)[CH][NW], u32x4 (&nl)[CH][NW], u32x4 (&nh)[CH][NW]) {
    if (s0 + CH < cnt) load_w(s0 + CH, nl, nh);
#pragma unroll
    for (int c = 0; c < CH; c += 2) {
      load_x(s0 + c + 1, xl1, xh1);
      if (s0 + c < cnt) mfma(wl[c], wh[c], xl0, xh0);
      load_x(s0 + c + 2, xl0, xh0);
      if (s0 + c + 1 < cnt) mfma(wl[c + 1], wh[c + 1], xl1, xh1);
    }
  };
  if (cnt > 0) {
    u32x4 wl0[CH][NW], wh0[CH][NW], wl1[CH][NW], wh1[CH][NW];
    load_w(0, wl0, wh0);
    load_x(0, xl0, xh0);
    for (int s0 = 0; s0 < cnt; s0 += 2 * CH) {
      chunk(s0, wl0, wh0, wl1, wh1);
      if (s0 + CH < cnt) chunk(s0 + CH, wl1, wh1, wl0, wh0);
    }
  }

  // Partial sums of the WPB waves meet in LDS. In the 16x16 result, lane l holds output
  // row m = 16 i + (l & 15) and the four consecutive columns n0 + 4 (l >> 4) + r.
#pragma unroll
  for (int j = 0; j < NW; ++j)
#pragma unroll
  for (int i = 0; i < MT; ++i) red[wave][j][i][lane] = acc[j][i];
  __syncthreads();
  // The element loop is compiled per (activation, bias): no branch inside it.
  epi_dispatch(ep.act, ep.bias != nullptr, [&](auto act_c, auto bias_c) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool BIAS = decltype(bias_c)::value;
    for (int idx = threadIdx.x; idx < NW * MT * 64; idx += WPB * 64) {
      const int j = idx / (MT * 64), i = (idx >> 6) % MT, l = idx & 63;
      acc_t s = red[0][j][i][l];
#pragma unroll
      for (int w = 1; w < WPB; ++w) s += red[w][j][i][l];
      const int m = 16 * i + (l & 15), n = n0 + 16 * j + 4 * (l >> 4);
      if (m >= M || n >= N) continue;
      const float sm = sx[m];
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int nn = min(n + r, N - 1);
        const float swn = sw[nn];
        if constexpr (KIND == 1) v[r] = mul_rn(mul_rn((float)s[r], sm), swn);
        else v[r] = s[r] * (sm * swn);
        if constexpr (BIAS) v[r] = add_rn(v[r], bf16_lo(ep.bias[nn]));
        v[r] = epi_act<ACT>(v[r]);
      }
      if constexpr (OF8) {
        constexpr bool EX = (KIND == 1);
        const uint32_t o = pack_e4m3x4(epi_requant<EX>(v[0], ep.s_out, ep.inv_s_out), epi_requant<EX>(v[1], ep.s_out, ep.inv_s_out),
                                       epi_requant<EX>(v[2], ep.s_out, ep.inv_s_out), epi_requant<EX>(v[3], ep.s_out, ep.inv_s_out));
        uint8_t* yr = reinterpret_cast<uint8_t*>(yp) + (size_t)m * N;
        if ((N & 3) == 0) {
          *reinterpret_cast<uint32_t*>(yr + n) = o;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) yr[n + r] = (uint8_t)((o >> (8 * r)) & 0xFFu);
        }
      } else {
        uint16_t* yr = reinterpret_cast<uint16_t*>(yp) + (size_t)m * N;
        if ((N & 3) == 0) {
          const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *reinterpret_cast<u32x2*>(yr + n) = o;
        } else {
          const uint32_t o[2] = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) yr[n + r] = (uint16_t)((o[r >> 1] >> (16 * (r & 1))) & 0xFFFFu);
        }
      }
    }
  });
}

template <int KIND, int MT, int WPB, int NW>
static hipError_t launch_cfg(const void* xq, const float* sx, const void* wq, const float* sw,
                             int64_t M, int64_t N, int64_t K, void* y, hipStream_t st,
                             const Epilogue& ep) {
  const int blocks = (int)((N + 16 * NW - 1) / (16 * NW));
  if (ep.out_fp8) {
    hipLaunchKernelGGL((gemm_skinny_kernel<KIND, MT, WPB, NW, true>), dim3((unsigned)blocks),
                       dim3(WPB * 64), 0, st, (const uint8_t*)xq, sx, (const uint8_t*)wq, sw,
                       (int)M, (int)N, (int)K, (int)(K / 128), y, ep);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<KIND, MT, WPB, NW, false>), dim3((unsigned)blocks),
                       dim3(WPB * 64), 0, st, (const uint8_t*)xq, sx, (const uint8_t*)wq, sw,
                       (int)M, (int)N, (int)K, (int)(K / 128), y, ep);
  }
  return hipGetLastError();
}

// One token (the dispatcher sends this kernel only the one-token shapes whose K the vector
// kernel does not take): one 16-row subtile of M, 8 waves splitting K; wide layers take 32
// weight rows per workgroup so that X is re-read fewer times (a sweep on MI355X at K = 4096,
// N in {4096, 14336}).
template <int KIND>
static hipError_t launch_kind(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, void* y, hipStream_t st,
                              const Epilogue& ep) {
  if (M > 16) return hipErrorInvalidValue;
  return N > 8192 ? launch_cfg<KIND, 1, 8, 2>(xq, sx, wq, sw, M, N, K, y, st, ep)
                  : launch_cfg<KIND, 1, 8, 1>(xq, sx, wq, sw, M, N, K, y, st, ep);
}

hipError_t launch_gemm_skinny(const void* xq, const float* sx, const void* wq, const float* sw,
                              int64_t M, int64_t N, int64_t K, int fmt, void* y, hipStream_t st,
                              const Epilogue& ep) {
  if (fmt == 1) return launch_kind<1>(xq, sx, wq, sw, M, N, K, y, st, ep);
  return launch_kind<0>(xq, sx, wq, sw, M, N, K, y, st, ep);
}

}  // namespace w8a8
