// Device-side helpers shared by the gfx950 kernels of the W8A8 library.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace w8a8 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 halves of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Four fp32 -> four OCP E4M3FN bytes (v_cvt_pk_fp8_f32: round to nearest even). The
// hardware returns NaN instead of saturating for |v| >= 464; callers guarantee
// |v| <= 448 * (1 + 2^-23) (dynamic amax scaling), where both behaviours agree.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Quotient x / s (s > 0) from a per-row reciprocal rcp = 1/s (itself an IEEE division):
// one product and two FMA corrections, then the sign of x (an exact zero sum would
// otherwise come out as +0 for x = -0). It equals the IEEE fp32 quotient except where
// the residual underflows, i.e. only for |x / s| < 2^-11, where every FP8 and INT8 code
// is a zero of the same sign either way; this is checked exhaustively on the host over
// all bf16 x and all bf16-derived scales.
__device__ __forceinline__ float div_by_scale(float x, float s, float rcp) {
  float q0 = __fmul_rn(x, rcp);
  float r = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(r, rcp, q0), x);
}

// x / s for an arbitrary scale s in [2^-60, 2^60] (rcp = 1/s): the quotient above, except
// that an overflowing first product is kept (an infinite quotient, which saturates,
// instead of the NaN the correction would make of it).
__device__ __forceinline__ float div_static(float x, float s, float rcp) {
  const float q0 = __fmul_rn(x, rcp);
  return __builtin_isfinite(q0) ? div_by_scale(x, s, rcp) : q0;
}

// Round to nearest even and clamp to [-127, 127], as a byte.
__device__ __forceinline__ uint32_t int8_code(float v) {
  int i = (int)__builtin_rintf(v);       // v_rndne_f32 + v_cvt_i32_f32 (exact integer)
  i = max(-127, min(127, i));
  return (uint32_t)(i & 0xFF);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// |x| maximum over the 8 bf16 values of a 16-byte chunk.
__device__ __forceinline__ float chunk_absmax(u32x4 v) {
  float m = fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x)));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return m;
}

// An fp32 product and an fp32 sum, each rounded on its own. HIP compiles with contraction
// on, and its __fmul_rn / __fadd_rn are the plain operators, so a product followed by a
// sum could become one FMA (one rounding); these keep the two roundings the INT8
// epilogue's fixed order asks for.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// GEMM epilogue activation: 0 identity, 1 ReLU max(v, 0), 2 SiLU v / (1 + e^-v) (with the
// hardware exponential and reciprocal; SiLU is compared within a tolerance).
template <int ACT>
__device__ __forceinline__ float epi_act(float v) {
  if constexpr (ACT == 1) return fmaxf(v, 0.f);
  else if constexpr (ACT == 2) return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
  else return v;
}
__device__ __forceinline__ float epi_activate(float v, int act) {
  if (act == 1) return epi_act<1>(v);
  if (act == 2) return epi_act<2>(v);
  return v;
}

// Calls f(integral_constant<int, act>, integral_constant<bool, bias>) once, so that an
// epilogue's element loop is compiled per (activation, bias) with no branch inside it.
template <class F>
__device__ __forceinline__ void epi_dispatch(int act, bool bias, F&& f) {
  using A0 = std::integral_constant<int, 0>;
  using A1 = std::integral_constant<int, 1>;
  using A2 = std::integral_constant<int, 2>;
  if (bias) {
    if (act == 1) f(A1{}, std::true_type{});
    else if (act == 2) f(A2{}, std::true_type{});
    else f(A0{}, std::true_type{});
  } else {
    if (act == 1) f(A1{}, std::false_type{});
    else if (act == 2) f(A2{}, std::false_type{});
    else f(A0{}, std::false_type{});
  }
}

// Sum of v over the 64 lanes of the wave, in lane 63, by DPP moves: pairs and quads
// (quad_perm), the 16 lanes of a row (row_ror 4, 8), then rows 0 + 1 and 2 + 3 (row_bcast15
// into rows 1 and 3) and all four (row_bcast31 into rows 2 and 3). A lane of a row that the
// row mask leaves out adds 0. Integer sums are exact.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_moved(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, false);
}
template <class T>
__device__ __forceinline__ T wave_sum_dpp(T v) {
  auto step = [](T a, int moved) {
    if constexpr (std::is_same<T, float>::value) return a + __int_as_float(moved);
    else return a + moved;
  };
  auto bits = [](T a) {
    if constexpr (std::is_same<T, float>::value) return __float_as_int(a);
    else return a;
  };
  v = step(v, dpp_moved<0xB1, 0xF>(bits(v)));     // quad_perm [1, 0, 3, 2]
  v = step(v, dpp_moved<0x4E, 0xF>(bits(v)));     // quad_perm [2, 3, 0, 1]
  v = step(v, dpp_moved<0x124, 0xF>(bits(v)));    // row_ror 4
  v = step(v, dpp_moved<0x128, 0xF>(bits(v)));    // row_ror 8
  v = step(v, dpp_moved<0x142, 0xA>(bits(v)));    // row_bcast15
  v = step(v, dpp_moved<0x143, 0xC>(bits(v)));    // row_bcast31
  return v;
}

// clamp(q, +-448); a NaN stays NaN (both comparisons are false).
__device__ __forceinline__ float clamp448(float q) {
  return q > 448.f ? 448.f : (q < -448.f ? -448.f : q);
}

// Requantization for an FP8 output, clamp(v / s, +-448). EXACT: the IEEE fp32 division
// (the INT8 operand path, whose outputs are bit-exact); otherwise the product with the
// fp32 reciprocal inv = 1/s (FP8 operands, whose outputs are compared within a tolerance).
template <bool EXACT>
__device__ __forceinline__ float epi_requant(float v, float s, float inv) {
  return clamp448(EXACT ? v / s : v * inv);
}

// max(amax, 1e-8) / qmax with a NaN amax passed through (all-NaN row).
__device__ __forceinline__ float amax_scale(float amax, float qmax) {
  float a = (amax != amax) ? amax : fmaxf(amax, 1e-8f);
  return a / qmax;                      // IEEE fp32 division
}

}  // namespace w8a8
