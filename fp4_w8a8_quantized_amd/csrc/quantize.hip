// Quantization kernels for gfx950: per-row (per-token / per-output-channel) FP8 E4M3FN and
// INT8, 1x128 activation groups, 128x128 weight blocks, and MXFP4 (E2M1 + E8M0 per 32).
//
// Definitions follow the pages' emulation of per-token FP8 quantization
// ("FP8 and FP4 inference, SmoothQuant and activation quantization", Implementation
// sketch), the symmetric INT8 rule ("Low-bit LLM Weights and Activations" §2.1) and the
// block formats (same page §2.4; "FP8 and INT8 Inference" §5, What DeepSeek did).
//
// All kernels are HBM-bound codecs: 16-byte coalesced loads of bf16, the row (or group,
// or block) amax kept in registers, codes written from registers with coalesced stores.
// The bf16 input is read once (non-temporal loads); the codes are stored with ordinary
// stores, so that the GEMM that reads them next finds them in the caches. Written
// non-temporally the per-token quantizer alone ran 6% faster at 2048 x 4096, but the
// prefill step (quantize + GEMM per linear) 2-3% slower.
#include "common.h"
#include "internal.h"

namespace w8a8 {

// ---------------------------------------------------------------------------------------
// Per-row quantization: one 256-thread block per row; thread t owns the 16-byte chunks
// t, t+256, ... (CH of them), so a row of up to 2048*CH elements stays in registers
// between the amax reduction and the encode.
template <int CH, bool INT8>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x,
                                                         int64_t K, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int nchunk = (int)(K >> 3);
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * K);
  u32x4 v[CH];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = t + i * 256;
    v[i] = (c < nchunk) ? __builtin_nontemporal_load(xr + c) : u32x4{0u, 0u, 0u, 0u};
    amax = fmaxf(amax, chunk_absmax(v[i]));
  }
  amax = wave_max(amax);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax_scale(amax, INT8 ? 127.0f : 448.0f);
  if (t == 0) scale[row] = s;
  const bool finite = __builtin_isfinite(s);
  const float rcp = 1.0f / s;
  u32x2* qr = reinterpret_cast<u32x2*>(q + row * K);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = t + i * 256;
    if (c >= nchunk) break;
    float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                  bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = finite ? div_by_scale(f[e], s, rcp) : f[e] / s;
    u32x2 o;
    if (INT8) {
      o.x = int8_code(f[0]) | (int8_code(f[1]) << 8) | (int8_code(f[2]) << 16) | (int8_code(f[3]) << 24);
      o.y = int8_code(f[4]) | (int8_code(f[5]) << 8) | (int8_code(f[6]) << 16) | (int8_code(f[7]) << 24);
    } else {
      o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
      o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
    }
    qr[c] = o;
  }
}

// Rows longer than 16384 elements: two passes over the row (amax, then encode).
template <bool INT8>
__global__ __launch_bounds__(256) void quant_rows_long_kernel(const uint16_t* __restrict__ x,
                                                              int64_t K, uint8_t* __restrict__ q,
                                                              float* __restrict__ scale) {
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int64_t nchunk = K >> 3;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + row * K);
  float amax = 0.0f;
  for (int64_t c = t; c < nchunk; c += 256) amax = fmaxf(amax, chunk_absmax(xr[c]));
  amax = wave_max(amax);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax_scale(amax, INT8 ? 127.0f : 448.0f);
  if (t == 0) scale[row] = s;
  const bool finite = __builtin_isfinite(s);
  const float rcp = 1.0f / s;
  u32x2* qr = reinterpret_cast<u32x2*>(q + row * K);
  for (int64_t c = t; c < nchunk; c += 256) {
    const u32x4 v = xr[c];
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = finite ? div_by_scale(f[e], s, rcp) : f[e] / s;
    u32x2 o;
    if (INT8) {
      o.x = int8_code(f[0]) | (int8_code(f[1]) << 8) | (int8_code(f[2]) << 16) | (int8_code(f[3]) << 24);
      o.y = int8_code(f[4]) | (int8_code(f[5]) << 8) | (int8_code(f[6]) << 16) | (int8_code(f[7]) << 24);
    } else {
      o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
      o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
    }
    qr[c] = o;
  }
}

template <bool INT8>
static hipError_t launch_rows(const uint16_t* x, int64_t R, int64_t K, uint8_t* q, float* s,
                              hipStream_t st) {
  const int64_t nchunk = K >> 3;
  const int ch = (int)((nchunk + 255) / 256);
  dim3 grid((unsigned)R), block(256);
  switch (ch) {
    case 0:
    case 1: hipLaunchKernelGGL((quant_rows_kernel<1, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 2: hipLaunchKernelGGL((quant_rows_kernel<2, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 3: hipLaunchKernelGGL((quant_rows_kernel<3, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 4: hipLaunchKernelGGL((quant_rows_kernel<4, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 5: hipLaunchKernelGGL((quant_rows_kernel<5, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 6: hipLaunchKernelGGL((quant_rows_kernel<6, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 7: hipLaunchKernelGGL((quant_rows_kernel<7, INT8>), grid, block, 0, st, x, K, q, s); break;
    case 8: hipLaunchKernelGGL((quant_rows_kernel<8, INT8>), grid, block, 0, st, x, K, q, s); break;
    default: hipLaunchKernelGGL((quant_rows_long_kernel<INT8>), grid, block, 0, st, x, K, q, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const void* x, int64_t R, int64_t K, int fmt, void* q,
                                float* scale, hipStream_t st) {
  if (fmt == 1)
    return launch_rows<true>((const uint16_t*)x, R, K, (uint8_t*)q, scale, st);
  return launch_rows<false>((const uint16_t*)x, R, K, (uint8_t*)q, scale, st);
}

// ---------------------------------------------------------------------------------------
// 1x128 groups: 16-byte chunks, 16 consecutive lanes form a group. Groups never straddle
// rows (K % 128 == 0), so the group index is the linear chunk index / 16, which is also the
// row-major index into sx [M, K/128]. Thread t of workgroup b encodes the chunks
// b * 256 * CH + t + 256 i, i < CH, whose loads are all issued first.
template <int CH>
__global__ __launch_bounds__(256) void quant_group_kernel(const uint16_t* __restrict__ x,
                                                          int64_t nchunk, uint8_t* __restrict__ q,
                                                          float* __restrict__ sx) {
  const int64_t c0 = (int64_t)blockIdx.x * (256 * CH) + threadIdx.x;
  u32x4 vs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = c0 + 256 * i;
    vs[i] = c < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + c)
                       : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = c0 + 256 * i;
    const u32x4 v = vs[i];
    float amax = chunk_absmax(v);
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kWave));
    const float s = amax_scale(amax, 448.0f);
    if (c >= nchunk) break;                        // the chunks past the end are the lane's last
    if ((threadIdx.x & 15) == 0) sx[c >> 4] = s;
    const bool finite = __builtin_isfinite(s);
    const float rcp = 1.0f / s;
    float f[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                  bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = finite ? div_by_scale(f[e], s, rcp) : f[e] / s;
    u32x2 o;
    o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
    o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
    reinterpret_cast<u32x2*>(q)[c] = o;
  }
}

template <int CH>
void launch_group_ch(const void* x, int64_t nchunk, void* q, float* sx, hipStream_t st) {
  dim3 grid((unsigned)((nchunk + 256 * CH - 1) / (256 * CH))), block(256);
  hipLaunchKernelGGL((quant_group_kernel<CH>), grid, block, 0, st, (const uint16_t*)x, nchunk,
                     (uint8_t*)q, sx);
}

hipError_t launch_quantize_group(const void* x, int64_t M, int64_t K, void* q, float* sx,
                                 hipStream_t st) {
  const int64_t nchunk = (M * K) >> 3;
  launch_group_ch<2>(x, nchunk, q, sx, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// 128x128 weight blocks: one 256-thread block per (row block, K block). The block's
// 128 rows x 16 chunks live in registers (8 chunks per thread) between the two passes.
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ w,
                                                          int64_t N, int64_t K,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ sw) {
  const int64_t kb = blockIdx.x, nb = blockIdx.y;
  const int64_t KB = K >> 7;
  const int t = threadIdx.x;
  u32x4 v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + i * 256;            // 0..2047
    const int64_t r = nb * 128 + (c >> 4);
    const int64_t col = kb * 128 + (c & 15) * 8;
    v[i] = (r < N) ? *reinterpret_cast<const u32x4*>(w + r * K + col) : u32x4{0u, 0u, 0u, 0u};
    amax = fmaxf(amax, chunk_absmax(v[i]));
  }
  amax = wave_max(amax);
  __shared__ float red[4];
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax_scale(amax, 448.0f);
  if (t == 0) sw[nb * KB + kb] = s;
  const bool finite = __builtin_isfinite(s);
  const float rcp = 1.0f / s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + i * 256;
    const int64_t r = nb * 128 + (c >> 4);
    if (r >= N) continue;
    const int64_t col = kb * 128 + (c & 15) * 8;
    float f[8] = {bf16_lo(v[i].x), bf16_hi(v[i].x), bf16_lo(v[i].y), bf16_hi(v[i].y),
                  bf16_lo(v[i].z), bf16_hi(v[i].z), bf16_lo(v[i].w), bf16_hi(v[i].w)};
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = finite ? div_by_scale(f[e], s, rcp) : f[e] / s;
    u32x2 o;
    o.x = pack_e4m3x4(f[0], f[1], f[2], f[3]);
    o.y = pack_e4m3x4(f[4], f[5], f[6], f[7]);
    *reinterpret_cast<u32x2*>(q + r * K + col) = o;
  }
}

hipError_t launch_quantize_block(const void* w, int64_t N, int64_t K, void* q, float* sw,
                                 hipStream_t st) {
  dim3 grid((unsigned)(K >> 7), (unsigned)((N + 127) >> 7)), block(256);
  hipLaunchKernelGGL(quant_block_kernel, grid, block, 0, st, (const uint16_t*)w, N, K,
                     (uint8_t*)q, sw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// MXFP4: 16-byte chunks (8 elements), four consecutive lanes form a 32-element block. Scale exponent e = floor(log2 amax) - 2 (E2M1's top binade is 2^2),
// clamped to [-127, 127], 0 for an all-zero block; elements x * 2^-e (exact) are
// rounded to E2M1 half-to-even and saturated to +-6. A block holding an infinity or a NaN
// gets the E8M0 NaN code 0xFF (the OCP MX format's one special scale value; the pages name
// the E8M0 scale but not its special value) and element codes 0, so it decodes to NaN: E2M1
// itself has no non-finite values.
// Thread t of workgroup b encodes the chunks b * 256 * CH + t + 256 i, i < CH, whose loads
// are all issued first; lanes 4j .. 4j + 3 hold the four chunks of one block.
template <int CH>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t* __restrict__ x,
                                                          int64_t nchunk, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ sc) {
  const int64_t c0 = (int64_t)blockIdx.x * (256 * CH) + threadIdx.x;
  u32x4 vs[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = c0 + 256 * i;
    vs[i] = c < nchunk ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x) + c)
                       : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int64_t c = c0 + 256 * i;
    const u32x4 v = vs[i];
    float amax = chunk_absmax(v);
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    // non-finite bf16: all exponent bits set
    int bad = 0;
    for (const uint32_t h : {v.x, v.y, v.z, v.w})
      bad |= (h & 0x7F80u) == 0x7F80u || (h & 0x7F800000u) == 0x7F800000u;
    bad |= __shfl_xor(bad, 1, kWave);
    bad |= __shfl_xor(bad, 2, kWave);
    if (c >= nchunk) break;                        // the chunks past the end are the lane's last
    int e = 0;
    if (amax > 0.0f && !bad) {
      e = __builtin_amdgcn_frexp_expf(amax) - 1 - 2;   // floor(log2 amax) - 2
      e = max(-127, min(127, e));
    }
    if ((threadIdx.x & 3) == 0) sc[c >> 2] = bad ? (uint8_t)0xFF : (uint8_t)(e + 127);
    // gfx950's converter divides each bf16 of a pair by the scale's power of two (only the
    // scale's exponent field is read: 2^e is passed as the fp32 pattern (e + 127) << 23),
    // rounds half to even onto the E2M1 grid and saturates at 6, element 2i to the low
    // nibble. The inputs' sign bits are ORed back in, so that values rounding to zero keep
    // their sign (a no-op wherever the converter already keeps it).
    const float scl = __uint_as_float((uint32_t)(e + 127) << 23);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out = 0, sgn = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2, w[0]), scl, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2, w[1]), scl, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2, w[2]), scl, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(out, __builtin_bit_cast(bf16x2, w[3]), scl, 3);
#pragma unroll
    for (int k = 0; k < 4; ++k) sgn |= (((w[k] >> 12) & 0x8u) | ((w[k] >> 24) & 0x80u)) << (8 * k);
    reinterpret_cast<uint32_t*>(q)[c] = bad ? 0u : out | sgn;
  }
}

template <int CH>
void launch_mx_ch(const void* x, int64_t nchunk, void* q, uint8_t* sc, hipStream_t st) {
  dim3 grid((unsigned)((nchunk + 256 * CH - 1) / (256 * CH))), block(256);
  hipLaunchKernelGGL((quant_mxfp4_kernel<CH>), grid, block, 0, st, (const uint16_t*)x, nchunk,
                     (uint8_t*)q, sc);
}

hipError_t launch_quantize_mxfp4(const void* x, int64_t R, int64_t K, void* q, uint8_t* sc,
                                 hipStream_t st) {
  // Two chunks per thread, four from 2^23 chunks up (8192 x 8192: 35.7 us at one, 30.1 at
  // two, 29.4 at four, 33.0 at eight; 4096 x 7168: 17.0, 15.0, 15.4, 17.1 us).
  const int64_t nchunk = (R * K) >> 3;
  if (nchunk >= ((int64_t)1 << 23)) launch_mx_ch<4>(x, nchunk, q, sc, st);
  else launch_mx_ch<2>(x, nchunk, q, sc, st);
  return hipGetLastError();
}

}  // namespace w8a8
