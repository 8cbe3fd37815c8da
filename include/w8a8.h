/*
 * w8a8.h - C ABI of the MI355X (gfx950) W8A8 / block-scaled FP8 / INT8 / MXFP4 / NVFP4 / W4A16
 * library.
 *
 * The calls follow the problem statement of three pages:
 *   [P-FP8FP4]  "FP8 and FP4 inference, SmoothQuant and activation quantization"
 *   [P-FP8INT8] "FP8 and INT8 Inference"
 *   [P-LOWBIT]  "Low-bit LLM Weights and Activations"
 * A quantized linear layer computes Y = X W^T as diag(s_X) (X_q W_q^T) diag(s_W): the
 * operands are quantized to 8-bit (or 4-bit) codes with one scale per token (row of X)
 * and one per output channel (row of W), the contraction runs in low precision with
 * FP32 (INT32 for INT8) accumulation, and the scales are applied after the reduction
 * ([P-FP8FP4] "Scale granularity"; [P-LOWBIT] §3.4).
 *
 * Conventions shared by every call:
 *  - Layouts are row-major. X is [M, K] (tokens x in-features), W is [N, K] (out x in,
 *    the layout of a PyTorch Linear weight), Y is [M, N]. K is contiguous in X and W.
 *  - bf16 means IEEE bfloat16 bit patterns (2 bytes); E4M3FN means OCP FP8 E4M3FN
 *    bytes (max 448, NaN 0x7F/0xFF); E2M1 codes are packed two per byte, element 2i in
 *    the low nibble; E8M0 scales are bytes whose value is 2^(c - 127).
 *  - Array arguments are device pointers that the caller allocated and owns, except
 *    where a comment says "host". The library keeps no pointer after a call returns,
 *    allocates no memory, holds no mutable global state and is re-entrant.
 *  - Device pointers must be 16-byte aligned. Inputs and outputs must not overlap.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream. Calls are
 *    asynchronous: they enqueue kernels and return; outputs are valid once the stream
 *    has synchronized.
 *  - Every argument check runs on the host before anything is enqueued. On a non-zero
 *    status nothing has been enqueued and no output has been written.
 *  - A dimension of 0 rows (M, N or R) is valid and enqueues nothing.
 *  - No operand (codes, bf16 input) may exceed 2^31 bytes, and M, N < 2^30: the kernels
 *    address one matrix with 32-bit byte offsets. Larger shapes return W8A8_ERR_SHAPE;
 *    split them along M or N.
 *  - Non-finite inputs are outside the contract: the kernels do not fault on them, a
 *    NaN element encodes to a NaN code, and a scale computed from an infinite amax is
 *    infinite.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL = 1,        /* a required pointer is NULL                              */
  W8A8_ERR_SHAPE = 2,       /* a dimension is negative, or an operand is too large     */
  W8A8_ERR_UNSUPPORTED = 3, /* K is not a multiple of the call's granule, bad format   */
  W8A8_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned                 */
  W8A8_ERR_HIP = 5,         /* the HIP runtime reported an error when enqueuing        */
  W8A8_ERR_ARG = 6          /* a scalar argument is out of range (e.g. alpha, mode)    */
} w8a8_status;

typedef enum {
  W8A8_FMT_E4M3FN = 0,      /* OCP FP8 E4M3FN codes, FP32 accumulation                 */
  W8A8_FMT_INT8 = 1         /* symmetric INT8 codes in [-127, 127], INT32 accumulation */
} w8a8_format;

/* Human-readable name of a status code (static string; never NULL). */
const char* w8a8_status_string(int status);

/* ------------------------------------------------------------------------------------
 * Per-token dynamic activation quantization ([P-FP8FP4] "Implementation sketch",
 * fp8_per_token; [P-FP8INT8] §5 "INT8 in practice": activations per-token, dynamic).
 *
 * For each row m of x_bf16 [M, K]:
 *   amax = max_k |x[m,k]|
 *   E4M3FN: s[m] = fp32(max(amax, 1e-8)) / 448   q[m,k] = e4m3_rne_sat(x[m,k] / s[m])
 *   INT8:   s[m] = fp32(max(amax, 1e-8)) / 127   q[m,k] = clamp(rne(x[m,k] / s[m]), +-127)
 * Both divisions are IEEE fp32 divisions rounded to nearest even; the E4M3FN encode
 * rounds to nearest even and saturates to +-448 (0x7E / 0xFE); zeros keep their sign.
 *   q:     [M, K] bytes (E4M3FN codes or int8)      scale: fp32 [M]
 * K must be a multiple of 16. Returns W8A8_ERR_UNSUPPORTED otherwise.
 */
w8a8_status w8a8_quantize_per_token(const void* x_bf16, int64_t M, int64_t K, int fmt,
                                    void* q, float* scale, void* stream);

/* Per-output-channel weight quantization: exactly the per-token rule applied to the
 * rows of w_bf16 [N, K] (one scale per output channel; [P-FP8FP4] "Scale granularity",
 * [P-FP8INT8] §5: weights per-channel, static). Done once, offline.
 *   q: [N, K] bytes    scale: fp32 [N]    K % 16 == 0. */
w8a8_status w8a8_quantize_weight_per_channel(const void* w_bf16, int64_t N, int64_t K, int fmt,
                                             void* q, float* scale, void* stream);

/* ------------------------------------------------------------------------------------
 * W8A8 GEMM with the fused scale epilogue ([P-FP8INT8] §5 and the epilogue of §6-9;
 * [P-LOWBIT] §3.4 and §4.3):
 *   E4M3FN: y[m,n] = bf16_rne( s_x[m] * s_w[n] * sum_k dec(xq[m,k]) * dec(wq[n,k]) ),
 *           products and sums in FP32 (the summation order is unspecified).
 *   INT8:   acc = sum_k xq[m,k] * wq[n,k] exactly in INT32;
 *           y[m,n] = bf16_rne( fp32( fp32(acc) * s_x[m] ) * s_w[n] ), bit-exact.
 *   xq [M, K], wq [N, K] codes; sx fp32 [M]; sw fp32 [N]; y_bf16 [M, N].
 * K must be a multiple of 128 (W8A8_ERR_UNSUPPORTED otherwise); K = 0 is not allowed.
 */
w8a8_status w8a8_gemm(const void* xq, const float* sx, const void* wq, const float* sw,
                      int64_t M, int64_t N, int64_t K, int fmt, void* y_bf16, void* stream);

/* ------------------------------------------------------------------------------------
 * One W8A8 linear layer on bf16 activations: the per-token quantization of
 * w8a8_quantize_per_token followed by the scaled GEMM of w8a8_gemm, as the pages run a
 * quantized linear ([P-FP8FP4] Implementation sketch: fp8_per_token on the activations, the
 * weights quantized offline, the scaled matrix product; [P-FP8INT8] §6-9 for the GEMM).
 *   x_bf16 [M, K] bf16 activations (read only);
 *   wq [N, K] weight codes and sw fp32 [N], from w8a8_quantize_weight_per_channel;
 *   xq [M, K] codes and sx fp32 [M]: written, exactly what w8a8_quantize_per_token gives;
 *   y_bf16 [M, N]: written, exactly what w8a8_gemm gives for (xq, sx, wq, sw).
 * One token (M = 1) with K a multiple of 1024 up to 16384 runs as one kernel that quantizes
 * the row and computes the GEMM (no quantizer launch); other shapes run the two kernels in
 * order on the stream. All pointers are device memory owned by the caller, 16-byte aligned;
 * x must not overlap xq, sx or y. Rules and errors as w8a8_gemm (K a multiple of 128, both
 * formats), plus those of the quantizer for x; with M = 0 or N = 0 nothing is written.
 */
w8a8_status w8a8_linear(const void* x_bf16, const void* wq, const float* sw, int64_t M, int64_t N,
                        int64_t K, int fmt, void* xq, float* sx, void* y_bf16, void* stream);

typedef enum {
  W8A8_ACT_NONE = 0,        /* identity                                                */
  W8A8_ACT_RELU = 1,        /* max(v, 0)                                               */
  W8A8_ACT_SILU = 2         /* v * sigmoid(v) = v / (1 + exp(-v))                      */
} w8a8_activation;

typedef enum {
  W8A8_OUT_BF16 = 0,        /* bf16 [M, N]                                             */
  W8A8_OUT_E4M3FN = 1       /* E4M3FN bytes [M, N], requantized with a static scale    */
} w8a8_output;

/* ------------------------------------------------------------------------------------
 * W8A8 GEMM with the whole epilogue of [P-FP8INT8] §6-9 ("Under the hood", the FP8 GEMM
 * epilogue), for the next layer's input:
 *   v = the dequantized sum of w8a8_gemm (same arithmetic, before its bf16 rounding)
 *   v = v + bias[n]                 if bias_bf16 != NULL (bf16 [N], widened exactly)
 *   v = act(v)                      act is a w8a8_activation
 *   BF16 output:    y[m,n] = bf16_rne(v)                                    y: bf16 [M, N]
 *   E4M3FN output:  y[m,n] = e4m3_rne(clamp(v / out_scale, -448, 448))      y: bytes [M, N]
 * With INT8 operands v is fp32(fp32(fp32(acc) s_x[m]) s_w[n]), the bias add is one fp32
 * addition and the division an IEEE fp32 division, so the outputs are bit-exact for
 * W8A8_ACT_NONE and W8A8_ACT_RELU. With E4M3FN operands (whose sums are order-free) the
 * division is a product with fp32(1 / out_scale). SiLU uses the hardware exponential and
 * reciprocal.
 * out_scale (the static per-tensor scale of the next layer's input) must be finite and
 * > 0 for E4M3FN output and is ignored for BF16. A bad act, out_fmt or fmt returns
 * W8A8_ERR_UNSUPPORTED, a bad out_scale W8A8_ERR_ARG; other rules as w8a8_gemm.
 * bias_bf16, when given, is a 16-byte aligned device array of N bf16 values.
 */
w8a8_status w8a8_gemm_ex(const void* xq, const float* sx, const void* wq, const float* sw,
                         int64_t M, int64_t N, int64_t K, int fmt, const void* bias_bf16,
                         int act, int out_fmt, float out_scale, void* y, void* stream);

/* ------------------------------------------------------------------------------------
 * Static per-tensor activation quantization with a saturation monitor ([P-FP8INT8] §5
 * "FP8 in practice": x_fp8 = clamp(x / s, -448, 448); [P-FP8FP4] "Failure modes and how
 * to detect them": log the fraction of saturated values per layer).
 *   E4M3FN: q = e4m3_rne(clamp(x / s, -448, 448));  saturated if |x / s| > 448
 *   INT8:   q = clamp(rne(x / s), +-127);            saturated if |rne(x / s)| > 127
 * x / s is an IEEE fp32 division; s = scale[0] is read on the device (so that a scale
 * produced by w8a8_delayed_scale_update needs no host round trip).
 *   x_bf16 [M, K]; q [M, K] bytes; K % 8 == 0.
 *   saturated (may be NULL): one uint32 to which the number of saturated elements is
 *     added (atomically; the caller zeroes it when a new count should start).
 *   amax (may be NULL): one float, set to max(amax, max |x|) (atomically; NaN elements
 *     are ignored; it must hold a value >= 0 before the call).
 * scale, saturated and amax need only 4-byte alignment. NaN elements encode to a NaN
 * code (E4M3FN) or 0 (INT8) and are not counted.
 */
w8a8_status w8a8_quantize_static(const void* x_bf16, int64_t M, int64_t K, int fmt,
                                 const float* scale, void* q, uint32_t* saturated,
                                 float* amax, void* stream);

/* Delayed scaling ([P-FP8INT8] §5 "FP8 in practice": the scale comes from a history of
 * recent amax values, avoiding a synchronization). On the device, in stream order:
 *   amax_history[step mod H] = *amax;  *amax = 0;
 *   *scale = fp32(max(max_i amax_history[i], 1e-8)) / qmax     (qmax 448 or 127 by fmt)
 * amax_history: float [H], 1 <= H <= 2^24, caller-initialised (e.g. with calibration
 * amax values). Run once per step after w8a8_quantize_static; the next step's quantize
 * then reads the new scale. All pointers 4-byte aligned device pointers; step >= 0.
 */
w8a8_status w8a8_delayed_scale_update(float* amax_history, int64_t H, float* amax, int64_t step,
                                      int fmt, float* scale, void* stream);

/* ------------------------------------------------------------------------------------
 * DeepSeek-V3-style fine-grained FP8 ([P-FP8INT8] §5 "What DeepSeek did" and "The
 * blockwise/fine-grained trend"; [P-FP8FP4] "Scale granularity").
 *
 * 1x128 activation groups: each run of 128 elements along K gets its own scale,
 *   sx[m, g] = fp32(max(amax_{m,g}, 1e-8)) / 448, codes as in w8a8_quantize_per_token.
 *   xq: [M, K] E4M3FN    sx: fp32 [M, K/128] (row-major)    K % 128 == 0.
 */
w8a8_status w8a8_quantize_per_token_group(const void* x_bf16, int64_t M, int64_t K,
                                          void* xq, float* sx, void* stream);

/* 128x128 weight blocks: one scale per (block of 128 output rows, block of 128 K).
 *   wq: [N, K] E4M3FN    sw: fp32 [ceil(N/128), K/128]    K % 128 == 0.
 * The last row block is partial when N % 128 != 0. */
w8a8_status w8a8_quantize_weight_block(const void* w_bf16, int64_t N, int64_t K,
                                       void* wq, float* sw, void* stream);

/* Block-scaled FP8 GEMM with FP32 promotion once per 128-wide K group:
 *   y[m,n] = bf16_rne( sum_g sx[m,g] * sw[n/128, g] * (sum_{k in g} dec(xq) dec(wq)) ),
 * the inner sum in FP32 from zero for each group, the outer running sum in FP32.
 * K % 128 == 0. */
w8a8_status w8a8_gemm_blockscaled(const void* xq, const float* sx, const void* wq,
                                  const float* sw, int64_t M, int64_t N, int64_t K,
                                  void* y_bf16, void* stream);

/* ------------------------------------------------------------------------------------
 * MXFP4 ([P-LOWBIT] §2.4: E2M1 elements, one E8M0 power-of-two scale per 32 elements,
 * 4.25 bits per weight; [P-FP8FP4] "Where it came from").
 *
 * Quantize the rows of any bf16 [R, K] matrix (activations or weights), per 32-element
 * block along K: amax of the block; e = floor(log2(amax)) - 2 clamped to [-127, 127]
 * (0 for an all-zero block); scale code e + 127; elements x / 2^e rounded to E2M1 with
 * round-to-nearest-even and saturation to +-6.
 *   q_packed: [R, K/2] bytes    scale_e8m0: [R, K/32] bytes    K % 32 == 0.
 */
w8a8_status w8a8_quantize_mxfp4(const void* x_bf16, int64_t R, int64_t K, void* q_packed,
                                uint8_t* scale_e8m0, void* stream);

/* MXFP4 x MXFP4 GEMM on the gfx950 block-scaled matrix cores:
 *   y[m,n] = bf16_rne( sum_b 2^(ex[m,b]-127) 2^(ew[n,b]-127) sum_{k in b} dec(xq) dec(wq) ),
 *   accumulated in FP32. xq [M, K/2], wq [N, K/2] packed; sx [M, K/32]; sw [N, K/32].
 * K % 256 == 0. */
w8a8_status w8a8_gemm_mxfp4(const void* xq, const uint8_t* sx, const void* wq,
                            const uint8_t* sw, int64_t M, int64_t N, int64_t K,
                            void* y_bf16, void* stream);

/* ------------------------------------------------------------------------------------
 * NVFP4 ([P-FP8FP4] "Implementation sketch", the `nvfp4` emulation, and the measured-model
 * section; [P-LOWBIT] §2.4: E2M1 elements, one E4M3 scale per 16 elements, 4.5 bits per
 * element, plus one fp32 scale per tensor).
 *
 * Quantize the rows of a bf16 [R, K] matrix (activations or weights):
 *   g = amax(|x| over the whole matrix) / 2688 (2688 = 448 * 6; g = 1 for an all-zero
 *       matrix), or the caller's g;
 *   per 16-element block b along K: code_b = E4M3FN((amax_b / 6) / g) (IEEE fp32 divisions
 *       in that order, round to nearest even, saturating at 448);
 *   s_b = dec(code_b) * g in fp32, replaced by 1 where it is 0;
 *   element code = E2M1(x / s_b) (IEEE fp32 quotient, nearest even, saturating at +-6).
 *   q_packed: [R, K/2] bytes (element 2i in the low nibble)   scale_e4m3: [R, K/16] bytes
 *   g: one fp32 on the device (4-byte aligned).               K % 16 == 0.
 * scale_mode W8A8_NVFP4_SCALE_COMPUTE computes g from x and writes it to *g (the slot holds
 * the running amax while the call's kernels run); W8A8_NVFP4_SCALE_GIVEN reads *g, which
 * must be finite and positive (it is not checked: it lives on the device). R == 0 or
 * K == 0 writes nothing. Any other scale_mode is W8A8_ERR_UNSUPPORTED.
 */
typedef enum { W8A8_NVFP4_SCALE_COMPUTE = 0, W8A8_NVFP4_SCALE_GIVEN = 1 } w8a8_nvfp4_scale_mode;
w8a8_status w8a8_quantize_nvfp4(const void* x_bf16, int64_t R, int64_t K, int scale_mode,
                                void* q_packed, uint8_t* scale_e4m3, float* g, void* stream);

/* NVFP4 x NVFP4 GEMM:
 *   y[m,n] = bf16_rne( sum_b s_x[m,b] s_w[n,b] sum_{k in b} dec(xq[m,k]) dec(wq[n,k]) )
 * with s as above (from the scale codes and gx / gw, each one fp32 on the device),
 * accumulated in FP32. The operands are dequantized to fp16 (element times dec(code_b),
 * exact) and contracted on the fp16 matrix cores; gx gw is applied after the reduction.
 * Two cases differ from the definition by fp32 rounding only: a block whose scale code is
 * 0 uses 1/g rounded to fp16, and a g small enough (below about 2^-117) that dec * g is
 * an fp32 subnormal.
 *   xq [M, K/2], wq [N, K/2] packed; sx [M, K/16], sw [N, K/16] E4M3 codes.  K % 64 == 0.
 */
w8a8_status w8a8_gemm_nvfp4(const void* xq, const uint8_t* sx, const float* gx, const void* wq,
                            const uint8_t* sw, const float* gw, int64_t M, int64_t N, int64_t K,
                            void* y_bf16, void* stream);

/* ------------------------------------------------------------------------------------
 * W4A16 weight-only decode path ([P-LOWBIT] §2.3: symmetric INT4, q in [-7, 7],
 * S = max|x| / 7 per group of 128 along K, 2 bytes of scale per group; §3.3: weights
 * unpacked and dequantized next to a 16-bit product, activations stay 16-bit).
 *
 * Quantize a bf16 weight matrix [N, K] per group of 128 along K:
 *   S = fp16_rne(fp32(amax) / 7) (1 for an all-zero group; 65504 where fp16 overflows);
 *   q = clamp(rint_half_even(x / S), -7, 7) with the IEEE fp32 quotient.
 *   q_packed: [N, K/2] bytes, 4-bit two's complement, element 2i in the low nibble.
 *   scale_f16: [N, K/128] IEEE fp16.    K % 128 == 0.
 */
w8a8_status w8a8_quantize_int4(const void* w_bf16, int64_t N, int64_t K, void* q_packed,
                               uint16_t* scale_f16, void* stream);

/* W4A16 GEMM: y[m,n] = bf16_rne( sum_g S[n,g] sum_{k in g} x[m,k] q[n,k] ), x bf16 [M, K],
 * FP32 accumulation on the bf16 matrix cores (the INT4 codes are exact in bf16, S is applied
 * to each group's partial sum). Built for decode (small M): W is streamed once per 128 rows
 * of M. K % 128 == 0. */
w8a8_status w8a8_gemm_w4a16(const void* x_bf16, const void* q_packed, const uint16_t* scale_f16,
                            int64_t M, int64_t N, int64_t K, void* y_bf16, void* stream);

/* ------------------------------------------------------------------------------------
 * SmoothQuant preparation for the INT8 variant ([P-FP8FP4] "SmoothQuant: move the
 * outliers into the weights" and the `smooth` emulation; [P-LOWBIT] §4.2-4.3). Offline.
 *
 * Column maxima of a bf16 [R, K] matrix: amax[j] = max_r |x[r, j]| (exact); for a
 * calibration batch this is max|X_:j|, for W [N, K] it is max|W_:j| over output rows.
 *   amax: fp32 [K]    K % 8 == 0. R = 0 writes zeros.
 */
w8a8_status w8a8_channel_absmax(const void* x_bf16, int64_t R, int64_t K, float* amax,
                                void* stream);

/* Smoothing factors s[j] = max(act_max[j], 1e-5)^alpha / max(w_max[j], 1e-5)^(1-alpha)
 * ([P-LOWBIT] §4.3, the migration strength alpha; [P-FP8FP4] `smooth`), evaluated in fp32
 * on the device, so that the maxima from w8a8_channel_absmax never go through the host. alpha = 0.5 uses correctly rounded square roots and one correctly
 * rounded division (a fully specified fp32 result); alpha = 0 and 1 reduce to 1/w and a;
 * other alpha in (0, 1) use exp2/log2 and are accurate to a few ulp.
 *   act_max, w_max, s: fp32 [K] device arrays.    0 <= alpha <= 1 (W8A8_ERR_ARG). */
w8a8_status w8a8_smoothquant_scales(const float* act_max, const float* w_max, int64_t K,
                                    float alpha, float* s, void* stream);

/* Apply smoothing to a bf16 [R, K] matrix, column j by s[j]:
 *   mode 0 (activations): out = bf16_rne(fp32(x) / s[j])   (IEEE fp32 division)
 *   mode 1 (weights):     out = bf16_rne(fp32(x) * s[j])
 * out_bf16: [R, K]    K % 8 == 0; other modes return W8A8_ERR_ARG. */
w8a8_status w8a8_smooth_apply(const void* x_bf16, int64_t R, int64_t K, const float* s,
                              int mode, void* out_bf16, void* stream);

/* ------------------------------------------------------------------------------------
 * Measurement helper (not part of the method): the shader clock a run actually held. The
 * MFMA peak of a roofline is quoted at the 2.4 GHz maximum clock; the rate of the matrix
 * cores is a fixed number of operations per shader cycle, so a kernel's fraction of the
 * peak at the clock it ran at is its spec-peak fraction times 2.4 GHz / f.
 *
 * Launches `blocks` one-wave workgroups. Each reads the shader-cycle counter and the
 * constant 100 MHz real-time counter at its start and again once `ticks` real-time ticks
 * have passed, then writes out[2 b] = real-time ticks elapsed and out[2 b + 1] = shader
 * cycles elapsed; f = out[2 b + 1] / out[2 b] * 100 MHz on workgroup b's XCD over that
 * window. Enqueue it on a second stream just before the kernels to be measured; it takes
 * one wave slot on `blocks` CUs.
 *   out: uint64 [2 * blocks], 16-byte aligned device array.
 *   1 <= blocks <= 1024 and 1 <= ticks <= 2^32 (W8A8_ERR_ARG otherwise).
 */
w8a8_status w8a8_sclk_probe(uint64_t* out, int blocks, int64_t ticks, void* stream);

/* Measurement helper (not part of the method): the HBM ceiling of the quantizers' traffic.
 * Reads n bf16 values of x_bf16 and writes one byte per value to y (the high byte of the
 * bf16), the 2-bytes-in, 1-byte-out split of the per-token and static quantizers, with no
 * arithmetic to speak of; each thread keeps four 16-byte loads in flight.
 *   x_bf16: [n] bf16, y: [n] bytes, both 16-byte aligned device arrays; n % 8 == 0
 *   (W8A8_ERR_UNSUPPORTED), 0 <= n <= 2^30 (W8A8_ERR_SHAPE). */
w8a8_status w8a8_stream_probe(const void* x_bf16, int64_t n, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
