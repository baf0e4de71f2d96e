/*
 * libw8a8 - the W8A8 linear layer on AMD Instinct MI355X (gfx950).
 *
 * The layer Y = X W is computed as Y = X~ W~ with X~[i, j] = X[i, j] / s_j and W~[j, n] = s_j W[j, n]
 * (SmoothQuant factors s), symmetric 8-bit quantization of both operands (one scale per token of
 * X, one per output channel of W), an 8-bit GEMM with 32-bit accumulation on the matrix cores,
 * and a dequantizing epilogue that writes bf16.  Sources, by page and section:
 *   [WAQ] "Weight-Activation Quantization" (infra.bea.ai inference guide):
 *         s2 "The Problem: Activation Outliers"  symmetric INT8, scale = absmax / 127;
 *         s3 "SmoothQuant: The Smoothing Trick"  Y = XW = (X S^-1)(S W), divide activation
 *             channel j by s_j and multiply weight channel j by s_j, smoothing offline then
 *             quantization at inference, the 8-bit product dequantized by the scales, and
 *             s_j = max|X_j|^alpha / max|W_j|^(1-alpha) with alpha in [0, 1];
 *         s4 "FP8 W8A8"  E4M3 operands, range [-448, 448], codes of x / s, x^ = s q,
 *             s = max|x| / 448.
 *   [ACT] "Define activation quantization ..." (zenaique flashcard): per-token activation and
 *         per-channel weight scaling.
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library allocates nothing and
 *     keeps no state between calls.  All matrices are dense and row-major.
 *   - X is [M, K] (M tokens, K input channels); W is [K, N] (N output channels); Y is [M, N].
 *     Quantized weights are stored transposed, [N, K], so that both GEMM operands have K
 *     contiguous.  Codes are one byte each: int8 for W8A8_INT8, OCP E4M3 ("fn": bias 7, max 448,
 *     no infinities) bit patterns for W8A8_FP8_E4M3.
 *   - Element types of X and W: float32 or bfloat16.  Y is bfloat16 (round to nearest even).
 *   - Every call is asynchronous on `stream` (0 = the default stream) and returns after queueing.
 *   - Shapes: M >= 0 and N >= 0 (0 = nothing to do, W8A8_OK with nothing launched); K >= 1.
 *     K must be a multiple of 16 and every pointer 16-byte aligned, else W8A8_ERR_UNSUPPORTED.
 *   - Errors: NULL required pointer, negative size, unknown enum, alpha outside [0, 1] ->
 *     W8A8_ERR_INVALID_ARG, checked before anything is queued; a failed launch -> W8A8_ERR_HIP.
 *   - Arithmetic: divisions are IEEE fp32 divisions and roundings are to nearest, ties to even,
 *     so the quantized codes, scales and int32 accumulators are deterministic and reproducible
 *     bit for bit.  A zero maximum gives s_j = 1; a row or column whose scale is 0 (all zero, or a
 *     maximum so small that its quotient by 127 or 448 rounds to 0) gets codes 0.  NaN and
 *     infinite inputs are not supported, nor are X / s or s * W that overflow.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations are int-sized as in C.  In C++ they get int as their fixed underlying type, so
 * that any int a caller passes is a value of the type and can be checked (an enumeration without
 * one cannot hold values outside its enumerators' range); the ABI is the same. */
#ifdef __cplusplus
#define W8A8_ENUM_BASE : int
#else
#define W8A8_ENUM_BASE
#endif

typedef enum w8a8_status W8A8_ENUM_BASE {
    W8A8_OK = 0,
    W8A8_ERR_INVALID_ARG = 1,
    W8A8_ERR_UNSUPPORTED = 2,
    W8A8_ERR_HIP = 3
} w8a8_status;

typedef enum w8a8_dtype W8A8_ENUM_BASE { W8A8_F32 = 0, W8A8_BF16 = 1 } w8a8_dtype;

typedef enum w8a8_qtype W8A8_ENUM_BASE { W8A8_INT8 = 0, W8A8_FP8_E4M3 = 1 } w8a8_qtype;

/*
 * Calibration maxima and SmoothQuant factors ([WAQ] s3 "Choosing the Smoothing Factor").
 *   ax[j] = max_i |X[i, j]|       (column maxima of the calibration activations X [M, K])
 *   aw[j] = max_n |W[j, n]|       (row maxima of the weights W [K, N])
 *   s[j]  = ax[j]^alpha / aw[j]^(1 - alpha); s[j] = 1 where ax[j] or aw[j] is 0.
 *           alpha = 0.5 is evaluated as sqrt(ax) / sqrt(aw) with correctly rounded fp32 roots and
 *           division (bit-reproducible); other alpha use pow in double rounded once to fp32.
 * ax, aw, s: caller-owned fp32 [K], all written.  accumulate != 0 folds the maxima of this X into
 * the values already in ax (max over several calibration batches); 0 overwrites ax.  M may be 0
 * (no calibration rows: ax is left as is with accumulate, else zero).
 */
w8a8_status w8a8_smooth_scales(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K,
                               const void* w, w8a8_dtype w_dtype, int64_t N, float alpha,
                               float* ax, float* aw, int accumulate, float* s, hipStream_t stream);

/*
 * Weight fold and quantize ([WAQ] s3 step 1, the weight rows scaled by s, and step 2, their
 * quantization; per-output-channel scales [ACT]; FP8 per [WAQ] s4).
 *   W~[j, n]   = s[j] * W[j, n]                               (fp32 multiply; s == NULL: s = 1)
 *   w_scale[n] = max_j |W~[j, n]| / Q                         (Q = 127 for INT8, 448 for E4M3)
 *   wq[n, j]   = INT8: clamp(round_half_even(W~[j, n] / w_scale[n]), -127, 127)
 *                E4M3: e4m3_round_half_even(clamp(W~[j, n] / w_scale[n], -448, 448))
 * w: [K, N] in w_dtype.  s: fp32 [K] or NULL.  wq: [N, K] bytes (written).  w_scale: fp32 [N]
 * (written; it accumulates the column maxima while the call runs).
 */
w8a8_status w8a8_fold_quant_weight(const void* w, w8a8_dtype w_dtype, int64_t K, int64_t N,
                                   const float* s, w8a8_qtype qtype, void* wq, float* w_scale,
                                   hipStream_t stream);

/*
 * Activation smooth + per-token quantize, one pass over X ([WAQ] s3: activation channel j
 * divided by s_j, and step 2, its quantization at inference; per-token scales [ACT]; FP8 [WAQ] s4).
 *   X~[i, j]   = X[i, j] / s[j]                               (fp32 division; s == NULL: s = 1)
 *   x_scale[i] = max_j |X~[i, j]| / Q                         (Q = 127 or 448)
 *   xq[i, j]   = the same rounding as w8a8_fold_quant_weight, with x_scale[i].
 * x: [M, K] in x_dtype.  s: fp32 [K] or NULL.  xq: [M, K] bytes.  x_scale: fp32 [M].
 */
w8a8_status w8a8_quant_act(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K,
                           const float* s, w8a8_qtype qtype, void* xq, float* x_scale,
                           hipStream_t stream);

/*
 * Calibration, smoothing factors, weight fold + quantize and activation quantize of one layer in
 * one call ([WAQ] s3 steps 1 and 2, the calibration of s3 "Choosing the Smoothing Factor"): the
 * results are those of w8a8_smooth_scales (accumulate = 0), then w8a8_fold_quant_weight with its
 * s, then w8a8_quant_act with its s, bit for bit.  ax, aw, s: fp32 [K]; wq [N, K], w_scale [N];
 * xq [M, K], x_scale [M]; all written, and none may overlap x or w.  X and W of one dtype,
 * N % 8 == 0 and K <= 8192 take four launches (zero ax and w_scale; both calibration maxima; s
 * and the weight scales; the activation and weight codes); other shapes take the three calls'
 * seven.  Errors as the three calls.
 */
w8a8_status w8a8_smooth_quant(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K,
                              const void* w, w8a8_dtype w_dtype, int64_t N, float alpha,
                              w8a8_qtype qtype, float* ax, float* aw, float* s, void* wq,
                              float* w_scale, void* xq, float* x_scale, hipStream_t stream);

/*
 * The codes of both operands in one launch, given the smoothing factors and the final weight
 * scales: the last step of w8a8_smooth_quant, for callers that hold s and w_scale already ([WAQ]
 * s3 step 2 for X, the quantization of the smoothed weights for W; scales per token and per output
 * channel [ACT]; FP8 [WAQ] s4).
 *   xq, x_scale: exactly as w8a8_quant_act(x, s) writes them;
 *   wq:          the codes of w8a8_fold_quant_weight(w, s) with the given w_scale, which must be
 *                the scales that call (or w8a8_smooth_quant) computes, max_j |s[j] W[j, n]| / Q.
 * x: [M, K], w: [K, N]; s: fp32 [K] (not NULL); w_scale: fp32 [N] (read only); xq [M, K], x_scale
 * [M], wq [N, K] written; none may overlap x, w, s or w_scale.  X and W of one dtype, N % 8 == 0
 * and K <= 8192 take one launch, other shapes two (the activation quantize, then the weight codes).
 * M or N may be 0 (that operand is skipped).  Errors as w8a8_quant_act and w8a8_fold_quant_weight.
 */
w8a8_status w8a8_quant_pair(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K, const void* w,
                            w8a8_dtype w_dtype, int64_t N, const float* s, const float* w_scale,
                            w8a8_qtype qtype, void* xq, float* x_scale, void* wq, hipStream_t stream);

/*
 * Quantized GEMM with the dequantizing epilogue ([WAQ] s3 step 2, the 8-bit product dequantized;
 * [WAQ] s4 x^ = s q for E4M3).
 *   INT8: acc[i, n] = sum_k xq[i, k] * wq[n, k] exactly in int32 (|acc| <= K * 127^2, so
 *         K <= 133144; codes must lie in [-127, 127], as the quantize calls write them: a -128
 *         code can overflow the sum at the largest K), y[i, n] = bf16(((float)acc * x_scale[i]) * w_scale[n]).
 *   E4M3: acc = sum_k e4m3(xq[i, k]) * e4m3(wq[n, k]) accumulated in fp32 on the matrix cores
 *         (products are exact; the summation order is the hardware's), y as above.
 * xq: [M, K] bytes, x_scale: fp32 [M], wq: [N, K] bytes, w_scale: fp32 [N], y: bf16 [M, N].
 */
w8a8_status w8a8_gemm_dequant(const void* xq, const float* x_scale, const void* wq,
                              const float* w_scale, w8a8_qtype qtype, int64_t M, int64_t N,
                              int64_t K, void* y, hipStream_t stream);

/*
 * The INT8 GEMM without the epilogue: acc[i, n] = sum_k xq[i, k] * wq[n, k] in int32 [M, N].
 * Same kernels and tiling as w8a8_gemm_dequant; exists so the integer accumulators can be
 * checked bit for bit.  K <= 133144, codes in [-127, 127] (as for w8a8_gemm_dequant).
 */
w8a8_status w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                          int32_t* acc, hipStream_t stream);

/*
 * The E4M3 GEMM without the epilogue: acc[i, n] = sum_k e4m3(xq[i, k]) * e4m3(wq[n, k]) as the
 * matrix cores accumulate it, fp32 [M, N].  Same kernels and tiling as w8a8_gemm_dequant with
 * W8A8_FP8_E4M3; exists so the accumulators can be compared with an exact dot product.
 */
w8a8_status w8a8_gemm_f32(const uint8_t* xq, const uint8_t* wq, int64_t M, int64_t N, int64_t K,
                          float* acc, hipStream_t stream);

/*
 * ---- Per-tensor scaling ([WAQ] s4 "Per-Tensor Scaling for FP8": one scale s = max|x| / 448 for a
 * whole tensor, codes of x / s, x^ = s q, no smoothing; the FP8-vs-INT8 table there names
 * delayed scaling, where s comes from the previous step's maximum.  [WAQ] s2 shows the same
 * recipe for INT8 with 127.)  Every scale and maximum below is ONE fp32 value in device memory.
 */

/*
 * Tensor maximum: amax[0] = max(accumulate ? amax[0] : 0, max_i |a[i]|) over n elements of a
 * (float32 or bf16).  n >= 0 and a multiple of 8; a 16-byte aligned (else W8A8_ERR_UNSUPPORTED).
 * Exact (no rounding), independent of how the work is split.
 */
w8a8_status w8a8_absmax(const void* a, w8a8_dtype dtype, int64_t n, float* amax, int accumulate,
                        hipStream_t stream);

/*
 * Per-tensor activation quantize, one pass over X [M, K]:
 *   x_scale[0] = amax_in[0] / Q                                (Q = 127 for INT8, 448 for E4M3)
 *   xq[i, j]   = INT8: clamp(round_half_even(X[i, j] / x_scale[0]), -127, 127)
 *                E4M3: e4m3_round_half_even(clamp(X[i, j] / x_scale[0], -448, 448))
 * amax_in: this X's own maximum (from w8a8_absmax: current scaling) or an earlier step's
 * (delayed scaling: values beyond Q * x_scale saturate).  amax_out: NULL, or a value that
 * receives max_{i,j} |X[i, j]| in the same pass (reset first unless accumulate != 0), for the
 * next step's amax_in; it must not be amax_in (W8A8_ERR_INVALID_ARG).  A zero amax_in gives
 * x_scale 0 and codes 0.  xq: [M, K] bytes.  x_scale, amax_in, amax_out: 4-byte aligned.
 */
w8a8_status w8a8_quant_act_tensor(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K,
                                  const float* amax_in, w8a8_qtype qtype, void* xq, float* x_scale,
                                  float* amax_out, int accumulate, hipStream_t stream);

/*
 * Per-tensor weight quantize: w_scale[0] = max_{j,n} |W[j, n]| / Q, and
 * wq[n, j] = the codes of W[j, n] / w_scale[0] (rounding as above), transposed to [N, K].
 * w: [K, N] in w_dtype.  w_scale: one fp32, 4-byte aligned (it holds the running maximum
 * divided by Q while the call runs).
 */
w8a8_status w8a8_quant_weight_tensor(const void* w, w8a8_dtype w_dtype, int64_t K, int64_t N,
                                     w8a8_qtype qtype, void* wq, float* w_scale, hipStream_t stream);

/*
 * The GEMM of w8a8_gemm_dequant with one scale per operand:
 *   y[i, n] = bf16(((float)acc[i, n] * x_scale[0]) * w_scale[0]).
 * Same kernels, tiling and accumulation; x_scale and w_scale are single fp32 values (4-byte aligned).
 */
w8a8_status w8a8_gemm_dequant_tensor(const void* xq, const float* x_scale, const void* wq,
                                     const float* w_scale, w8a8_qtype qtype, int64_t M, int64_t N,
                                     int64_t K, void* y, hipStream_t stream);

/*
 * ---- The smoothing folded into the layer before ([WAQ] s3 step 1: the SmoothQuant transform is
 * done offline, during model preparation; the W8A16-vs-W8A8 lesson, s2: no runtime overhead).
 * The activations X come from an RMS norm (or a LayerNorm) of the residual stream h with gain g
 * (and bias b); 1/s is folded into them once, and the norm, the smoothing and the per-token
 * quantize run as one pass over h.
 */

/* g_out[j] = g[j] / s[j] (fp32, correctly rounded); g or s NULL count as 1.  K >= 1. */
w8a8_status w8a8_fold_norm_gain(const float* g, const float* s, int64_t K, float* g_out, hipStream_t stream);

/*
 * Per row i of h [M, K] (h_dtype):
 *   ms       = (float)(sum_j (double)h[i, j]^2 / K)   (the sum exact to about 2^-100: order-free)
 *   r        = 1 / sqrt(ms + eps)                     (fp32, correctly rounded root and division)
 *   X~[i, j] = (h[i, j] * r) * g[j]                   (fp32, in this order; g NULL: 1)
 * then x_scale[i] and xq[i, :] exactly as w8a8_quant_act gives for X~ with s == NULL.
 * g: fp32 [K], normally the output of w8a8_fold_norm_gain.  eps in [0, 1).  K <= 8192 (rows are
 * held in registers), else W8A8_ERR_UNSUPPORTED.  xq: [M, K] bytes, x_scale: fp32 [M].
 */
w8a8_status w8a8_norm_quant_act(const void* h, w8a8_dtype h_dtype, int64_t M, int64_t K, const float* g,
                                float eps, w8a8_qtype qtype, void* xq, float* x_scale, hipStream_t stream);

/*
 * The same with a LayerNorm before the layer ([WAQ] s3 step 1; 1/s is folded into both its gain
 * and its bias, b'[j] = b[j] / s[j], by w8a8_fold_norm_gain(b, s, ...)).  Per row i of h:
 *   mu       = (float)(sum_j (double)h[i, j] / K)     (the sum exact to about 2^-100: order-free)
 *   d[j]     = h[i, j] - mu                           (fp32)
 *   var      = (float)(sum_j (double)d[j]^2 / K)      (likewise)
 *   r        = 1 / sqrt(var + eps)
 *   X~[i, j] = (d[j] * r) * g[j] + b[j]               (fp32, rounded after each operation, no fused
 *                                                      multiply-add; g NULL: 1, b NULL: 0)
 * then x_scale[i] and xq[i, :] as w8a8_norm_quant_act.  Arguments, limits and errors as there.
 */
w8a8_status w8a8_layer_norm_quant_act(const void* h, w8a8_dtype h_dtype, int64_t M, int64_t K, const float* g,
                                      const float* b, float eps, w8a8_qtype qtype, void* xq, float* x_scale,
                                      hipStream_t stream);

/*
 * ---- Weight-only W8A16, the contrast the pages draw with W8A8 ([WAQ] s1 "Why Quantize Activations
 * Too?": weight-only quantization keeps the GEMM in 16-bit; the W8A16-vs-W8A8 lesson, s1: the 8-bit
 * weights are dequantized to 16-bit on the fly and the multiply runs on 16-bit tensor cores).
 *   y[i, n] = bf16(w_scale[n] * sum_k x[i, k] * wq[n, k])
 * x: bf16 [M, K] (not quantized).  wq: int8 [N, K] and w_scale: fp32 [N], the per-output-channel
 * codes and scales of w8a8_fold_quant_weight (with s == NULL for plain weight-only quantization).
 * The codes are converted to bf16 exactly (|q| <= 127), multiplied on the bf16 matrix cores with
 * fp32 accumulation (products exact, summation order the hardware's), and the channel scale is
 * applied to the sum (the dequantized weight q * w_scale factors out of it).  y: bf16 [M, N].
 */
w8a8_status w8a8_gemm_w8a16(const void* x, const int8_t* wq, const float* w_scale, int64_t M, int64_t N,
                            int64_t K, void* y, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* w8a8_status_string(w8a8_status status);

/* Static version string of the library. */
const char* w8a8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
