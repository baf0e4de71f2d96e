// Host-side launchers of the libw8a8 kernels.  Arguments are validated by the C-ABI layer
// (api.hip) before any of these is called; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Fill n floats with v (used instead of a memset so the call sequence stays capturable).
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st);

// out[c] = max(out[c], m_c) with m_c = max_r |a[r, c] * (row_scale ? row_scale[r] : 1)| for a
// row-major [R, C] matrix of float32 or bf16, divided by divisor (rounded once) when divisor != 0.
// Exact; concurrent blocks merge with an order-independent atomic maximum.
hipError_t launch_absmax_cols(const void* a, bool bf16, int64_t R, int64_t C, const float* row_scale,
                              float divisor, float* out, hipStream_t st);

// out[r] = max_c |a[r, c]| for a row-major [R, C] matrix (one wave per row, no atomics); with
// ax != NULL also s[r] = smoothing factor of (ax[r], out[r]).
hipError_t launch_absmax_rows(const void* a, bool bf16, int64_t R, int64_t C, float* out, const float* ax,
                              float alpha, float* s, hipStream_t st);

// Zero p[0, n) and q[0, m) in one launch.
hipError_t launch_zero2(float* p, int64_t n, float* q, int64_t m, hipStream_t st);

// One launch for the two calibration reductions of a layer: ax[k] = max(ax[k], max_m |X[m, k]|)
// (atomic, ax zeroed beforehand) and aw[k] = max_n |W[k, n]|.  X, W of one dtype, K % 8 == 0,
// N % 8 == 0, M, N >= 1.
hipError_t launch_calib_pair(const void* x, const void* w, bool bf16, int64_t M, int64_t K, int64_t N, float* ax,
                             float* aw, hipStream_t st);

// w_scale[n] = max(w_scale[n], max_k |s[k] W[k, n]| / divisor) (atomic, w_scale zeroed
// beforehand) with s[k] = smoothing factor of (ax[k], aw[k]) computed in the kernel, which also
// writes s.  N % 8 == 0.
hipError_t launch_fold_cols(const void* w, bool bf16, int64_t K, int64_t N, const float* ax, const float* aw,
                            float alpha, float divisor, float* s, float* w_scale, hipStream_t st);

// One launch for the activation codes (as launch_quant_act with s) and the weight codes (as
// launch_quant_weight_t with per-column scales).  K <= 8192, N % 8 == 0, M, N >= 1.
hipError_t launch_quant_pair(const void* x, bool bf16, int64_t M, int64_t K, const float* s, bool fp8, uint8_t* xq,
                             float* x_scale, const void* w, int64_t N, const float* w_scale, uint8_t* wq,
                             hipStream_t st);

// s[j] = ax[j]^alpha / aw[j]^(1-alpha), s = 1 where a maximum is 0.
hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s,
                                 hipStream_t st);

// Per-row smooth + quantize of X [M, K]: xq [M, K] codes and x_scale [M].
hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, const float* s, bool fp8,
                            uint8_t* xq, float* x_scale, hipStream_t st);

// Quantize W~ = s * W [K, N] with the per-column scales w_scale [N] (from launch_absmax_cols with
// divisor 127 or 448), or with tensor_scale the one scale w_scale[0], and write the codes
// transposed, wq [N, K].
hipError_t launch_quant_weight_t(const void* w, bool bf16, int64_t K, int64_t N, const float* s,
                                 const float* w_scale, bool tensor_scale, bool fp8, uint8_t* wq, hipStream_t st);

// out[0] = max(out[0], max_i |a[i]| / divisor (rounded once; divisor 0: no division)) over n
// elements, n a multiple of 8, a 16-byte aligned.  Exact; blocks merge with an atomic maximum.
hipError_t launch_absmax_tensor(const void* a, bool bf16, int64_t n, float divisor, float* out, hipStream_t st);

// Per-tensor quantize of n elements (a multiple of 8): scale = amax_in[0] / Q, q[i] = code of
// a[i] / scale saturated at +-Q (scale 0: codes 0), scale_out[0] = scale.  amax_out != nullptr:
// max_i |a[i]| is merged into amax_out[0] in the same pass (it must not be amax_in).
hipError_t launch_quant_tensor(const void* a, bool bf16, int64_t n, const float* amax_in, bool fp8, uint8_t* q,
                               float* scale_out, float* amax_out, hipStream_t st);

// GEMM over K-contiguous operands xq [M, K] and wq [N, K]:
//   acc != nullptr: the raw accumulators [M, N] (int32 for INT8, fp32 for E4M3)
//   else: y bf16 [M, N] = ((float)acc * x_scale[m]) * w_scale[n], or with tensor_scales the one
//   scale of each operand, x_scale[0] and w_scale[0].
hipError_t launch_gemm(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale,
                       bool fp8, bool tensor_scales, int64_t M, int64_t N, int64_t K, uint16_t* y, void* acc,
                       hipStream_t st);

// RMS norm with gain g (g' = g / s folded in; NULL = 1), or with layer a LayerNorm with gain g and
// bias b (NULL = 1 and 0), and the per-token quantize, one pass over h [M, K] (K <= 8192):
// xq [M, K] codes and x_scale [M].
hipError_t launch_norm_quant_act(const void* h, bool bf16, int64_t M, int64_t K, const float* g, const float* b,
                                 bool layer, float eps, bool fp8, uint8_t* xq, float* x_scale, hipStream_t st);

// out[j] = g[j] / s[j] (correctly rounded; NULL operands are 1).
hipError_t launch_fold_norm_gain(const float* g, const float* s, int64_t K, float* out, hipStream_t st);

// Weight-only W8A16: y bf16 [M, N] = bf16(w_scale[n] * sum_k x[m, k] * wq[n, k]), x bf16 [M, K],
// wq int8 [N, K] (codes converted to bf16 on the fly, bf16 matrix cores, fp32 sums).
hipError_t launch_gemm_w8a16(const uint16_t* x, const int8_t* wq, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t st);

}  // namespace w8a8
