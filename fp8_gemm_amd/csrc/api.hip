// The C ABI of libw8a8 (declared in include/w8a8.h): argument validation, then kernel launches on
// the caller's stream.  Nothing is allocated and no state is kept between calls.
#include "w8a8.h"

#include <stdint.h>

#include "launch.h"

#define W8A8_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;   // per-dimension limit (32-bit grid arithmetic)
constexpr int64_t kMaxKInt8 = 133144;           // K * 127^2 < 2^31

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool valid_dtype(w8a8_dtype t) { return t == W8A8_F32 || t == W8A8_BF16; }
bool valid_qtype(w8a8_qtype t) { return t == W8A8_INT8 || t == W8A8_FP8_E4M3; }

w8a8_status from_hip(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_ERR_HIP; }

// Common shape rules: M, N >= 0, K >= 1, all below 2^31; K a multiple of 16.
w8a8_status check_dims(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 1 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return W8A8_ERR_INVALID_ARG;
    if (K % 16 != 0) return W8A8_ERR_UNSUPPORTED;
    if (M / 32 >= 65535 || K / 32 >= 65535 || K / 128 >= 65535) return W8A8_ERR_UNSUPPORTED;  // 2-D grid limits
    if (K >= (int64_t(1) << 24)) return W8A8_ERR_UNSUPPORTED;   // 32-bit in-tile offsets of the GEMM
    return W8A8_OK;
}

}  // namespace

W8A8_API w8a8_status w8a8_smooth_scales(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K, const void* w,
                                        w8a8_dtype w_dtype, int64_t N, float alpha, float* ax, float* aw,
                                        int accumulate, float* s, hipStream_t stream) {
    if (!ax || !aw || !s || !valid_dtype(x_dtype) || !valid_dtype(w_dtype)) return W8A8_ERR_INVALID_ARG;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && !x) return W8A8_ERR_INVALID_ARG;
    if (N > 0 && !w) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (!aligned16(x) || !aligned16(w) || !aligned16(ax) || !aligned16(aw) || !aligned16(s)) return W8A8_ERR_UNSUPPORTED;
    hipError_t e = hipSuccess;
    if (!accumulate) e = w8a8::launch_fill(ax, K, 0.0f, stream);
    if (e == hipSuccess) e = w8a8::launch_absmax_cols(x, x_dtype == W8A8_BF16, M, K, nullptr, 0.0f, ax, stream);
    if (e == hipSuccess) {
        if (N > 0) {
            // row maxima of W and, fused, the smoothing factors from the finished ax
            e = w8a8::launch_absmax_rows(w, w_dtype == W8A8_BF16, K, N, aw, ax, alpha, s, stream);
        } else {
            e = w8a8::launch_fill(aw, K, 0.0f, stream);
            if (e == hipSuccess) e = w8a8::launch_smooth_factors(ax, aw, K, alpha, s, stream);
        }
    }
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_fold_quant_weight(const void* w, w8a8_dtype w_dtype, int64_t K, int64_t N, const float* s,
                                            w8a8_qtype qtype, void* wq, float* w_scale, hipStream_t stream) {
    if (!valid_dtype(w_dtype) || !valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (N > 0 && (!w || !wq || !w_scale)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(0, N, K);
    if (st != W8A8_OK) return st;
    if (N == 0) return W8A8_OK;
    if (!aligned16(w) || !aligned16(s) || !aligned16(wq) || !aligned16(w_scale)) return W8A8_ERR_UNSUPPORTED;
    const bool bf16 = w_dtype == W8A8_BF16, fp8 = qtype == W8A8_FP8_E4M3;
    // The column pass leaves the scales max_j |W~[j, n]| / Q in w_scale; the codes use them.
    hipError_t e = w8a8::launch_fill(w_scale, N, 0.0f, stream);
    if (e == hipSuccess) e = w8a8::launch_absmax_cols(w, bf16, K, N, s, fp8 ? 448.0f : 127.0f, w_scale, stream);
    if (e == hipSuccess)
        e = w8a8::launch_quant_weight_t(w, bf16, K, N, s, w_scale, false, fp8, static_cast<uint8_t*>(wq), stream);
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_smooth_quant(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K, const void* w,
                                       w8a8_dtype w_dtype, int64_t N, float alpha, w8a8_qtype qtype, float* ax,
                                       float* aw, float* s, void* wq, float* w_scale, void* xq, float* x_scale,
                                       hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_dtype(w_dtype) || !valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return W8A8_ERR_INVALID_ARG;
    if (!ax || !aw || !s) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!x || !xq || !x_scale)) return W8A8_ERR_INVALID_ARG;
    if (N > 0 && (!w || !wq || !w_scale)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (!aligned16(x) || !aligned16(w) || !aligned16(ax) || !aligned16(aw) || !aligned16(s) || !aligned16(wq) ||
        !aligned16(w_scale) || !aligned16(xq) || !aligned16(x_scale))
        return W8A8_ERR_UNSUPPORTED;
    const bool fp8 = qtype == W8A8_FP8_E4M3;
    const bool fused = x_dtype == w_dtype && M >= 1 && N >= 1 && N % 8 == 0 && K <= 8192 && M < (int64_t(1) << 23) &&
                       N < (int64_t(1) << 23);
    if (!fused) {
        st = w8a8_smooth_scales(x, x_dtype, M, K, w, w_dtype, N, alpha, ax, aw, 0, s, stream);
        if (st == W8A8_OK) st = w8a8_fold_quant_weight(w, w_dtype, K, N, s, qtype, wq, w_scale, stream);
        if (st == W8A8_OK) st = w8a8_quant_act(x, x_dtype, M, K, s, qtype, xq, x_scale, stream);
        return st;
    }
    const bool bf16 = x_dtype == W8A8_BF16;
    hipError_t e = w8a8::launch_zero2(ax, K, w_scale, N, stream);
    if (e == hipSuccess) e = w8a8::launch_calib_pair(x, w, bf16, M, K, N, ax, aw, stream);
    if (e == hipSuccess)
        e = w8a8::launch_fold_cols(w, bf16, K, N, ax, aw, alpha, fp8 ? 448.0f : 127.0f, s, w_scale, stream);
    if (e == hipSuccess)
        e = w8a8::launch_quant_pair(x, bf16, M, K, s, fp8, static_cast<uint8_t*>(xq), x_scale, w, N, w_scale,
                                    static_cast<uint8_t*>(wq), stream);
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_quant_act(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K, const float* s,
                                    w8a8_qtype qtype, void* xq, float* x_scale, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!x || !xq || !x_scale)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, 0, K);
    if (st != W8A8_OK) return st;
    if (M == 0) return W8A8_OK;
    if (!aligned16(x) || !aligned16(s) || !aligned16(xq) || !aligned16(x_scale)) return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_quant_act(x, x_dtype == W8A8_BF16, M, K, s, qtype == W8A8_FP8_E4M3,
                                           static_cast<uint8_t*>(xq), x_scale, stream));
}

W8A8_API w8a8_status w8a8_quant_pair(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K, const void* w,
                                     w8a8_dtype w_dtype, int64_t N, const float* s, const float* w_scale,
                                     w8a8_qtype qtype, void* xq, float* x_scale, void* wq, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_dtype(w_dtype) || !valid_qtype(qtype) || !s) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!x || !xq || !x_scale)) return W8A8_ERR_INVALID_ARG;
    if (N > 0 && (!w || !wq || !w_scale)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (!aligned16(x) || !aligned16(w) || !aligned16(s) || !aligned16(w_scale) || !aligned16(xq) ||
        !aligned16(x_scale) || !aligned16(wq))
        return W8A8_ERR_UNSUPPORTED;
    const bool fp8 = qtype == W8A8_FP8_E4M3;
    const bool one_launch = x_dtype == w_dtype && M >= 1 && N >= 1 && N % 8 == 0 && K <= 8192 &&
                            M < (int64_t(1) << 23) && N < (int64_t(1) << 23);
    hipError_t e = hipSuccess;
    if (one_launch) {
        e = w8a8::launch_quant_pair(x, x_dtype == W8A8_BF16, M, K, s, fp8, static_cast<uint8_t*>(xq), x_scale, w, N,
                                    w_scale, static_cast<uint8_t*>(wq), stream);
    } else {
        if (M > 0)
            e = w8a8::launch_quant_act(x, x_dtype == W8A8_BF16, M, K, s, fp8, static_cast<uint8_t*>(xq), x_scale,
                                       stream);
        if (e == hipSuccess && N > 0)
            e = w8a8::launch_quant_weight_t(w, w_dtype == W8A8_BF16, K, N, s, w_scale, false, fp8,
                                            static_cast<uint8_t*>(wq), stream);
    }
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_gemm_dequant(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                                       w8a8_qtype qtype, int64_t M, int64_t N, int64_t K, void* y,
                                       hipStream_t stream) {
    if (!valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (!xq || !x_scale || !wq || !w_scale || !y)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (qtype == W8A8_INT8 && K > kMaxKInt8) return W8A8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(x_scale) || !aligned16(w_scale))
        return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_gemm(static_cast<const uint8_t*>(xq), x_scale, static_cast<const uint8_t*>(wq),
                                      w_scale, qtype == W8A8_FP8_E4M3, false, M, N, K, static_cast<uint16_t*>(y),
                                      nullptr, stream));
}

W8A8_API w8a8_status w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                                   int32_t* acc, hipStream_t stream) {
    if (M > 0 && N > 0 && (!xq || !wq || !acc)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (K > kMaxKInt8) return W8A8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(acc)) return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_gemm(reinterpret_cast<const uint8_t*>(xq), nullptr,
                                      reinterpret_cast<const uint8_t*>(wq), nullptr, false, false, M, N, K, nullptr,
                                      acc, stream));
}

W8A8_API w8a8_status w8a8_gemm_f32(const uint8_t* xq, const uint8_t* wq, int64_t M, int64_t N, int64_t K,
                                   float* acc, hipStream_t stream) {
    if (M > 0 && N > 0 && (!xq || !wq || !acc)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(acc)) return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_gemm(xq, nullptr, wq, nullptr, true, false, M, N, K, nullptr, acc, stream));
}

// ---- per-tensor scaling -------------------------------------------------------------------------

W8A8_API w8a8_status w8a8_absmax(const void* a, w8a8_dtype dtype, int64_t n, float* amax, int accumulate,
                                 hipStream_t stream) {
    if (!amax || !valid_dtype(dtype) || n < 0) return W8A8_ERR_INVALID_ARG;
    if (n > 0 && !a) return W8A8_ERR_INVALID_ARG;
    if (n % 8 != 0 || !aligned16(a) || !aligned4(amax)) return W8A8_ERR_UNSUPPORTED;
    hipError_t e = hipSuccess;
    if (!accumulate) e = w8a8::launch_fill(amax, 1, 0.0f, stream);
    if (e == hipSuccess) e = w8a8::launch_absmax_tensor(a, dtype == W8A8_BF16, n, 0.0f, amax, stream);
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_quant_act_tensor(const void* x, w8a8_dtype x_dtype, int64_t M, int64_t K,
                                           const float* amax_in, w8a8_qtype qtype, void* xq, float* x_scale,
                                           float* amax_out, int accumulate, hipStream_t stream) {
    if (!valid_dtype(x_dtype) || !valid_qtype(qtype) || !amax_in || !x_scale) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!x || !xq)) return W8A8_ERR_INVALID_ARG;
    if (amax_out && amax_out == amax_in) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, 0, K);
    if (st != W8A8_OK) return st;
    if (!aligned16(x) || !aligned16(xq) || !aligned4(amax_in) || !aligned4(x_scale) || !aligned4(amax_out))
        return W8A8_ERR_UNSUPPORTED;
    hipError_t e = hipSuccess;
    if (amax_out && !accumulate) e = w8a8::launch_fill(amax_out, 1, 0.0f, stream);
    if (e == hipSuccess)     // M == 0 still writes x_scale
        e = w8a8::launch_quant_tensor(x, x_dtype == W8A8_BF16, M * K, amax_in, qtype == W8A8_FP8_E4M3,
                                      static_cast<uint8_t*>(xq), x_scale, amax_out, stream);
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_quant_weight_tensor(const void* w, w8a8_dtype w_dtype, int64_t K, int64_t N,
                                              w8a8_qtype qtype, void* wq, float* w_scale, hipStream_t stream) {
    if (!valid_dtype(w_dtype) || !valid_qtype(qtype) || !w_scale) return W8A8_ERR_INVALID_ARG;
    if (N > 0 && (!w || !wq)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(0, N, K);
    if (st != W8A8_OK) return st;
    if (!aligned16(w) || !aligned16(wq) || !aligned4(w_scale)) return W8A8_ERR_UNSUPPORTED;
    const bool bf16 = w_dtype == W8A8_BF16, fp8 = qtype == W8A8_FP8_E4M3;
    // The maximum divided by Q, merged block by block (correctly rounded division is monotone, so
    // the merged value is max|W| / Q rounded once); then the codes with that one scale.
    hipError_t e = w8a8::launch_fill(w_scale, 1, 0.0f, stream);
    if (e == hipSuccess && N > 0) e = w8a8::launch_absmax_tensor(w, bf16, K * N, fp8 ? 448.0f : 127.0f, w_scale, stream);
    if (e == hipSuccess && N > 0)
        e = w8a8::launch_quant_weight_t(w, bf16, K, N, nullptr, w_scale, true, fp8, static_cast<uint8_t*>(wq), stream);
    return from_hip(e);
}

W8A8_API w8a8_status w8a8_gemm_dequant_tensor(const void* xq, const float* x_scale, const void* wq,
                                              const float* w_scale, w8a8_qtype qtype, int64_t M, int64_t N,
                                              int64_t K, void* y, hipStream_t stream) {
    if (!valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (!xq || !x_scale || !wq || !w_scale || !y)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (qtype == W8A8_INT8 && K > kMaxKInt8) return W8A8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned4(x_scale) || !aligned4(w_scale))
        return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_gemm(static_cast<const uint8_t*>(xq), x_scale, static_cast<const uint8_t*>(wq),
                                      w_scale, qtype == W8A8_FP8_E4M3, true, M, N, K, static_cast<uint16_t*>(y),
                                      nullptr, stream));
}

// ---- RMS norm with the smoothing folded into its gain -------------------------------------------------

W8A8_API w8a8_status w8a8_fold_norm_gain(const float* g, const float* s, int64_t K, float* g_out, hipStream_t stream) {
    if (!g_out || K < 1 || K >= kMaxDim) return W8A8_ERR_INVALID_ARG;
    return from_hip(w8a8::launch_fold_norm_gain(g, s, K, g_out, stream));
}

W8A8_API w8a8_status w8a8_norm_quant_act(const void* h, w8a8_dtype h_dtype, int64_t M, int64_t K, const float* g,
                                         float eps, w8a8_qtype qtype, void* xq, float* x_scale, hipStream_t stream) {
    if (!valid_dtype(h_dtype) || !valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (!(eps >= 0.0f && eps < 1.0f)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!h || !xq || !x_scale)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, 0, K);
    if (st != W8A8_OK) return st;
    if (K > 8192) return W8A8_ERR_UNSUPPORTED;            // rows are held in registers
    if (M == 0) return W8A8_OK;
    if (!aligned16(h) || !aligned16(g) || !aligned16(xq) || !aligned16(x_scale)) return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_norm_quant_act(h, h_dtype == W8A8_BF16, M, K, g, nullptr, false, eps,
                                                qtype == W8A8_FP8_E4M3, static_cast<uint8_t*>(xq), x_scale, stream));
}

W8A8_API w8a8_status w8a8_layer_norm_quant_act(const void* h, w8a8_dtype h_dtype, int64_t M, int64_t K, const float* g,
                                               const float* b, float eps, w8a8_qtype qtype, void* xq, float* x_scale,
                                               hipStream_t stream) {
    if (!valid_dtype(h_dtype) || !valid_qtype(qtype)) return W8A8_ERR_INVALID_ARG;
    if (!(eps >= 0.0f && eps < 1.0f)) return W8A8_ERR_INVALID_ARG;
    if (M > 0 && (!h || !xq || !x_scale)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, 0, K);
    if (st != W8A8_OK) return st;
    if (K > 8192) return W8A8_ERR_UNSUPPORTED;            // rows are held in registers
    if (M == 0) return W8A8_OK;
    if (!aligned16(h) || !aligned16(g) || !aligned16(b) || !aligned16(xq) || !aligned16(x_scale))
        return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_norm_quant_act(h, h_dtype == W8A8_BF16, M, K, g, b, true, eps,
                                                qtype == W8A8_FP8_E4M3, static_cast<uint8_t*>(xq), x_scale, stream));
}

// ---- weight-only W8A16 ------------------------------------------------------------------------------

W8A8_API w8a8_status w8a8_gemm_w8a16(const void* x, const int8_t* wq, const float* w_scale, int64_t M, int64_t N,
                                     int64_t K, void* y, hipStream_t stream) {
    if (M > 0 && N > 0 && (!x || !wq || !w_scale || !y)) return W8A8_ERR_INVALID_ARG;
    w8a8_status st = check_dims(M, N, K);
    if (st != W8A8_OK) return st;
    if (M == 0 || N == 0) return W8A8_OK;
    if (!aligned16(x) || !aligned16(wq) || !aligned16(y) || !aligned16(w_scale)) return W8A8_ERR_UNSUPPORTED;
    return from_hip(w8a8::launch_gemm_w8a16(static_cast<const uint16_t*>(x), wq, w_scale, M, N, K,
                                            static_cast<uint16_t*>(y), stream));
}

W8A8_API const char* w8a8_status_string(w8a8_status status) {
    switch (status) {
        case W8A8_OK: return "ok";
        case W8A8_ERR_INVALID_ARG: return "invalid argument";
        case W8A8_ERR_UNSUPPORTED: return "unsupported shape or alignment (K % 16, 16-byte pointers, size limits)";
        case W8A8_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

W8A8_API const char* w8a8_version(void) { return "libw8a8 0.1 gfx950"; }
