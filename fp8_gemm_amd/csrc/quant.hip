// Activation smooth + per-token quantize, and the weight quantize-and-transpose.
// ("Weight-Activation Quantization", section 3: divide activation channel j by s_j, multiply
// weight channel j by s_j, then X_int8 = quantize(X_tilde), W_int8 = quantize(W_tilde); section 2:
// symmetric INT8 with scale = absmax / 127; section 4: E4M3 with scale = absmax / 448.)
#include "device.h"
#include "launch.h"

namespace w8a8 {

namespace {

// ---- activations: one wave per row ---------------------------------------------------------------
//
// The row is read once from HBM into registers (kChunks 16-byte chunks of 8 elements per lane),
// divided by s, reduced to its maximum with a wave butterfly, and quantized from registers.
// Lane l owns chunks l, l + 64, l + 128, ... so every load instruction of the wave reads 512
// consecutive elements.
template <bool kBf16, bool kFp8, int kChunks>
__global__ __launch_bounds__(256) void quant_act_kernel(const void* __restrict__ x, const float* __restrict__ s,
                                                        int64_t M, int64_t K, uint8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= M) return;
    const int64_t nchunk = K / 8;
    float v[kChunks][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int64_t c = lane + static_cast<int64_t>(kWave) * i;
        if (c < nchunk) {
            load8<kBf16>(x, row * K + c * 8, v[i]);
            if (s) {
                float sv[8];
                load8<false>(s, c * 8, sv);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[i][e] = div_rn(v[i][e], sv[e]);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
        }
    }
    amax = wave_max(amax);
    const float sc = div_rn(amax, qmax<kFp8>());
    if (lane == 0) scale[row] = sc;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int64_t c = lane + static_cast<int64_t>(kWave) * i;
        if (c < nchunk) {
            uint32_t lo = 0, hi = 0;
            if (amax != 0.0f) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo |= code_of<kFp8>(v[i][e], sc) << (8 * e);
                    hi |= code_of<kFp8>(v[i][e + 4], sc) << (8 * e);
                }
            }
            *reinterpret_cast<uint2*>(q + row * K + c * 8) = make_uint2(lo, hi);
        }
    }
}

// Rows longer than the register-resident variants: two passes over the row (the second mostly
// hits the cache), same arithmetic.
template <bool kBf16, bool kFp8>
__global__ __launch_bounds__(256) void quant_act_long_kernel(const void* __restrict__ x, const float* __restrict__ s,
                                                             int64_t M, int64_t K, uint8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= M) return;
    const int64_t nchunk = K / 8;
    float amax = 0.0f;
    for (int64_t c = lane; c < nchunk; c += kWave) {
        float v[8];
        load8<kBf16>(x, row * K + c * 8, v);
        if (s) {
            float sv[8];
            load8<false>(s, c * 8, sv);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], sv[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
    amax = wave_max(amax);
    const float sc = div_rn(amax, qmax<kFp8>());
    if (lane == 0) scale[row] = sc;
    for (int64_t c = lane; c < nchunk; c += kWave) {
        uint32_t lo = 0, hi = 0;
        if (amax != 0.0f) {
            float v[8];
            load8<kBf16>(x, row * K + c * 8, v);
            if (s) {
                float sv[8];
                load8<false>(s, c * 8, sv);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = div_rn(v[e], sv[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lo |= code_of<kFp8>(v[e], sc) << (8 * e);
                hi |= code_of<kFp8>(v[e + 4], sc) << (8 * e);
            }
        }
        *reinterpret_cast<uint2*>(q + row * K + c * 8) = make_uint2(lo, hi);
    }
}

// ---- weights: W~ = s * W [K, N] -> codes transposed to wq [N, K] --------------------------------
//
// A block owns a tile of kTJ rows (j) x kTN columns (n) of W.  It reads the tile row by row
// (coalesced along n), forms W~ = s[j] * W[j, n] and its code with the column's scale, writes the
// codes into LDS as [n][j], and stores them as rows of wq (contiguous along j).
constexpr int kTJ = 128;
constexpr int kTN = 64;

template <bool kBf16>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
    if constexpr (kBf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
    else return static_cast<const float*>(base)[i];
}

template <bool kBf16, bool kFp8, bool kVec>
__global__ __launch_bounds__(256) void quant_weight_t_kernel(const void* __restrict__ w, int64_t K, int64_t N,
                                                             const float* __restrict__ s,
                                                             const float* __restrict__ amax,
                                                             uint8_t* __restrict__ wq) {
    __shared__ uint8_t tile[kTN][kTJ + 4];
    __shared__ float col_scale[kTN];
    __shared__ float col_amax[kTN];
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTN;
    const int64_t j0 = static_cast<int64_t>(blockIdx.y) * kTJ;
    if (threadIdx.x < kTN) {
        const int64_t n = n0 + threadIdx.x;
        const float a = (n < N) ? amax[n] : 0.0f;
        col_amax[threadIdx.x] = a;
        col_scale[threadIdx.x] = div_rn(a, qmax<kFp8>());
    }
    __syncthreads();
    // kTJ rows x (kTN / 8) chunks of 8 columns = 1024 chunks, 4 per thread.
    for (int idx = threadIdx.x; idx < kTJ * (kTN / 8); idx += blockDim.x) {
        const int jl = idx / (kTN / 8);
        const int cl = (idx % (kTN / 8)) * 8;
        const int64_t j = j0 + jl;
        const int64_t n = n0 + cl;
        float v[8];
        if (j < K && n < N) {
            if constexpr (kVec) {
                load8<kBf16>(w, j * N + n, v);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (n + e < N) ? load1<kBf16>(w, j * N + n + e) : 0.0f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
        const float sj = (s && j < K) ? s[j] : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ws = s ? sj * v[e] : v[e];
            const uint32_t code = (col_amax[cl + e] != 0.0f) ? code_of<kFp8>(ws, col_scale[cl + e]) : 0u;
            tile[cl + e][jl] = static_cast<uint8_t>(code);
        }
    }
    __syncthreads();
    // kTN rows of kTJ bytes = 64 x 8 chunks of 16 bytes, 2 per thread.
    for (int idx = threadIdx.x; idx < kTN * (kTJ / 16); idx += blockDim.x) {
        const int nl = idx / (kTJ / 16);
        const int jc = (idx % (kTJ / 16)) * 16;
        const int64_t n = n0 + nl;
        const int64_t j = j0 + jc;
        if (n < N && j < K) {   // K is a multiple of 16: a 16-byte chunk is all in or all out
            const uint8_t* src = &tile[nl][jc];
            uint4 u;
            u.x = src[0] | (src[1] << 8) | (src[2] << 16) | (static_cast<uint32_t>(src[3]) << 24);
            u.y = src[4] | (src[5] << 8) | (src[6] << 16) | (static_cast<uint32_t>(src[7]) << 24);
            u.z = src[8] | (src[9] << 8) | (src[10] << 16) | (static_cast<uint32_t>(src[11]) << 24);
            u.w = src[12] | (src[13] << 8) | (src[14] << 16) | (static_cast<uint32_t>(src[15]) << 24);
            *reinterpret_cast<uint4*>(wq + n * K + j) = u;
        }
    }
}

__global__ void finalize_scales_kernel(float* p, int64_t n, float qm) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = div_rn(p[i], qm);
}

template <bool kBf16, bool kFp8>
hipError_t quant_act_dispatch(const void* x, int64_t M, int64_t K, const float* s, uint8_t* xq, float* xs,
                              hipStream_t st) {
    dim3 grid(static_cast<unsigned>((M + 3) / 4)), block(256);
    const int64_t per_lane = (K / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, 1>), grid, block, 0, st, x, s, M, K, xq, xs);
    else if (per_lane <= 2) hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, 2>), grid, block, 0, st, x, s, M, K, xq, xs);
    else if (per_lane <= 4) hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, 4>), grid, block, 0, st, x, s, M, K, xq, xs);
    else if (per_lane <= 8) hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, 8>), grid, block, 0, st, x, s, M, K, xq, xs);
    else if (per_lane <= 16) hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, 16>), grid, block, 0, st, x, s, M, K, xq, xs);
    else hipLaunchKernelGGL((quant_act_long_kernel<kBf16, kFp8>), grid, block, 0, st, x, s, M, K, xq, xs);
    return hipGetLastError();
}

template <bool kBf16, bool kFp8>
hipError_t quant_weight_dispatch(const void* w, int64_t K, int64_t N, const float* s, const float* amax,
                                 uint8_t* wq, hipStream_t st) {
    dim3 grid(static_cast<unsigned>((N + kTN - 1) / kTN), static_cast<unsigned>((K + kTJ - 1) / kTJ));
    if (N % 8 == 0) hipLaunchKernelGGL((quant_weight_t_kernel<kBf16, kFp8, true>), grid, dim3(256), 0, st, w, K, N, s, amax, wq);
    else hipLaunchKernelGGL((quant_weight_t_kernel<kBf16, kFp8, false>), grid, dim3(256), 0, st, w, K, N, s, amax, wq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, const float* s, bool fp8,
                            uint8_t* xq, float* x_scale, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (bf16) return fp8 ? quant_act_dispatch<true, true>(x, M, K, s, xq, x_scale, st)
                         : quant_act_dispatch<true, false>(x, M, K, s, xq, x_scale, st);
    return fp8 ? quant_act_dispatch<false, true>(x, M, K, s, xq, x_scale, st)
               : quant_act_dispatch<false, false>(x, M, K, s, xq, x_scale, st);
}

hipError_t launch_quant_weight_t(const void* w, bool bf16, int64_t K, int64_t N, const float* s,
                                 const float* amax, bool fp8, uint8_t* wq, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    if (bf16) return fp8 ? quant_weight_dispatch<true, true>(w, K, N, s, amax, wq, st)
                         : quant_weight_dispatch<true, false>(w, K, N, s, amax, wq, st);
    return fp8 ? quant_weight_dispatch<false, true>(w, K, N, s, amax, wq, st)
               : quant_weight_dispatch<false, false>(w, K, N, s, amax, wq, st);
}

hipError_t launch_finalize_scales(float* p, int64_t n, bool fp8, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(finalize_scales_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       p, n, fp8 ? 448.0f : 127.0f);
    return hipGetLastError();
}

}  // namespace w8a8
