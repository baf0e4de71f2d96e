// Calibration reductions and SmoothQuant factors ("Weight-Activation Quantization", section 3,
// "Choosing the Smoothing Factor": s_j = max|X_j|^alpha / max|W_j|^(1-alpha)).
//
// Both reductions are HBM-bound streams.  Loads are 16 bytes per lane (8 bf16 or 2x4 fp32), a
// wave covers 512 consecutive columns of a row, and every maximum is exact (fp32 max needs no
// rounding), so the result does not depend on how the work is split.
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int kColsPerWave = 8 * kWave;   // 512 columns: one 16-byte chunk of 8 elements per lane
constexpr int kRowsPerBlock = 32;         // 4 waves x 8 rows each

__global__ void fill_kernel(float* p, int64_t n, float v) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Zeroes p[0, n) and q[0, m) in one launch.
__global__ void zero2_kernel(float* p, int64_t n, float* q, int64_t m) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
    else if (i - n < m) q[i - n] = 0.0f;
}

template <bool kBf16>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
    if constexpr (kBf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
    else return static_cast<const float*>(base)[i];
}

// 8 elements starting at column c of a row, c < C.  kVec: the row is 16-byte aligned and C is a
// multiple of 8, so the chunk is inside the row; otherwise columns past C re-read column C - 1
// (harmless for a maximum).  Loads are unconditional so that a wave's loads are all in flight
// together.
template <bool kBf16, bool kVec>
__device__ __forceinline__ void load_chunk(const void* base, int64_t row_start, int64_t c, int64_t C,
                                           float (&v)[8]) {
    if constexpr (kVec) {
        load8<kBf16>(base, row_start + c, v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = load1<kBf16>(base, row_start + (c + e < C ? c + e : C - 1));
    }
}

// Column maxima of |a[r, c] * row_scale[r]| over a block of kRowsPerBlock rows and 512 columns,
// merged across waves in LDS and across blocks with an atomic maximum.  Rows past R re-read row
// R - 1 and columns past C re-read the last chunk: duplicates do not change a maximum.  With
// divisor != 0 the block maxima are divided by it before they are merged: correctly rounded
// division is monotone, so the merged value is the maximum divided by divisor, rounded once.
//
// The body serves a block of 4 waves (bx, by) = (column block, row block); row_scale[i] is the
// factor of row r0 + i of the block (rows past R use that of row R - 1).  pre() runs once the
// block's loads are in flight and before the factors are read (the fold computes them there).
template <bool kBf16, bool kVec, bool kScaled, typename Pre>
__device__ __forceinline__ void cols_body(const void* __restrict__ a, int64_t R, int64_t C,
                                          const float* row_scale, float divisor, float* __restrict__ out,
                                          int64_t bx, int64_t by, float (*part)[kColsPerWave], Pre pre) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t c = bx * kColsPerWave + lane * 8;
    const int64_t cl = c < C ? c : (kVec ? C - 8 : C - 1);
    const int64_t r0 = by * kRowsPerBlock;
    constexpr int kRows = kRowsPerBlock / 4;
    float v[kRows][8];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        int64_t r = r0 + wave + 4 * i;
        r = r < R ? r : R - 1;
        load_chunk<kBf16, kVec>(a, r * C, cl, C, v[i]);
    }
    pre();
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        float rs = 1.0f;
        if constexpr (kScaled) {
            const int64_t r = r0 + wave + 4 * i;
            rs = row_scale[(r < R ? r : R - 1) - r0];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf(kScaled ? rs * v[i][e] : v[i][e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave][lane * 8 + e] = m[e];
    __syncthreads();
    for (int i = threadIdx.x; i < kColsPerWave; i += 4 * kWave) {
        const int64_t col = bx * kColsPerWave + i;
        if (col < C) {
            float mv = fmaxf(fmaxf(part[0][i], part[1][i]), fmaxf(part[2][i], part[3][i]));
            if (divisor != 0.0f) mv = div_rn(mv, divisor);
            atomic_max_nonneg(out + col, mv);
        }
    }
}

struct NoPre {
    __device__ void operator()() const {}
};

template <bool kBf16, bool kVec, bool kScaled>
__global__ __launch_bounds__(256) void absmax_cols_kernel(const void* __restrict__ a, int64_t R, int64_t C,
                                                          const float* __restrict__ row_scale, float divisor,
                                                          float* __restrict__ out) {
    __shared__ float part[4][kColsPerWave];
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kRowsPerBlock;
    cols_body<kBf16, kVec, kScaled>(a, R, C, kScaled ? row_scale + r0 : nullptr, divisor, out, blockIdx.x, blockIdx.y,
                                    part, NoPre{});
}

// s_j = ax^alpha / aw^(1-alpha).  alpha = 0.5: correctly rounded roots and division; alpha = 1 and
// alpha = 0 reduce to ax and 1/aw exactly; otherwise pow in double, rounded once to fp32.
__device__ __forceinline__ float smooth_factor(float a, float b, float alpha) {
    if (a == 0.0f || b == 0.0f) return 1.0f;
    if (alpha == 0.5f) return div_rn(__builtin_sqrtf(a), __builtin_sqrtf(b));
    if (alpha == 1.0f) return a;
    if (alpha == 0.0f) return div_rn(1.0f, b);
    return static_cast<float>(pow(static_cast<double>(a), static_cast<double>(alpha)) /
                              pow(static_cast<double>(b), 1.0 - static_cast<double>(alpha)));
}

// Row maxima: one wave per row, 8 chunks of 16 bytes in flight per lane per iteration (chunks past
// the row end re-read the last one).  With ax != NULL the row index is the channel j of the
// smoothing factors and the wave also writes s[j] = smooth_factor(ax[j], max_n |W[j, n]|, alpha);
// ax is complete when this kernel starts (the column maxima are computed by an earlier launch on
// the same stream).
template <bool kBf16, bool kVec>
__device__ __forceinline__ void rows_body(const void* __restrict__ a, int64_t R, int64_t C, float* __restrict__ out,
                                          const float* __restrict__ ax, float alpha, float* __restrict__ s,
                                          int64_t bx) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t r = bx * 4 + wave;
    if (r >= R) return;
    const int64_t last = kVec ? C - 8 : C - 1;
    float m = 0.0f;
    for (int64_t c0 = static_cast<int64_t>(lane) * 8; c0 < C; c0 += 8 * kColsPerWave) {
        float v[8][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t c = c0 + u * kColsPerWave;
            load_chunk<kBf16, kVec>(a, r * C, c < C ? c : last, C, v[u]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
    }
    m = wave_max(m);
    if (lane == 0) {
        out[r] = m;
        if (ax) s[r] = smooth_factor(ax[r], m, alpha);
    }
}

template <bool kBf16, bool kVec>
__global__ __launch_bounds__(256) void absmax_rows_kernel(const void* __restrict__ a, int64_t R, int64_t C,
                                                          float* __restrict__ out, const float* __restrict__ ax,
                                                          float alpha, float* __restrict__ s) {
    rows_body<kBf16, kVec>(a, R, C, out, ax, alpha, s, blockIdx.x);
}

// ---- the calibration and fold passes of one layer, fused by launch ----------------------------
// The column maxima of X and the row maxima of W read different tensors and depend on nothing, so
// one launch runs both: blocks [0, nx) are column blocks of X (gx across, by rows), merged into the
// zeroed ax with atomic maxima, the rest row blocks of W.  X rows must be whole 16-byte chunks
// (K % 8 == 0) and so must W rows (N % 8 == 0).  (Partial maxima reduced by the next launch instead
// of the zeroing launch and the atomics were measured slower: the fold's blocks then read them.  So
// was one block of 16 waves per 64-column strip of X reading all of its rows at once, which stores
// ax without a merge and lets the zeroing move into this launch: at 2048 x 4096 the call took 42.5
// instead of 39.9 us, the 64 long strip blocks outlasting the rest of the grid.)
template <bool kBf16>
__global__ __launch_bounds__(256) void calib_pair_kernel(const void* __restrict__ x, int64_t M, int64_t K,
                                                         const void* __restrict__ w, int64_t N, float* __restrict__ ax,
                                                         float* __restrict__ aw, unsigned gx, unsigned nx) {
    __shared__ float part[4][kColsPerWave];
    if (blockIdx.x < nx)
        cols_body<kBf16, true, false>(x, M, K, nullptr, 0.0f, ax, blockIdx.x % gx, blockIdx.x / gx, part, NoPre{});
    else
        rows_body<kBf16, true>(w, K, N, aw, nullptr, 0.0f, nullptr, blockIdx.x - nx);
}

// Column maxima of W~ = s W divided by Q (the weight scales, merged into the zeroed w_scale with
// atomic maxima), with s[j] = smooth_factor(ax[j], aw[j]) computed by each block for its own rows
// while its loads are in flight; the blocks of the first column block also write s.  ax and aw are
// complete (an earlier launch on the stream).
template <bool kBf16>
__global__ __launch_bounds__(256) void fold_cols_kernel(const void* __restrict__ w, int64_t K, int64_t N,
                                                        const float* __restrict__ ax, const float* __restrict__ aw,
                                                        float alpha, float divisor, float* __restrict__ s,
                                                        float* __restrict__ w_scale) {
    __shared__ float part[4][kColsPerWave];
    __shared__ float srow[kRowsPerBlock];
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kRowsPerBlock;
    auto pre = [&]() {
        if (threadIdx.x < kRowsPerBlock) {
            const int64_t j = r0 + threadIdx.x;
            const int64_t jc = j < K ? j : K - 1;
            const float sv = smooth_factor(ax[jc], aw[jc], alpha);
            srow[threadIdx.x] = sv;
            if (blockIdx.x == 0 && j < K) s[j] = sv;
        }
        __syncthreads();
    };
    cols_body<kBf16, true, true>(w, K, N, srow, divisor, w_scale, blockIdx.x, blockIdx.y, part, pre);
}

__global__ void smooth_factors_kernel(const float* __restrict__ ax, const float* __restrict__ aw, int64_t K,
                                      float alpha, float* __restrict__ s) {
    int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j >= K) return;
    s[j] = smooth_factor(ax[j], aw[j], alpha);
}

// Maximum of |a| over a whole tensor of nchunk 16-byte chunks (8 elements each), divided by
// divisor when it is not 0.  Block b streams its own contiguous range of chunks, 8 chunks in
// flight per thread (chunks past the range re-read its last one).  The block's maximum is merged
// into out[0] with an atomic maximum, skipped when out[0] already holds at least as much (out[0]
// only grows, so a stale read can only cause a redundant atomic, never a missed one).
template <bool kBf16>
__global__ __launch_bounds__(256) void absmax_tensor_kernel(const void* __restrict__ a, int64_t nchunk, float divisor,
                                                            float* __restrict__ out) {
    __shared__ float part[4];
    constexpr int kU = 8;
    const int64_t lo = block_range_lo(nchunk), hi = block_range_hi(nchunk);
    float m = 0.0f;
    for (int64_t c0 = lo + threadIdx.x; c0 < hi; c0 += kU * blockDim.x) {
        float v[kU][8];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t c = c0 + u * blockDim.x;
            load8<kBf16>(a, (c < hi ? c : hi - 1) * 8, v[u]);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[u][e]));
    }
    m = wave_max(m);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (lane == 0) part[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
        if (divisor != 0.0f) b = div_rn(b, divisor);
        if (b > *out) atomic_max_nonneg(out, b);
    }
}

template <bool kBf16, bool kVec>
void cols_launch(dim3 grid, const void* a, int64_t R, int64_t C, const float* row_scale, float divisor, float* out,
                 hipStream_t st) {
    if (row_scale)
        hipLaunchKernelGGL((absmax_cols_kernel<kBf16, kVec, true>), grid, dim3(256), 0, st, a, R, C, row_scale,
                           divisor, out);
    else
        hipLaunchKernelGGL((absmax_cols_kernel<kBf16, kVec, false>), grid, dim3(256), 0, st, a, R, C, row_scale,
                           divisor, out);
}

}  // namespace

hipError_t launch_zero2(float* p, int64_t n, float* q, int64_t m, hipStream_t st) {
    if (n + m <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero2_kernel, dim3(static_cast<unsigned>((n + m + 255) / 256)), dim3(256), 0, st, p, n, q, m);
    return hipGetLastError();
}

hipError_t launch_calib_pair(const void* x, const void* w, bool bf16, int64_t M, int64_t K, int64_t N, float* ax,
                             float* aw, hipStream_t st) {
    const int64_t gx = (K + kColsPerWave - 1) / kColsPerWave;
    const int64_t nx = gx * ((M + kRowsPerBlock - 1) / kRowsPerBlock);
    const int64_t nw = (K + 3) / 4;
    const dim3 grid(static_cast<unsigned>(nx + nw));
    if (bf16)
        hipLaunchKernelGGL(calib_pair_kernel<true>, grid, dim3(256), 0, st, x, M, K, w, N, ax, aw,
                           static_cast<unsigned>(gx), static_cast<unsigned>(nx));
    else
        hipLaunchKernelGGL(calib_pair_kernel<false>, grid, dim3(256), 0, st, x, M, K, w, N, ax, aw,
                           static_cast<unsigned>(gx), static_cast<unsigned>(nx));
    return hipGetLastError();
}

hipError_t launch_fold_cols(const void* w, bool bf16, int64_t K, int64_t N, const float* ax, const float* aw,
                            float alpha, float divisor, float* s, float* w_scale, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((N + kColsPerWave - 1) / kColsPerWave),
                    static_cast<unsigned>((K + kRowsPerBlock - 1) / kRowsPerBlock));
    if (bf16)
        hipLaunchKernelGGL(fold_cols_kernel<true>, grid, dim3(256), 0, st, w, K, N, ax, aw, alpha, divisor, s, w_scale);
    else
        hipLaunchKernelGGL(fold_cols_kernel<false>, grid, dim3(256), 0, st, w, K, N, ax, aw, alpha, divisor, s,
                           w_scale);
    return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, p, n, v);
    return hipGetLastError();
}

hipError_t launch_absmax_cols(const void* a, bool bf16, int64_t R, int64_t C, const float* row_scale,
                              float divisor, float* out, hipStream_t st) {
    if (R <= 0 || C <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((C + kColsPerWave - 1) / kColsPerWave),
              static_cast<unsigned>((R + kRowsPerBlock - 1) / kRowsPerBlock));
    const bool vec = (C % 8) == 0;
    if (bf16) {
        if (vec) cols_launch<true, true>(grid, a, R, C, row_scale, divisor, out, st);
        else cols_launch<true, false>(grid, a, R, C, row_scale, divisor, out, st);
    } else {
        if (vec) cols_launch<false, true>(grid, a, R, C, row_scale, divisor, out, st);
        else cols_launch<false, false>(grid, a, R, C, row_scale, divisor, out, st);
    }
    return hipGetLastError();
}

hipError_t launch_absmax_rows(const void* a, bool bf16, int64_t R, int64_t C, float* out, const float* ax,
                              float alpha, float* s, hipStream_t st) {
    if (R <= 0) return hipSuccess;
    dim3 grid(static_cast<unsigned>((R + 3) / 4));
    const bool vec = (C % 8) == 0;
    if (bf16) {
        if (vec) hipLaunchKernelGGL((absmax_rows_kernel<true, true>), grid, dim3(256), 0, st, a, R, C, out, ax, alpha, s);
        else hipLaunchKernelGGL((absmax_rows_kernel<true, false>), grid, dim3(256), 0, st, a, R, C, out, ax, alpha, s);
    } else {
        if (vec) hipLaunchKernelGGL((absmax_rows_kernel<false, true>), grid, dim3(256), 0, st, a, R, C, out, ax, alpha, s);
        else hipLaunchKernelGGL((absmax_rows_kernel<false, false>), grid, dim3(256), 0, st, a, R, C, out, ax, alpha, s);
    }
    return hipGetLastError();
}

hipError_t launch_absmax_tensor(const void* a, bool bf16, int64_t n, float divisor, float* out, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t nchunk = n / 8;
    // At most 256 blocks (one per CU): every block ends with one atomic on the same address, and
    // blocks that finish together queue behind each other there.  Fill + maximum, graph replay over
    // rotating buffers, at 1024 / 512 / 256 / 128 blocks: 33.5 MB 18.1 / 13.3 / 11.5 / 12.5 us,
    // 470 MB 85.5 / 85.1 / 82.0 / 106.9 us.
    const int64_t blocks = std::min<int64_t>((nchunk + 256 * 8 - 1) / (256 * 8), 256);
    if (bf16)
        hipLaunchKernelGGL(absmax_tensor_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a, nchunk,
                           divisor, out);
    else
        hipLaunchKernelGGL(absmax_tensor_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a, nchunk,
                           divisor, out);
    return hipGetLastError();
}

hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s,
                                 hipStream_t st) {
    hipLaunchKernelGGL(smooth_factors_kernel, dim3(static_cast<unsigned>((K + 255) / 256)), dim3(256), 0, st,
                       ax, aw, K, alpha, s);
    return hipGetLastError();
}

}  // namespace w8a8
