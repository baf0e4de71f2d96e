// Quantized GEMM with the dequantizing epilogue on the gfx950 matrix cores.
// ("Weight-Activation Quantization", section 3 step 2: Y = dequantize(X_int8 @ W_int8); section 4:
// x^ = s q for E4M3.)
//
// Both operands are K-contiguous: xq [M, K] and wq [N, K].  The matrix-core instructions are
//   INT8: v_mfma_i32_16x16x64_i8          (int32 accumulate, exact)
//   E4M3: v_mfma_f32_16x16x128_f8f6f4     (fp32 accumulate; e4m3 x e4m3 products are exact)
// Each lane feeds 16 (INT8) or 32 (E4M3) consecutive K bytes of one row of each operand; the
// instruction pairs the bytes of A and B the same way, so any assignment of K to lanes that is
// the same for both operands gives the full dot product.
//
// The W tile is the instruction's A operand and the X tile its B operand, so the 16x16 result
// block held by a lane is Y[m = lane % 16][n = 4 * (lane / 16) + r], r = 0..3: four consecutive
// outputs of one row, stored as one 8-byte write after the epilogue.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace w8a8 {

namespace {

// ------------------------------------------------------------------------------------------------
// Large-M kernel: block tile kBM x kBN, K step 128 bytes, 4 waves in a 2 x 2 grid, each wave
// kBM/2 x kBN/2.  Tiles are staged global -> registers -> LDS with two LDS buffers (one barrier per
// K step).  LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored at position
// c ^ (r & 7), so the 8 lanes of a 128-byte LDS phase (8 consecutive rows, same chunk) hit 8
// different bank groups on both the writes and the fragment reads.
// ------------------------------------------------------------------------------------------------
constexpr int kBK = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

template <int kRows>
struct TileLoad {
    static constexpr int kPerThread = kRows * (kBK / 16) / kThreads;
    v4i reg[kPerThread];

    // Rows beyond `rows` re-read the last valid row (their results are never stored); chunks at
    // or beyond K read as zero, which adds nothing to any dot product.
    __device__ __forceinline__ void load(const uint8_t* __restrict__ g, int64_t row0, int64_t rows, int64_t K,
                                         int64_t k0, bool full_k) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int idx = threadIdx.x + kThreads * i;
            const int r = idx >> 3, c = idx & 7;
            int64_t gr = row0 + r;
            gr = gr < rows ? gr : rows - 1;
            const int64_t k = k0 + c * 16;
            if (full_k || k < K) reg[i] = *reinterpret_cast<const v4i*>(g + gr * K + k);
            else reg[i] = v4i{0, 0, 0, 0};
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int idx = threadIdx.x + kThreads * i;
            *reinterpret_cast<v4i*>(lds + swz(idx >> 3, idx & 7)) = reg[i];
        }
    }
};

// Map the linear block id to a (tile_m, tile_n) pair.  Consecutive block ids are dispatched to
// the 8 XCDs in turn; the remap gives each XCD a contiguous range of the grouped tile order, and
// the grouped order walks `group_m` tile rows before moving to the next tile column, so the blocks
// sharing one XCD's L2 share operand tiles.
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_m, int tiles_n, int group_m,
                                              int& tm, int& tn) {
    const int full = (nblocks / 8) * 8;
    if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
    const int per_group = group_m * tiles_n;
    const int g = bid / per_group;
    const int first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int in = bid % per_group;
    tm = first_m + in % gm;
    tn = in / gm;
}

template <bool kFp8>
struct Mfma;

template <>
struct Mfma<false> {
    using Acc = v4i;
    static constexpr int kKStep = 64;     // bytes of K per instruction
    static constexpr int kChunks = 1;     // 16-byte chunks per lane per instruction
    __device__ static __forceinline__ Acc zero() { return Acc{0, 0, 0, 0}; }
    __device__ static __forceinline__ Acc run(const v4i (&a)[1], const v4i (&b)[1], Acc c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[0], c, 0, 0, 0);
    }
    __device__ static __forceinline__ float to_float(int v) { return static_cast<float>(v); }
};

template <>
struct Mfma<true> {
    using Acc = v4f;
    static constexpr int kKStep = 128;
    static constexpr int kChunks = 2;
    __device__ static __forceinline__ Acc zero() { return Acc{0.f, 0.f, 0.f, 0.f}; }
    __device__ static __forceinline__ Acc run(const v4i (&a)[2], const v4i (&b)[2], Acc c) {
        v8i a8 = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
        v8i b8 = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
        // format codes 0, 0: both operands OCP E4M3; scale operands 0 select the unscaled form.
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, 0, 0, 0, 0, 0, 0);
    }
    __device__ static __forceinline__ float to_float(float v) { return v; }
};

// Dequantize and store four consecutive outputs of row m starting at column n.
template <bool kFp8, bool kOutAcc, typename Acc>
__device__ __forceinline__ void store4(const Acc& acc, int64_t m, int64_t n, int64_t M, int64_t N,
                                       float sxm, const float* __restrict__ w_scale, uint16_t* __restrict__ y,
                                       void* __restrict__ out_acc) {
    if (m >= M) return;
    if constexpr (kOutAcc) {
        using T = typename std::remove_cv<typename std::remove_reference<decltype(acc[0])>::type>::type;
        T* p = static_cast<T*>(out_acc) + m * N + n;
        if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<Acc*>(p) = acc;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) p[r] = acc[r];
        }
    } else {
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float swn = (n + r < N) ? w_scale[n + r] : 0.0f;
            h[r] = bf16_bits((Mfma<kFp8>::to_float(acc[r]) * sxm) * swn);
        }
        uint16_t* p = y + m * N + n;
        if (n + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<uint2*>(p) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N) p[r] = static_cast<uint16_t>(h[r]);
        }
    }
}

template <int kBM, int kBN, bool kFp8, bool kOutAcc>
__global__ __launch_bounds__(kThreads, 1) void gemm_tile_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc, int tiles_m, int tiles_n, int group_m) {
    using MF = Mfma<kFp8>;
    using Acc = typename MF::Acc;
    constexpr int kWM = kBM / 2, kWN = kBN / 2;
    constexpr int kMT = kWM / 16, kNT = kWN / 16;
    __shared__ __attribute__((aligned(16))) uint8_t lds_x[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint8_t lds_w[2][kBN * kBK];

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int wm = wave >> 1, wn = wave & 1;

    Acc acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = MF::zero();

    TileLoad<kBM> gx;
    TileLoad<kBN> gw;
    const int nk = static_cast<int>((K + kBK - 1) / kBK);
    const bool ragged_k = (K % kBK) != 0;

    gx.load(xq, m0, M, K, 0, !(ragged_k && nk == 1));
    gw.load(wq, n0, N, K, 0, !(ragged_k && nk == 1));
    gx.store(lds_x[0]);
    gw.store(lds_w[0]);
    __syncthreads();

    const int frag_row = lane & 15, frag_grp = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const bool full = !(ragged_k && kt + 2 == nk);
            gx.load(xq, m0, M, K, static_cast<int64_t>(kt + 1) * kBK, full);
            gw.load(wq, n0, N, K, static_cast<int64_t>(kt + 1) * kBK, full);
        }
        const uint8_t* lx = lds_x[cur];
        const uint8_t* lw = lds_w[cur];
#pragma unroll
        for (int ks = 0; ks < kBK / MF::kKStep; ++ks) {
            v4i fx[kMT][MF::kChunks], fw[kNT][MF::kChunks];
#pragma unroll
            for (int c = 0; c < MF::kChunks; ++c) {
                const int chunk = ks * (MF::kKStep / 16) + frag_grp * MF::kChunks + c;
#pragma unroll
                for (int i = 0; i < kMT; ++i)
                    fx[i][c] = *reinterpret_cast<const v4i*>(lx + swz(wm * kWM + i * 16 + frag_row, chunk));
#pragma unroll
                for (int j = 0; j < kNT; ++j)
                    fw[j][c] = *reinterpret_cast<const v4i*>(lw + swz(wn * kWN + j * 16 + frag_row, chunk));
            }
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j) acc[i][j] = MF::run(fw[j], fx[i], acc[i][j]);
        }
        if (more) {
            gx.store(lds_x[cur ^ 1]);
            gw.store(lds_w[cur ^ 1]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < kMT; ++i) {
        const int64_t m = m0 + wm * kWM + i * 16 + frag_row;
        const float sxm = (!kOutAcc && m < M) ? x_scale[m] : 0.0f;
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int64_t n = n0 + wn * kWN + j * 16 + frag_grp * 4;
            store4<kFp8, kOutAcc>(acc[i][j], m, n, M, N, sxm, w_scale, y, out_acc);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Small-M kernel (decode-shaped: M <= 16 * kMT).  The GEMM is bound by reading W once, so a block
// owns 16 output columns and all of K, its 4 waves take interleaved K steps, operands come straight
// from global memory (X is small and stays in cache), and the 4 partial sums are added in LDS at
// the end (exact for INT8).  N / 16 blocks keep every CU streaming.
// ------------------------------------------------------------------------------------------------
template <int kMT, bool kFp8, bool kOutAcc>
__global__ __launch_bounds__(kThreads) void gemm_small_m_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc) {
    using MF = Mfma<kFp8>;
    using Acc = typename MF::Acc;
    __shared__ Acc red[3][kMT][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int frag_row = lane & 15, frag_grp = lane >> 4;
    int64_t nrow = n0 + frag_row;
    nrow = nrow < N ? nrow : N - 1;
    const uint8_t* wrow = wq + nrow * K;
    const uint8_t* xrow[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
        int64_t m = static_cast<int64_t>(i) * 16 + frag_row;
        m = m < M ? m : M - 1;
        xrow[i] = xq + m * K;
    }
    Acc acc[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) acc[i] = MF::zero();

    const int64_t nsteps = (K + MF::kKStep - 1) / MF::kKStep;
    for (int64_t st = wave; st < nsteps; st += 4) {
        v4i fw[MF::kChunks], fx[kMT][MF::kChunks];
#pragma unroll
        for (int c = 0; c < MF::kChunks; ++c) {
            const int64_t k = st * MF::kKStep + (frag_grp * MF::kChunks + c) * 16;
            const bool ok = k < K;
            fw[c] = ok ? *reinterpret_cast<const v4i*>(wrow + k) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                fx[i][c] = ok ? *reinterpret_cast<const v4i*>(xrow[i] + k) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i) acc[i] = MF::run(fw, fx[i], acc[i]);
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < kMT; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            Acc a = acc[i];
#pragma unroll
            for (int w = 0; w < 3; ++w) a += red[w][i][lane];
            const int64_t m = static_cast<int64_t>(i) * 16 + frag_row;
            const float sxm = (!kOutAcc && m < M) ? x_scale[m] : 0.0f;
            store4<kFp8, kOutAcc>(a, m, n0 + frag_grp * 4, M, N, sxm, w_scale, y, out_acc);
        }
    }
}

template <bool kFp8, bool kOutAcc>
hipError_t gemm_dispatch(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, void* out_acc, hipStream_t st) {
    if (M <= 64) {
        dim3 grid(static_cast<unsigned>((N + 15) / 16));
        if (M <= 16)
            hipLaunchKernelGGL((gemm_small_m_kernel<1, kFp8, kOutAcc>), grid, dim3(kThreads), 0, st, xq, x_scale, wq,
                               w_scale, M, N, K, y, out_acc);
        else if (M <= 32)
            hipLaunchKernelGGL((gemm_small_m_kernel<2, kFp8, kOutAcc>), grid, dim3(kThreads), 0, st, xq, x_scale, wq,
                               w_scale, M, N, K, y, out_acc);
        else
            hipLaunchKernelGGL((gemm_small_m_kernel<4, kFp8, kOutAcc>), grid, dim3(kThreads), 0, st, xq, x_scale, wq,
                               w_scale, M, N, K, y, out_acc);
        return hipGetLastError();
    }
    constexpr int kBM = 256, kBN = 128;
    const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
    const int tiles_n = static_cast<int>((N + kBN - 1) / kBN);
    const int group_m = 4;
    hipLaunchKernelGGL((gemm_tile_kernel<kBM, kBN, kFp8, kOutAcc>), dim3(tiles_m * tiles_n), dim3(kThreads), 0, st,
                       xq, x_scale, wq, w_scale, M, N, K, y, out_acc, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, bool fp8,
                       int64_t M, int64_t N, int64_t K, uint16_t* y, void* out_acc, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (out_acc) {
        if (fp8) return gemm_dispatch<true, true>(xq, nullptr, wq, nullptr, M, N, K, nullptr, out_acc, st);
        return gemm_dispatch<false, true>(xq, nullptr, wq, nullptr, M, N, K, nullptr, out_acc, st);
    }
    if (fp8) return gemm_dispatch<true, false>(xq, x_scale, wq, w_scale, M, N, K, y, nullptr, st);
    return gemm_dispatch<false, false>(xq, x_scale, wq, w_scale, M, N, K, y, nullptr, st);
}

}  // namespace w8a8
