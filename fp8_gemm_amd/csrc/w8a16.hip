// Weight-only W8A16 GEMM: 16-bit (bf16) X times INT8 weights converted to bf16 on the fly, on the
// bf16 matrix cores ("Weight-Activation Quantization", s1 "Why Quantize Activations Too?": the
// weight-only GEMM still runs in 16-bit; the W8A16-vs-W8A8 lesson, s1: 8-bit weights are
// dequantized to 16-bit on the fly and the multiply runs on the 16-bit cores).
//
//   y[m, n] = bf16(sw[n] * sum_k x[m, k] * q[n, k])
//
// A code q (|q| <= 127) is exact in bf16, so the weights are converted, not rounded, and the
// per-output-channel scale multiplies the fp32 sum in the epilogue (the dequantized weight q * sw
// factors out of the sum over k).  Products of a bf16 value and a small integer are exact in fp32;
// the summation is the matrix cores'.
//
// v_mfma_f32_16x16x32_bf16: A = a 16 (output channels) x 32 (k) block of W, B = a 16 (rows of X) x
// 32 (k) block of X; lane l supplies row l % 16 and 8 k of each operand (8 codes converted to bf16,
// and 8 bf16 of X).  Results: lane l holds row m = l % 16 and columns n = 4 (l / 16) + r, r = 0..3.
// The instruction pairs the k of A and B lane by lane, so any assignment of k to lanes that is the
// same for both operands gives the dot product.  K is taken in chunks of 64: lane group g = l / 16
// owns k = 16 g .. 16 g + 15 of a chunk, 16 contiguous codes (one 16-byte load, 64 contiguous bytes
// per row per instruction) and 16 contiguous bf16 of X, and feeds the first 8 to one instruction
// and the last 8 to the next.
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace w8a8 {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
constexpr int kChunk = 64;              // k per chunk: two instructions
constexpr int kThreads16 = 256;         // 4 waves

// Eight int8 codes -> eight bf16 (exact): a sign-extending byte convert each (one SDWA
// instruction), then pairs packed to bf16.
__device__ __forceinline__ v8bf codes_to_bf16(uint2 w) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[i] = static_cast<float>(static_cast<int8_t>(w.x >> (8 * i)));
        f[4 + i] = static_cast<float>(static_cast<int8_t>(w.y >> (8 * i)));
    }
    const uint4 u = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                               pack_bf16x2(f[6], f[7]));
    return __builtin_bit_cast(v8bf, u);
}

__device__ __forceinline__ v8bf as_bf16x8(uint4 u) { return __builtin_bit_cast(v8bf, u); }

__device__ __forceinline__ v4f mma_bf16(v8bf w, v8bf x, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, x, c, 0, 0, 0);
}

// One 64-k chunk: 16 codes of W (w) and 16 bf16 of X (x0 = the first 8, x1 = the last 8).
__device__ __forceinline__ v4f mma_chunk(uint4 w, uint4 x0, uint4 x1, v4f c) {
    c = mma_bf16(codes_to_bf16(make_uint2(w.x, w.y)), as_bf16x8(x0), c);
    return mma_bf16(codes_to_bf16(make_uint2(w.z, w.w)), as_bf16x8(x1), c);
}

// The scales of four consecutive columns n .. n + 3 (0 past N).
__device__ __forceinline__ v4f load_scales4(const float* __restrict__ w_scale, int64_t n, int64_t N) {
    v4f sc;
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (n + r < N) ? w_scale[n + r] : 0.0f;
    return sc;
}

// The same without branches: columns past N repeat column N - 1 (their outputs are not stored).
__device__ __forceinline__ v4f load_scales4_clamped(const float* __restrict__ w_scale, int64_t n, int64_t N) {
    v4f sc;
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = w_scale[n + r < N ? n + r : N - 1];
    return sc;
}

// y = bf16(acc[r] * sc[r]) for four consecutive columns n of row m.
__device__ __forceinline__ void store_w8a16(const v4f& acc, const v4f& sc, int64_t m, int64_t n, int64_t M, int64_t N,
                                            uint16_t* __restrict__ y) {
    if (m >= M) return;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[r] * sc[r];
    const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
    uint16_t* p = y + m * N + n;
    if (n + 3 < N && (N & 3) == 0) {
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    } else {
        const uint16_t h[4] = {static_cast<uint16_t>(lo), static_cast<uint16_t>(lo >> 16), static_cast<uint16_t>(hi),
                               static_cast<uint16_t>(hi >> 16)};
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (n + r < N) p[r] = h[r];
    }
}

// ------------------------------------------------------------------------------------------------
// Decode kernel (M <= 16, K = kWaves * kS * 64): bound by reading W once.  Each wave owns a
// contiguous 1/kWaves of K and holds its X fragments for it in registers for the whole kernel; a
// block walks the 16-column output tiles t = blockIdx.x, blockIdx.x + gridDim.x, ..., loads a
// tile's codes, runs them through the matrix cores and adds the waves' partial sums in LDS.  The
// weights are single-buffered so that two blocks fit on a CU (at most 128 VGPRs): while one block
// waits for its codes the other computes.  The block's outputs stay in LDS and are stored after
// its last tile (a store in the loop would make every later wait for a load a wait for all
// outstanding memory operations, which the counter does not order against stores).
// ------------------------------------------------------------------------------------------------
constexpr int kMaxTiles = 32;

template <int kWaves, int kS>
__global__ __launch_bounds__(kWaves * kWave, 2) void w8a16_decode_kernel(const uint16_t* __restrict__ x,
                                                                          const int8_t* __restrict__ wq,
                                                                          const float* __restrict__ w_scale,
                                                                          int64_t M, int64_t N, int64_t K,
                                                                          uint16_t* __restrict__ y) {
    __shared__ v4f red[kWaves - 1][kWave];
    __shared__ __attribute__((aligned(16))) uint16_t ybuf[kMaxTiles][16][16];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int frag_row = lane & 15, frag_grp = lane >> 4;
    const int64_t kw0 = static_cast<int64_t>(wave) * kS * kChunk + 16 * frag_grp;
    const int ntiles = static_cast<int>((N + 15) / 16);
    const int G = static_cast<int>(gridDim.x);

    uint4 fx[kS][2];
    {
        const int64_t m = frag_row < M ? frag_row : M - 1;
        const uint16_t* xr = x + m * K + kw0;
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            fx[s][0] = *reinterpret_cast<const uint4*>(xr + s * kChunk);
            fx[s][1] = *reinterpret_cast<const uint4*>(xr + s * kChunk + 8);
        }
    }
    for (int t = blockIdx.x, j = 0; t < ntiles; t += G, ++j) {
        const int64_t n0 = static_cast<int64_t>(t) * 16 + 4 * frag_grp;
        const v4f sc = load_scales4_clamped(w_scale, n0, N);
        uint4 fw[kS];
        int64_t n = static_cast<int64_t>(t) * 16 + frag_row;
        n = n < N ? n : N - 1;
        const int8_t* wr = wq + n * K + kw0;
#pragma unroll
        for (int s = 0; s < kS; ++s) fw[s] = *reinterpret_cast<const uint4*>(wr + s * kChunk);
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < kS; ++s) acc = mma_chunk(fw[s], fx[s][0], fx[s][1], acc);
        if (wave > 0) red[wave - 1][lane] = acc;
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int w = 0; w < kWaves - 1; ++w) acc += red[w][lane];
            *reinterpret_cast<uint2*>(&ybuf[j][frag_row][4 * frag_grp]) =
                make_uint2(pack_bf16x2(acc[0] * sc[0], acc[1] * sc[1]), pack_bf16x2(acc[2] * sc[2], acc[3] * sc[3]));
        }
        __syncthreads();                 // red is reused by the next tile
    }
    const int nt = (ntiles - static_cast<int>(blockIdx.x) + G - 1) / G;
    store_tiles_bf16(ybuf, nt, blockIdx.x, G, M, N, y);
}

// ------------------------------------------------------------------------------------------------
// General kernel (any M, any K): a block owns 16 output columns and 16 kMT rows; its 4 waves take
// contiguous ranges of 64-wide K chunks, load both operands straight from global memory, and add
// their partial sums in LDS.  The k of a partial last chunk past K (K % 64 = 16, 32 or 48: whole
// 16-k pieces) use zero operands.  It is a correct general path, not a fast one past a few rows:
// without LDS tiling every 16-row fragment comes from L2 (about 140 TFLOP/s at M = 4096).
// ------------------------------------------------------------------------------------------------
template <int kMT>
__global__ __launch_bounds__(kThreads16) void w8a16_kernel(const uint16_t* __restrict__ x,
                                                           const int8_t* __restrict__ wq,
                                                           const float* __restrict__ w_scale, int64_t M, int64_t N,
                                                           int64_t K, uint16_t* __restrict__ y) {
    __shared__ v4f red[3][kMT][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int frag_row = lane & 15, frag_grp = lane >> 4;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
    const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 16 * kMT;
    int64_t nrow = n0 + frag_row;
    nrow = nrow < N ? nrow : N - 1;
    const int8_t* wrow = wq + nrow * K + 16 * frag_grp;
    const uint16_t* xrow[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
        int64_t m = m0 + i * 16 + frag_row;
        m = m < M ? m : M - 1;
        xrow[i] = x + m * K + 16 * frag_grp;
    }
    v4f acc[kMT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) acc[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Full steps, kU at a time with every load issued first, in a contiguous range per wave; then
    // the remaining steps (and a partial last one) spread over the waves.
    constexpr int kU = kMT == 1 ? 4 : 2;
    const int64_t nfull = K / kChunk;
    const int64_t nsteps = (K + kChunk - 1) / kChunk;
    const int64_t per_w = (nfull / 4 / kU) * kU;
    int64_t st0 = wave * per_w;
    for (int64_t it = 0; it < per_w; it += kU, st0 += kU) {
        uint4 fw[kU];
        uint4 fx[kU][kMT][2];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t k = (st0 + u) * kChunk;
            fw[u] = *reinterpret_cast<const uint4*>(wrow + k);
#pragma unroll
            for (int i = 0; i < kMT; ++i) {
                fx[u][i][0] = *reinterpret_cast<const uint4*>(xrow[i] + k);
                fx[u][i][1] = *reinterpret_cast<const uint4*>(xrow[i] + k + 8);
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const v8bf w0 = codes_to_bf16(make_uint2(fw[u].x, fw[u].y));
            const v8bf w1 = codes_to_bf16(make_uint2(fw[u].z, fw[u].w));
#pragma unroll
            for (int i = 0; i < kMT; ++i) {
                acc[i] = mma_bf16(w0, as_bf16x8(fx[u][i][0]), acc[i]);
                acc[i] = mma_bf16(w1, as_bf16x8(fx[u][i][1]), acc[i]);
            }
        }
    }
    for (int64_t st = 4 * per_w + wave; st < nsteps; st += 4) {
        const int64_t k = st * kChunk;
        const bool ok = k + 16 * frag_grp < K;   // K % 16 == 0: a lane's 16 k are all in or all out
        const uint4 fw = ok ? *reinterpret_cast<const uint4*>(wrow + k) : make_uint4(0u, 0u, 0u, 0u);
        const v8bf w0 = codes_to_bf16(make_uint2(fw.x, fw.y));
        const v8bf w1 = codes_to_bf16(make_uint2(fw.z, fw.w));
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            const uint4 f0 = ok ? *reinterpret_cast<const uint4*>(xrow[i] + k) : z;
            const uint4 f1 = ok ? *reinterpret_cast<const uint4*>(xrow[i] + k + 8) : z;
            acc[i] = mma_bf16(w0, as_bf16x8(f0), acc[i]);
            acc[i] = mma_bf16(w1, as_bf16x8(f1), acc[i]);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < kMT; ++i) red[wave - 1][i][lane] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            v4f a = acc[i];
#pragma unroll
            for (int w = 0; w < 3; ++w) a += red[w][i][lane];
            store_w8a16(a, load_scales4(w_scale, n0 + 4 * frag_grp, N), m0 + i * 16 + frag_row, n0 + 4 * frag_grp, M,
                        N, y);
        }
    }
}

}  // namespace

hipError_t launch_gemm_w8a16(const uint16_t* x, const int8_t* wq, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    constexpr int kDecWaves = 8, kDecS = 8;
    if (M <= 16 && K == kDecWaves * kDecS * kChunk) {
        // Two blocks per CU walking their tiles, at most kMaxTiles of them per block.
        const int64_t ntiles = (N + 15) / 16;
        const int64_t grid = std::min<int64_t>(ntiles, std::max<int64_t>(512, (ntiles + kMaxTiles - 1) / kMaxTiles));
        hipLaunchKernelGGL((w8a16_decode_kernel<kDecWaves, kDecS>), dim3(static_cast<unsigned>(grid)),
                           dim3(kDecWaves * kWave), 0, st, x, wq, w_scale, M, N, K, y);
        return hipGetLastError();
    }
    if (M <= 16) {
        hipLaunchKernelGGL((w8a16_kernel<1>), dim3(static_cast<unsigned>((N + 15) / 16), 1), dim3(kThreads16), 0, st, x,
                           wq, w_scale, M, N, K, y);
    } else {
        hipLaunchKernelGGL((w8a16_kernel<4>), dim3(static_cast<unsigned>((N + 15) / 16), static_cast<unsigned>((M + 63) / 64)),
                           dim3(kThreads16), 0, st, x, wq, w_scale, M, N, K, y);
    }
    return hipGetLastError();
}

}  // namespace w8a8
