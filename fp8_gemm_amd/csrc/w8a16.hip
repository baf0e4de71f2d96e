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
// Small-M kernel (any K): a block owns 16 output columns and 16 kMT rows; its 4 waves take
// contiguous ranges of 64-wide K chunks, load both operands straight from global memory, and add
// their partial sums in LDS.  The k of a partial last chunk past K (K % 64 = 16, 32 or 48: whole
// 16-k pieces) use zero operands.  Without LDS tiling every 16-row fragment comes from L2, so it
// serves only a few rows (up to 128), where its N / 16 blocks keep the chip busy.
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

// ------------------------------------------------------------------------------------------------
// Tiled kernel (batches past the decode shape): a block owns a kBM x kBN output tile; its waves in a
// kGM x kGN grid own (kBM / kGM) x (kBN / kGN) each, as 32 x 32 blocks of v_mfma_f32_32x32x16_bf16
// (A = 32 output channels of W, B = 32 rows of X; lane l supplies row l % 32 and 8 k of each operand).
// 128 x 128 tiles take 4 waves of 64 x 64 (two blocks per CU); 256 x 256 tiles take 8 waves of
// 128 x 64 (one block per CU, two waves per SIMD), which moves a third less through LDS per product:
// per K step and CU, 128 KB of fragment reads and staging against 96 KB for two 128 x 128 blocks
// with the same matrix-core work halved.
// K is taken 32 at a time.  Both operands go through LDS as bf16: the W codes are converted once,
// while staged, so each W element is converted once per block and both tiles share one layout:
// 64 bytes per row and K step, as four 16-byte chunks; chunk c of row r is stored at chunk
// c ^ ((r >> 2) & 3), which makes the 16-lane phases of a fragment read (16 rows at one chunk)
// hit 16 different 16-byte bank groups.  Two LDS stages and two register sets for the global
// loads: the loads of step t + 2 go out when step t starts, and step t + 1's (loaded during step
// t - 1) are written to LDS when step t ends, so each load has two steps to land.  Rows past M or
// N re-read the last row (never stored); the k past K (K % 32 = 16) are zero.
// With kSK > 1 the block holds kSK groups of kGM x kGN waves, each with its own two stages, for
// shapes with too few tiles to keep the CUs' waves busy: group g takes K steps g, g + kSK, ..., and
// at the end groups 1.. hand their accumulators to group 0 through LDS, which adds them in group
// order (an fp32 sum whose order depends on the split, not on the run).
// ------------------------------------------------------------------------------------------------
typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kW8a16Big = 192;           // 256 x 256 tiles from this many on (three quarters of the CUs)
constexpr int64_t kW8a16SplitK4Tiles = 256, kW8a16SplitK2Tiles = 512;   // 64 x 64 tiles split K 4 or 2 ways
// 128 x 128 tiles with K split 2 ways (one block of 8 waves per CU) from 160 to 256 of them: fewer
// leave too many CUs idle, more need a second round of blocks.
constexpr int64_t kW8a16Split128Min = 160, kW8a16Split128Max = 256;
constexpr int kKS = 32;                  // k per step
constexpr int kRowBytes = kKS * 2;       // bytes per row and step (bf16)

__device__ __forceinline__ int tswz(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row >> 2) & 3)) << 4); }

template <int kBM, int kBN, int kGM, int kGN, int kSK, int kBlocksPerCU>
__global__ __launch_bounds__(kGM * kGN * kSK * kWave, kBlocksPerCU) void w8a16_tile_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ wq, const float* __restrict__ w_scale, int64_t M,
    int64_t N, int64_t K, uint16_t* __restrict__ y, int tiles_m, int tiles_n) {
    constexpr int kWM = kBM / kGM, kWN = kBN / kGN;         // each wave's outputs
    constexpr int kMT = kWM / 32, kNT = kWN / 32;           // 32 x 32 blocks per wave along M and N
    constexpr int kXChunks = kBM * 4, kWChunks = kBN * 2;  // 16-byte X chunks, 16-code W chunks per step
    constexpr int kWavesMN = kGM * kGN;
    constexpr int kThreads = kWavesMN * kWave;              // threads of one K group
    constexpr int kXPer = (kXChunks + kThreads - 1) / kThreads, kWPer = (kWChunks + kThreads - 1) / kThreads;
    constexpr int kXStage = kBM * kRowBytes, kWStage = kBN * kRowBytes;
    // After the K loop the same LDS takes the other K groups' accumulators, then each wave's bf16
    // output tile (rows padded to kOutStride).
    constexpr int kOutStride = kWN * 2 + 16;
    constexpr int kOutBytes = kWavesMN * kWM * kOutStride;
    constexpr int kStageBytes = 2 * (kXStage + kWStage);
    constexpr int kAccFloats = kMT * kNT * 16;
    constexpr int kPartBytes = (kSK - 1) * kWavesMN * kAccFloats * kWave * 4;
    constexpr int kSmem0 = kSK * kStageBytes > kOutBytes ? kSK * kStageBytes : kOutBytes;
    constexpr int kSmem = kSmem0 > kPartBytes ? kSmem0 : kPartBytes;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
    // K group: K steps group, group + kSK, ...  (0 when K is not split, known at compile time).
    const int group = kSK == 1 ? 0 : static_cast<int>(threadIdx.x) / kThreads;
    const int tid = kSK == 1 ? static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x) % kThreads;
    uint8_t* const xs = smem + group * kStageBytes;
    uint8_t* const ws = xs + 2 * kXStage;

    // XCD-aware order: consecutive block ids go to the 8 XCDs in turn; give each XCD a contiguous
    // range of tiles, walked 4 tile rows at a time, so the blocks sharing an L2 share operands.
    int bid = blockIdx.x;
    const int nblocks = gridDim.x, full = (nblocks / 8) * 8;
    if (bid < full) bid = (bid % 8) * (full / 8) + bid / 8;
    constexpr int kGroupM = 4;
    const int g = bid / (kGroupM * tiles_n), first = g * kGroupM;
    const int gm = min(tiles_m - first, kGroupM);
    const int in = bid % (kGroupM * tiles_n);
    const int64_t m0 = static_cast<int64_t>(first + in % gm) * kBM, n0 = static_cast<int64_t>(in / gm) * kBN;

    const unsigned utid = static_cast<unsigned>(tid);
    const int wave = utid / kWave, lane = utid % kWave;
    const int wm = wave / kGN, wn = wave % kGN;
    const int r32 = lane % 32, g32 = lane / 32;

    // Staging: X chunk p = tid + kThreads i is row p / 4, chunk p % 4 (8 bf16); W chunk p = tid +
    // kThreads i is row p / 2, half p % 2 (16 codes, two bf16 chunks).
    const uint16_t* xsrc[kXPer];
    int xl[kXPer], xk[kXPer];
#pragma unroll
    for (int i = 0; i < kXPer; ++i) {
        const int p = min(tid + kThreads * i, kXChunks - 1), row = p / 4, c = p % 4;
        const int64_t gr = min(m0 + row, M - 1);
        xsrc[i] = x + gr * K + c * 8;
        xl[i] = tswz(row, c);
        xk[i] = c * 8;
    }
    const int8_t* wsrc[kWPer];
    int wl[kWPer], wk[kWPer];
#pragma unroll
    for (int i = 0; i < kWPer; ++i) {
        const int p = min(tid + kThreads * i, kWChunks - 1), row = p / 2, h = p % 2;
        const int64_t gr = min(n0 + row, N - 1);
        wsrc[i] = wq + gr * K + h * 16;
        wl[i] = row;
        wk[i] = h * 16;
    }
    uint4 xr[2][kXPer], wr[2][kWPer];
    auto load = [&](int set, int t) {
        const int64_t k0 = (static_cast<int64_t>(t) * kSK + group) * kKS;
#pragma unroll
        for (int i = 0; i < kXPer; ++i)
            xr[set][i] = k0 + xk[i] < K ? *reinterpret_cast<const uint4*>(xsrc[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < kWPer; ++i)
            wr[set][i] = k0 + wk[i] < K ? *reinterpret_cast<const uint4*>(wsrc[i] + k0) : make_uint4(0u, 0u, 0u, 0u);
    };
    // Threads past the chunk count (small tiles) load a duplicate of the last chunk and store nothing.
    auto store = [&](int set, int stage) {
#pragma unroll
        for (int i = 0; i < kXPer; ++i)
            if (tid + kThreads * i < kXChunks) *reinterpret_cast<uint4*>(xs + stage * kXStage + xl[i]) = xr[set][i];
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            if (tid + kThreads * i >= kWChunks) continue;
            const int c0 = 2 * (wk[i] / 16);
            *reinterpret_cast<v8bf*>(ws + stage * kWStage + tswz(wl[i], c0)) =
                codes_to_bf16(make_uint2(wr[set][i].x, wr[set][i].y));
            *reinterpret_cast<v8bf*>(ws + stage * kWStage + tswz(wl[i], c0 + 1)) =
                codes_to_bf16(make_uint2(wr[set][i].z, wr[set][i].w));
        }
    };

    v16f acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = v16f{};

    // Steps of this K group (all groups take the same count; steps past K load zeros).
    const int nk = static_cast<int>(((K + kKS - 1) / kKS + kSK - 1) / kSK);
    // Register set t % 2 holds the loads of step t; LDS stage t % 2 the tile of step t.
    load(0, 0);
    if (nk > 1) load(1, 1);
    store(0, 0);
    __syncthreads();
    auto step = [&](int t, auto SET) {
        constexpr int set = decltype(SET)::value;   // t % 2, known at compile time
        const int stage = set;
        if (t + 2 < nk) load(set, t + 2);           // set t % 2 was stored at the end of step t - 1
        // instruction u of the step takes k 16 u .. 16 u + 15: lane group g32 supplies chunk 2 u + g32
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            v8bf fx[kMT], fw[kNT];
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                fx[i] = *reinterpret_cast<const v8bf*>(xs + stage * kXStage + tswz(wm * kWM + 32 * i + r32, 2 * u + g32));
#pragma unroll
            for (int j = 0; j < kNT; ++j)
                fw[j] = *reinterpret_cast<const v8bf*>(ws + stage * kWStage + tswz(wn * kWN + 32 * j + r32, 2 * u + g32));
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], fx[i], acc[i][j], 0, 0, 0);
        }
        if (t + 1 < nk) store(set ^ 1, stage ^ 1);   // step t + 1's loads; that stage was last read in step t - 1
        __syncthreads();
    };
    int t = 0;
    for (; t + 1 < nk; t += 2) {
        step(t, std::integral_constant<int, 0>{});
        step(t + 1, std::integral_constant<int, 1>{});
    }
    if (t < nk) step(t, std::integral_constant<int, 0>{});
    // Lane results of block (i, j): row m = m0 + wm kWM + 32 i + r32, columns
    // n = n0 + wn kWN + 32 j + 8 q + 4 g32 + r (r = 0..3) in acc[4 q + r].  They are scaled, rounded
    // to bf16 and staged in LDS, then written as 16-byte pieces of whole output rows with
    // nontemporal stores (the output is written once; cached stores would displace operand tiles
    // that other blocks still read).
    if constexpr (kSK > 1) {
        // K groups 1.. hand their accumulators to group 0 through LDS, which adds them in group order
        // (lane-major, so each access is 64 consecutive floats).
        __syncthreads();                 // every wave has finished reading the stages
        float* const part = reinterpret_cast<float*>(smem);
        if (group > 0) {
            float* const dst = part + ((group - 1) * kWavesMN + wave) * kAccFloats * kWave + lane;
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) dst[((i * kNT + j) * 16 + e) * kWave] = acc[i][j][e];
        }
        __syncthreads();
        if (group == 0) {
#pragma unroll
            for (int g2 = 1; g2 < kSK; ++g2) {
                const float* const src = part + ((g2 - 1) * kWavesMN + wave) * kAccFloats * kWave + lane;
#pragma unroll
                for (int i = 0; i < kMT; ++i)
#pragma unroll
                    for (int j = 0; j < kNT; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e) acc[i][j][e] += src[((i * kNT + j) * 16 + e) * kWave];
            }
        }
    }
    __syncthreads();                     // every wave has finished reading the stages (and the partial sums)
    uint8_t* const ot = smem + wave * (kWM * kOutStride);
    if (group == 0) {                    // group 0 holds the sums; the other groups only meet the barrier
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 32 * j + 8 * q + 4 * g32;
                const v4f sc = load_scales4(w_scale, n0 + wn * kWN + col, N);
#pragma unroll
                for (int i = 0; i < kMT; ++i) {
                    const int row = 32 * i + r32;
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] * sc[r];
                    *reinterpret_cast<uint2*>(ot + row * kOutStride + col * 2) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }
    }
    __syncthreads();                     // the staged rows are complete before they are read back
    if (group > 0) return;               // no barrier follows
    constexpr int kPieces = kWM * kWN * 2 / 16;
    const int64_t mw0 = m0 + wm * kWM, nw0 = n0 + wn * kWN;
#pragma unroll
    for (int p = lane; p < kPieces; p += kWave) {
        const int row = p / (kWN / 8), c = p % (kWN / 8);
        const int64_t m = mw0 + row, n = nw0 + c * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(ot + row * kOutStride + c * 16);
        if (m >= M) continue;
        uint16_t* dst = y + m * N + n;
        if ((N % 8) == 0 && n + 7 < N) {
            typedef unsigned int v4u __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = static_cast<uint16_t>(w4[e / 2] >> (16 * (e % 2)));
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
        return hipGetLastError();
    }
    if (M <= 128 && M * N <= 128 * 4096) {
        // Few rows: the untiled kernel's N / 16 blocks fill the chip, where the tiled kernel has a
        // few dozen tiles each walking all of K (measured: 20.6 against 51 us at M = 64, N = 4096).
        hipLaunchKernelGGL((w8a16_kernel<4>), dim3(static_cast<unsigned>((N + 15) / 16), static_cast<unsigned>((M + 63) / 64)),
                           dim3(kThreads16), 0, st, x, wq, w_scale, M, N, K, y);
        return hipGetLastError();
    }
    // Tiled: 256 x 256 tiles when there are enough of them for about one per CU, else 128 x 128 when
    // there are enough for one and a half per CU, else 64 x 64.
    auto launch_tiled = [&](auto kernel, int bm, int bn, int threads) {
        const int tm = static_cast<int>((M + bm - 1) / bm), tn = static_cast<int>((N + bn - 1) / bn);
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(tm * tn)), dim3(threads), 0, st, x, wq, w_scale, M, N, K,
                           y, tm, tn);
    };
    // 64 x 64 tiles that do not fill the chip twice over split K among 4 or 2 groups of waves, and
    // so do 128 x 128 tiles that fill most of it once.
    const int64_t tiles64 = ((M + 63) / 64) * ((N + 63) / 64), tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (((M + 255) / 256) * ((N + 255) / 256) >= kW8a16Big)
        launch_tiled(w8a16_tile_kernel<256, 256, 2, 4, 1, 1>, 256, 256, 512);
    else if (tiles128 >= 384)
        launch_tiled(w8a16_tile_kernel<128, 128, 2, 2, 1, 2>, 128, 128, 256);
    else if (tiles128 >= kW8a16Split128Min && tiles128 <= kW8a16Split128Max)
        launch_tiled(w8a16_tile_kernel<128, 128, 2, 2, 2, 1>, 128, 128, 512);
    else if (tiles64 <= kW8a16SplitK4Tiles)
        launch_tiled(w8a16_tile_kernel<64, 64, 2, 2, 4, 1>, 64, 64, 1024);
    else if (tiles64 <= kW8a16SplitK2Tiles)
        launch_tiled(w8a16_tile_kernel<64, 64, 2, 2, 2, 2>, 64, 64, 512);
    else
        launch_tiled(w8a16_tile_kernel<64, 64, 2, 2, 1, 2>, 64, 64, 256);
    return hipGetLastError();
}

}  // namespace w8a8
