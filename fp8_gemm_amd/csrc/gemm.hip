// Quantized GEMM with the dequantizing epilogue on the gfx950 matrix cores.
// ("Weight-Activation Quantization", section 3 step 2: the product of the code matrices, dequantized; section 4:
// x^ = s q for E4M3.)
//
// Both operands are K-contiguous: xq [M, K] and wq [N, K].  Matrix-core instructions:
//   INT8: v_mfma_i32_32x32x32_i8            (large-M kernel; int32 accumulate, exact)
//         v_mfma_i32_16x16x64_i8            (small-M kernel)
//   E4M3: v_mfma_f32_32x32x64_f8f6f4        (large-M kernel)
//         v_mfma_f32_16x16x128_f8f6f4       (small-M kernel)
//         fp32 accumulate; e4m3 x e4m3 products are exact, the summation is the hardware's.
// Each lane feeds 16 (INT8) or 32 (E4M3) consecutive K bytes of one row of each operand; the
// instruction pairs the bytes of A and B the same way, so any assignment of K to lanes that is the
// same for both operands gives the full dot product.
//
// The W tile is the instruction's A operand and the X tile its B operand, so a lane's results are
// runs of four consecutive outputs n of one row m, which the epilogue stores as 8-byte writes:
//   16x16 block: m = lane % 16, n = 4 * (lane / 16) + r                      (r = 0..3)
//   32x32 block: m = lane % 32, n = 8 * g + 4 * (lane / 32) + r, acc[4g + r]  (g, r = 0..3)
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace w8a8 {

namespace {

constexpr int kBK = 128;        // K bytes per pipeline stage
constexpr int kThreads = 256;   // 4 waves

typedef float v16f __attribute__((ext_vector_type(16)));

// ---- matrix-core instruction wrappers ------------------------------------------------------------

// kTile: block edge; kKStep: K bytes per instruction; kChunks: 16-byte chunks per lane per
// instruction; kGroups: runs of four outputs per lane.
struct MmaI8x16 {               // v_mfma_i32_16x16x64_i8
    using Acc = v4i;
    static constexpr int kTile = 16, kKStep = 64, kChunks = 1, kGroups = 1;
    __device__ static __forceinline__ Acc zero() { return Acc{0, 0, 0, 0}; }
    __device__ static __forceinline__ Acc run(const v4i* a, const v4i* b, Acc c) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], b[0], c, 0, 0, 0);
    }
};

typedef int v16i __attribute__((ext_vector_type(16)));

struct MmaI8x32 {               // v_mfma_i32_32x32x32_i8
    using Acc = v16i;
    static constexpr int kTile = 32, kKStep = 32, kChunks = 1, kGroups = 4;
    __device__ static __forceinline__ Acc zero() { return Acc{}; }
    __device__ static __forceinline__ Acc run(const v4i* a, const v4i* b, Acc c) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a[0], b[0], c, 0, 0, 0);
    }
};

__device__ __forceinline__ v8i cat(const v4i* p) {
    return v8i{p[0][0], p[0][1], p[0][2], p[0][3], p[1][0], p[1][1], p[1][2], p[1][3]};
}

struct MmaF8x16 {               // v_mfma_f32_16x16x128_f8f6f4, both operands E4M3
    using Acc = v4f;
    static constexpr int kTile = 16, kKStep = 128, kChunks = 2, kGroups = 1;
    __device__ static __forceinline__ Acc zero() { return Acc{0.f, 0.f, 0.f, 0.f}; }
    __device__ static __forceinline__ Acc run(const v4i* a, const v4i* b, Acc c) {
        // format codes 0, 0: both operands OCP E4M3; zero scale operands select the unscaled form.
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat(a), cat(b), c, 0, 0, 0, 0, 0, 0);
    }
};

struct MmaF8x32 {               // v_mfma_f32_32x32x64_f8f6f4, both operands E4M3
    using Acc = v16f;
    static constexpr int kTile = 32, kKStep = 64, kChunks = 2, kGroups = 4;
    __device__ static __forceinline__ Acc zero() { return Acc{}; }
    __device__ static __forceinline__ Acc run(const v4i* a, const v4i* b, Acc c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cat(a), cat(b), c, 0, 0, 0, 0, 0, 0);
    }
};

// Row m and first column n of group g of a lane's results in a kTile x kTile block.
template <int kTile>
__device__ __forceinline__ int out_row(int lane) { return lane % kTile; }
template <int kTile>
__device__ __forceinline__ int out_col(int lane, int g) {
    return kTile == 16 ? 4 * (lane / 16) : 8 * g + 4 * (lane / 32);
}

// Dequantize and store four consecutive outputs of row m starting at column n (or store the raw
// accumulators when kOutAcc).  tensor: one scale for all of W (w_scale[0]) instead of one per column.
// Columns at or past ncap (<= N) are not stored; ld is the row stride of the output (>= N).
template <bool kOutAcc, typename T>
__device__ __forceinline__ void store4(const T (&a)[4], int64_t m, int64_t n, int64_t M, int64_t N, float sxm,
                                       const float* __restrict__ w_scale, bool tensor, uint16_t* __restrict__ y,
                                       void* __restrict__ out_acc, int64_t ncap, int64_t ld) {
    if (m >= M) return;
    if constexpr (kOutAcc) {
        T* p = static_cast<T*>(out_acc) + m * ld + n;
        if (n + 3 < ncap && (ld & 3) == 0) {
            typedef T v4t __attribute__((ext_vector_type(4)));
            *reinterpret_cast<v4t*>(p) = v4t{a[0], a[1], a[2], a[3]};
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < ncap) p[r] = a[r];
        }
    } else {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float swn = (n + r < N) ? w_scale[tensor ? 0 : n + r] : 0.0f;
            v[r] = (static_cast<float>(a[r]) * sxm) * swn;
        }
        const uint32_t lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
        uint16_t* p = y + m * ld + n;
        if (n + 3 < ncap && (ld & 3) == 0) {
            *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
        } else {
            const uint16_t h[4] = {static_cast<uint16_t>(lo), static_cast<uint16_t>(lo >> 16),
                                   static_cast<uint16_t>(hi), static_cast<uint16_t>(hi >> 16)};
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < ncap) p[r] = h[r];
        }
    }
}

// Epilogue of one kTile x kTile accumulator block whose rows start at m_base and columns at n_base.
// tensor: x_scale[0] and w_scale[0] are the one scale of each operand (per-tensor scaling).
template <typename MM, bool kOutAcc>
__device__ __forceinline__ void store_block(const typename MM::Acc& acc, int64_t m_base, int64_t n_base, int lane,
                                            int64_t M, int64_t N, const float* __restrict__ x_scale,
                                            const float* __restrict__ w_scale, bool tensor,
                                            uint16_t* __restrict__ y, void* __restrict__ out_acc, int64_t ncap,
                                            int64_t ld) {
    using T = typename std::remove_cv<typename std::remove_reference<decltype(acc[0])>::type>::type;
    const int64_t m = m_base + out_row<MM::kTile>(lane);
    const float sxm = (!kOutAcc && m < M) ? x_scale[tensor ? 0 : m] : 0.0f;
#pragma unroll
    for (int g = 0; g < MM::kGroups; ++g) {
        const T a[4] = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        store4<kOutAcc>(a, m, n_base + out_col<MM::kTile>(lane, g), M, N, sxm, w_scale, tensor, y, out_acc, ncap, ld);
    }
}

// ------------------------------------------------------------------------------------------------
// Large-M kernel: block tile kBM x kBN, 4 waves in a 2 x 2 grid, each wave kBM/2 x kBN/2.
//
// LDS holds three stages per operand, each one K step of 128 bytes per row.  A row is 8 chunks of
// 16 bytes, stored in the swizzled order of swz() so that fragment reads are free of bank
// conflicts.
//
// Stages are filled by direct global -> LDS copies (global_load_lds_dwordx4).  The copies are
// written as inline assembly so that the compiler's wait-count pass does not serialise them with
// the fragment reads of other stages; ordering is explicit: a wave waits (s_waitcnt vmcnt) for its
// own copies of a stage, then the block meets at a barrier.
//
// Schedule of K step kt (each half-step h = K bytes [64h, 64h + 64) of the stage):
//   read fragments of half 1 of stage kt    | 512 matrix-core cycles of half 0 of stage kt
//   wait for stage kt + 1, barrier, copy K step kt + 3 into the stage of kt (now fully read)
//   read fragments of half 0 of stage kt+1  | 512 matrix-core cycles of half 1 of stage kt
// so fragment reads overlap the matrix cores and copies run three K steps ahead.
// ------------------------------------------------------------------------------------------------

// 16 zero bytes: the source of copies for K positions beyond the end of a row.
__device__ __attribute__((aligned(16))) uint8_t g_zero16[16] = {0};

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int kN>
__device__ __forceinline__ void wait_copies() {
    static_assert(kN >= 0 && kN < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kN) : "memory");
}

__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Byte address of a __shared__ object inside the block's LDS allocation (what M0 expects).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    const __attribute__((address_space(3))) void* l = (const __attribute__((address_space(3))) void*)(p);
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(l));
}

// One 16-byte-per-lane copy into LDS bytes [lds, lds + 1024): lane l writes lds + 16 l.
//
// Written as inline asm rather than the compiler's LDS-DMA builtin: the compiler cannot tell which
// stage a DMA writes, so before any LDS read that follows one it waits for every copy in flight,
// which would empty the pipeline each half step.  Here the waits are explicit (wait_copies).  The
// asm sets M0 (the LDS destination of the DMA).  The compiler reserves M0 and does not preserve it
// around asm, so these kernels must use M0 for nothing else: tests/test_codegen.py compiles this
// file and checks that every write of M0 in the GEMM kernels is this sequence and that no other
// instruction writes or (implicitly) reads it.  The compiler's warning about the clobber is
// silenced for these two functions.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy_sv(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2"
        :
        : "s"(lds), "v"(voff), "s"(sbase)
        : "memory", "m0");
}
// The same copy marked nontemporal, for data that is read once (a streamed weight matrix).
__device__ __forceinline__ void copy_sv_nt(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt"
        :
        : "s"(lds), "v"(voff), "s"(sbase)
        : "memory", "m0");
}
__device__ __forceinline__ void copy_v(uintptr_t src, uint32_t lds) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds), "v"(src)
        : "memory", "m0");
}
#pragma clang diagnostic pop

// Copies of one K step of a tile: kRows rows x 128 bytes.  One wave instruction fills 1 KB of LDS
// (8 rows): lane l lands at row l / 8 of the block, stored chunk l % 8, which holds the logical
// chunk that swz() places there.  A lane's source offset inside the tile is fixed for the whole K
// loop.  Rows
// past the end re-read the last row (never stored); in the last K step of a ragged K, chunks past
// K come from g_zero16.
template <int kRows, int kWaves>
struct CopyPlan {
    static constexpr int kPerWave = kRows / (8 * kWaves);
    static_assert(kPerWave * 8 * kWaves == kRows && kWaves % 2 == 0, "whole 1 KB blocks per wave");
    uint32_t off[kPerWave];
    int chunk;

    __device__ __forceinline__ void init(int64_t row0, int64_t rows, int64_t K, int wave, int lane) {
        const int rl = lane >> 3;
        // copy i of this wave fills rows 8 * blk + rl, blk = wave + kWaves * i (so blk is odd iff
        // wave is); its stored chunk lane % 8 holds logical chunk (lane % 8) ^ ((row >> 1) & 7).
        chunk = (lane & 7) ^ ((4 * (wave & 1) + (rl >> 1)) & 7);
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            int64_t gr = row0 + (wave + kWaves * i) * 8 + rl;
            gr = gr < rows ? gr : rows - 1;
            off[i] = static_cast<uint32_t>((gr - row0) * K + chunk * 16);
        }
    }
    // Copy i of a K step.  tile: first byte of the K step in the tile's first row; k_left: K minus
    // the K step's first byte (only looked at when !full_k).
    __device__ __forceinline__ void one(int i, const uint8_t* tile, const uint8_t* lds, int wave, bool full_k,
                                        int64_t k_left) const {
        const uint32_t l = lds_addr(lds) + wave * 1024 + kWaves * 1024 * i;
        if (full_k) {
            copy_sv(tile, off[i], l);
        } else {
            const bool in_k = chunk * 16 < k_left;
            copy_v(in_k ? reinterpret_cast<uintptr_t>(tile + off[i]) : reinterpret_cast<uintptr_t>(g_zero16), l);
        }
    }
};

// LDS position of chunk c of row r: c ^ ((r >> 1) & 7).  ds_read_b128 is served 16 lanes (256
// bytes, all 64 banks) at a time; a fragment read puts 16 consecutive rows at one chunk in those 16
// lanes, and with this swizzle the 8 even rows fill one 128-byte half of the banks and the 8 odd
// rows the other, without a conflict.
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 7)) << 4); }

// Map the linear block id to a (tile_m, tile_n) pair.  Consecutive block ids are dispatched to the
// 8 XCDs in turn; the remap gives each XCD a contiguous range of the grouped tile order, and the
// grouped order walks `group_m` tile rows before moving to the next tile column, so the blocks
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

template <int kBM, int kBN, int kGM, int kGN, int kStages, int kWavesPerSimd, typename MM, bool kOutAcc>
__global__ __launch_bounds__(kGM * kGN * kWave, 1)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void gemm_tile_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc, int tiles_m, int tiles_n, int group_m, int tensor_scales, int64_t ldy) {
    using Acc = typename MM::Acc;
    constexpr int kWaves = kGM * kGN;                 // a kGM x kGN grid of waves
    constexpr int kWM = kBM / kGM, kWN = kBN / kGN;   // each wave's kWM x kWN outputs
    constexpr int kMT = kWM / MM::kTile, kNT = kWN / MM::kTile;
    constexpr int kC = MM::kChunks;
    constexpr int kSub = 64 / MM::kKStep;            // instructions per 64-byte half-step
    static_assert(kSub >= 1 && kSub * MM::kKStep == 64, "a half-step is 64 K bytes");
    using CopyX = CopyPlan<kBM, kWaves>;
    using CopyW = CopyPlan<kBN, kWaves>;
    constexpr int kCopies = CopyX::kPerWave + CopyW::kPerWave;   // copy instructions per wave per stage
    // kStages X stages, then kStages W stages; after the K loop the same LDS stages the bf16 output.
    static_assert(kStages == 2 || kStages == 3, "two or three stages");
    constexpr int kOutStride = kWN * 2 + 16;         // bytes per staged output row (padded)
    constexpr int kStageBytes = kStages * (kBM + kBN) * kBK;
    constexpr int kOutBytes = kWaves * kWM * kOutStride;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[kStageBytes > kOutBytes ? kStageBytes : kOutBytes];
    uint8_t* const xs0 = smem;
    uint8_t* const xs1 = smem + kBM * kBK;
    uint8_t* const xs2 = smem + 2 * kBM * kBK;      // kStages == 3 only
    uint8_t* const ws0 = smem + kStages * kBM * kBK;
    uint8_t* const ws1 = ws0 + kBN * kBK;
    uint8_t* const ws2 = ws0 + 2 * kBN * kBK;       // kStages == 3 only

    int tm, tn;
    tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
    // The wave index is uniform within a wave; readfirstlane lets the compiler keep it (and the
    // LDS addresses of the copies, which must be scalar) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = threadIdx.x % kWave;
    const int wm = wave / kGN, wn = wave % kGN;
    const int frag_row = lane % MM::kTile, frag_grp = lane / MM::kTile;

    Acc acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) acc[i][j] = MM::zero();

    // Scales of this lane's outputs: requested before the K loop, so that they arrive during it,
    // when the registers allow (small per-wave tiles); otherwise at the start of the epilogue.
    constexpr int kG = MM::kGroups;
    constexpr bool kPreloadScales = kMT * kNT <= 8;
    const int64_t mw0 = m0 + wm * kWM, nw0 = n0 + wn * kWN;
    float sx_l[kMT];
    v4f sw_l[kNT][kG];
    auto load_scales = [&]() {
#pragma unroll
        for (int i = 0; i < kMT; ++i) {
            const int64_t m = mw0 + i * MM::kTile + out_row<MM::kTile>(lane);
            sx_l[i] = m < M ? x_scale[tensor_scales ? 0 : m] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const int64_t n = nw0 + j * MM::kTile + out_col<MM::kTile>(lane, g);
                if (tensor_scales) {
                    const float w0 = w_scale[0];
                    sw_l[j][g] = v4f{w0, w0, w0, w0};
                } else if (n + 3 < N) {
                    sw_l[j][g] = *reinterpret_cast<const v4f*>(w_scale + n);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sw_l[j][g][r] = (n + r < N) ? w_scale[n + r] : 0.0f;
                }
            }
    };
    if constexpr (!kOutAcc && kPreloadScales) load_scales();

    const int nk = static_cast<int>((K + kBK - 1) / kBK);
    const bool ragged_k = (K % kBK) != 0;
    CopyX cx;
    CopyW cw;
    cx.init(m0, M, K, wave, lane);
    cw.init(n0, N, K, wave, lane);
    const uint8_t* xtile = xq + m0 * K;
    const uint8_t* wtile = wq + n0 * K;
    auto stage_x = [&](int kt) {
        return kStages == 2 ? ((kt & 1) ? xs1 : xs0) : (kt % 3 == 0 ? xs0 : (kt % 3 == 1 ? xs1 : xs2));
    };
    auto stage_w = [&](int kt) {
        return kStages == 2 ? ((kt & 1) ? ws1 : ws0) : (kt % 3 == 0 ? ws0 : (kt % 3 == 1 ? ws1 : ws2));
    };
    // Copy c (0 <= c < kCopies) of K step kt: the X copies first, then the W copies.  A stage's
    // copies go out in two parts, A = [0, kCopies / 2) and B = [kCopies / 2, kCopies).
    constexpr int kPartA = kCopies / 2;
    auto copy = [&](int c, int kt, const uint8_t* lx, const uint8_t* lw, bool plain) {
        const int64_t k0 = static_cast<int64_t>(kt) * kBK;
        if (c < CopyX::kPerWave) cx.one(c, xtile + k0, lx, wave, plain, K - k0);
        else cw.one(c - CopyX::kPerWave, wtile + k0, lw, wave, plain, K - k0);
    };
    auto copies = [&](int c0, int c1, int kt) {      // part of K step kt, any kt < nk
        const bool plain = !(ragged_k && kt == nk - 1);
        for (int c = c0; c < c1; ++c) copy(c, kt, stage_x(kt), stage_w(kt), plain);
    };

    struct Frags {
        v4i x[kSub][kMT][kC];
        v4i w[kSub][kNT][kC];
    };
    // Fragment read r of a half-step (s outer, then chunk, then the X tiles and the W tiles).
    auto read_one = [&](Frags& f, const uint8_t* lx, const uint8_t* lw, int half, int r) {
        constexpr int kPerSC = kMT + kNT;
        const int s = r / (kC * kPerSC), rem = r % (kC * kPerSC);
        const int c = rem / kPerSC, tt = rem % kPerSC;
        const int chunk = half * 4 + s * (MM::kKStep / 16) + frag_grp * kC + c;
        if (tt < kMT)
            f.x[s][tt][c] = *reinterpret_cast<const v4i*>(lx + swz(wm * kWM + tt * MM::kTile + frag_row, chunk));
        else
            f.w[s][tt - kMT][c] =
                *reinterpret_cast<const v4i*>(lw + swz(wn * kWN + (tt - kMT) * MM::kTile + frag_row, chunk));
    };
    auto mma_one = [&](const Frags& f, int q) {
        const int s = q / (kMT * kNT), i = (q / kNT) % kMT, j = q % kNT;
        acc[i][j] = MM::run(f.w[s][j], f.x[s][i], acc[i][j]);
    };
    constexpr int kReads = (kMT + kNT) * kC * kSub, kMmas = kMT * kNT * kSub;

    // One half-step of the steady state, in a fixed order: slot q issues matrix-core instruction q
    // of the current fragments, the fragment reads of the next half assigned to slot q, and the
    // copies assigned to slot q (copies [c0, c0 + kPartA) of K step ckt, which is plain).
    auto half_step = [&](const Frags& cur, Frags& nxt, const uint8_t* lx, const uint8_t* lw, int half, int c0,
                         int ckt, const uint8_t* cxl, const uint8_t* cwl) {
        const int64_t k0 = static_cast<int64_t>(ckt) * kBK;
#pragma unroll
        for (int q = 0; q < kMmas; ++q) {
            mma_one(cur, q);
#pragma unroll
            for (int r = 0; r < kReads; ++r)
                if (r * kMmas / kReads == q) read_one(nxt, lx, lw, half, r);
#pragma unroll
            for (int c = 0; c < kPartA; ++c)
                if (c * kMmas / kPartA == q) {
                    const int cc = c0 + c;
                    if (cc < CopyX::kPerWave) cx.one(cc, xtile + k0, cxl, wave, true, 0);
                    else cw.one(cc - CopyX::kPerWave, wtile + k0, cwl, wave, true, 0);
                }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    Frags f0, f1;
    // Steady-state K step kt (all copies plain and in range): the first half multiplies f0 (half 0
    // of stage kt) while reading f1 (half 1) and sending copies B of K step kt + 2; then the stage
    // of kt + 1 is waited for and the block meets; the second half multiplies f1 while reading f0
    // (half 0 of stage kt + 1) and sending copies A of K step kt + 3 into the stage just read.
    // Stages: (lx, lw) of kt, (nx, nw) of kt + 1, (bx, bw) of kt + 2; kt + 3 reuses (lx, lw).
    auto full_step = [&](int kt, const uint8_t* lx, const uint8_t* lw, const uint8_t* nx, const uint8_t* nw,
                         const uint8_t* bx, const uint8_t* bw) {
        half_step(f0, f1, lx, lw, 1, kPartA, kt + 2, bx, bw);
        wait_lds_reads();
        wait_copies<kCopies>();
        block_barrier();
        half_step(f1, f0, nx, nw, 0, 0, kt + 3, lx, lw);
    };
    // The same protocol for any kt, with the copies and the next stage guarded.
    auto step = [&](int kt) {
        for (int r = 0; r < kReads; ++r) read_one(f1, stage_x(kt), stage_w(kt), 1, r);
        for (int q = 0; q < kMmas; ++q) mma_one(f0, q);
        if (kt + 2 < nk) copies(kPartA, kCopies, kt + 2);
        wait_lds_reads();
        if (kt + 1 < nk) {
            if (kt + 2 < nk) wait_copies<kCopies>();
            else wait_copies<0>();
            block_barrier();
            if (kt + 3 < nk) copies(0, kPartA, kt + 3);
            for (int r = 0; r < kReads; ++r) read_one(f0, stage_x(kt + 1), stage_w(kt + 1), 0, r);
        }
        for (int q = 0; q < kMmas; ++q) mma_one(f1, q);
    };

    const int n_plain = ragged_k ? nk - 1 : nk;     // K steps that need no zero fill
    if constexpr (kStages == 3) {
        // Prologue: K steps 0 and 1 whole and part A of K step 2; wait for step 0.
        copies(0, kCopies, 0);
        if (nk > 1) copies(0, kCopies, 1);
        if (nk > 2) copies(0, kPartA, 2);
        if (nk > 2) wait_copies<kCopies + kPartA>();
        else if (nk > 1) wait_copies<kCopies>();
        else wait_copies<0>();
        block_barrier();
        for (int r = 0; r < kReads; ++r) read_one(f0, xs0, ws0, 0, r);
        int kt = 0;
        for (; kt + 5 < n_plain; kt += 3) {      // steps kt .. kt + 2 copy plain K steps up to kt + 5
            full_step(kt, xs0, ws0, xs1, ws1, xs2, ws2);
            full_step(kt + 1, xs1, ws1, xs2, ws2, xs0, ws0);
            full_step(kt + 2, xs2, ws2, xs0, ws0, xs1, ws1);
        }
        for (; kt < nk; ++kt) step(kt);          // the last (at most five) steps
    } else {
        // Two stages (for tiles whose three stages would not fit in LDS).  K step kt:
        //   first half:  matrix cores on f0 (half 0 of stage kt) | read f1 (half 1 of stage kt)
        //   wait for this wave's copies of kt + 1 and for its fragment reads; the block meets
        //   second half: matrix cores on f1 | read f0 (half 0 of stage kt + 1) | copy K step kt + 2
        //                into the stage of kt, which nobody reads any more
        // so a copy has about one K step to land.  (Issuing the copies in a burst early in the
        // half-step is slower: with one wave per SIMD, a stalled copy issue idles the matrix core.)
        auto half2 = [&](const Frags& cur, Frags& nxt, const uint8_t* lx, const uint8_t* lw, int half, int ckt,
                         const uint8_t* cxl, const uint8_t* cwl, bool with_copies) {
            const int64_t k0 = static_cast<int64_t>(ckt) * kBK;
#pragma unroll
            for (int q = 0; q < kMmas; ++q) {
                mma_one(cur, q);
#pragma unroll
                for (int r = 0; r < kReads; ++r)
                    if (r * kMmas / kReads == q) read_one(nxt, lx, lw, half, r);
                if (with_copies) {
#pragma unroll
                    for (int c = 0; c < kCopies; ++c)
                        if (c * kMmas / kCopies == q) {
                            if (c < CopyX::kPerWave) cx.one(c, xtile + k0, cxl, wave, true, 0);
                            else cw.one(c - CopyX::kPerWave, wtile + k0, cwl, wave, true, 0);
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto full2 = [&](int kt, const uint8_t* lx, const uint8_t* lw, const uint8_t* nx, const uint8_t* nw) {
            half2(f0, f1, lx, lw, 1, 0, nullptr, nullptr, false);
            wait_lds_reads();
            wait_copies<0>();
            block_barrier();
            half2(f1, f0, nx, nw, 0, kt + 2, lx, lw, true);
        };
        auto step2 = [&](int kt) {
            for (int r = 0; r < kReads; ++r) read_one(f1, stage_x(kt), stage_w(kt), 1, r);
            for (int q = 0; q < kMmas; ++q) mma_one(f0, q);
            wait_lds_reads();
            if (kt + 1 < nk) {
                wait_copies<0>();
                block_barrier();
                if (kt + 2 < nk) copies(0, kCopies, kt + 2);
                for (int r = 0; r < kReads; ++r) read_one(f0, stage_x(kt + 1), stage_w(kt + 1), 0, r);
            }
            for (int q = 0; q < kMmas; ++q) mma_one(f1, q);
        };
        copies(0, kCopies, 0);
        if (nk > 1) copies(0, kCopies, 1);
        if (nk > 1) wait_copies<kCopies>();
        else wait_copies<0>();
        block_barrier();
        for (int r = 0; r < kReads; ++r) read_one(f0, xs0, ws0, 0, r);
        int kt = 0;
        for (; kt + 3 < n_plain; kt += 2) {      // steps kt, kt + 1 copy plain K steps kt + 2, kt + 3
            full2(kt, xs0, ws0, xs1, ws1);
            full2(kt + 1, xs1, ws1, xs0, ws0);
        }
        for (; kt < nk; ++kt) step2(kt);
    }

    if constexpr (kOutAcc) {
#pragma unroll
        for (int i = 0; i < kMT; ++i)
#pragma unroll
            for (int j = 0; j < kNT; ++j)
                store_block<MM, kOutAcc>(acc[i][j], mw0 + i * MM::kTile, nw0 + j * MM::kTile, lane, M, N, x_scale,
                                         w_scale, tensor_scales != 0, y, out_acc, N, ldy);
    } else {
        // Dequantize in registers, stage the wave's kWM x kWN bf16 tile in LDS (rows padded to
        // kOutStride bytes), and write it back as 16-byte pieces of whole output rows.
        if constexpr (!kPreloadScales) load_scales();
        block_barrier();                 // every wave has finished reading the stages
        uint8_t* const ot = smem + wave * (kWM * kOutStride);
#pragma unroll
        for (int i = 0; i < kMT; ++i)
#pragma unroll
            for (int j = 0; j < kNT; ++j)
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = (static_cast<float>(acc[i][j][4 * g + r]) * sx_l[i]) * sw_l[j][g][r];
                    const int row = i * MM::kTile + out_row<MM::kTile>(lane);
                    const int col = j * MM::kTile + out_col<MM::kTile>(lane, g);
                    *reinterpret_cast<uint2*>(ot + row * kOutStride + col * 2) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
        wait_lds_reads();                // this wave's LDS writes are complete before it reads them
        constexpr int kPieces = kWM * kWN * 2 / 16;  // 16-byte pieces in the wave's tile
        const bool vec_ok = (ldy % 8) == 0;
#pragma unroll
        for (int p = lane; p < kPieces; p += kWave) {
            const int row = p / (kWN / 8), c = p % (kWN / 8);
            const int64_t m = mw0 + row, n = nw0 + c * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(ot + row * kOutStride + c * 16);
            if (m >= M) continue;
            uint16_t* dst = y + m * ldy + n;
            if (vec_ok && n + 7 < N) {
                // Nontemporal: the output is written once and not read here, so it does not displace
                // the operand panels the other tiles still read from the caches.
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
}

// ------------------------------------------------------------------------------------------------
// Small-M kernel (decode-shaped: M <= 16 * kMT).  The GEMM is bound by reading W once, so a block
// owns 16 output columns and all of K, its 4 waves take interleaved K steps, operands come straight
// from global memory (X is small and stays in cache), and the 4 partial sums are added in LDS at
// the end (exact for INT8).  N / 16 blocks keep every CU streaming.
// ------------------------------------------------------------------------------------------------
template <int kMT, typename MM, bool kOutAcc>
__global__ __launch_bounds__(kThreads) void gemm_small_m_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc, int tensor_scales) {
    using Acc = typename MM::Acc;
    static_assert(MM::kTile == 16, "16x16 blocks");
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
    for (int i = 0; i < kMT; ++i) acc[i] = MM::zero();

    // Steps with all K bytes inside the rows run kU at a time with every load issued before the
    // matrix-core work, so a wave keeps (1 + kMT) * kChunks * kU 16-byte loads in flight.  Each wave
    // takes a contiguous range of per_w such steps (consecutive requests to a row stay together);
    // the remaining steps (and a partial last one) are spread over the waves and zero the bytes past K.
    constexpr int kU = (16 / ((1 + kMT) * MM::kChunks)) > 0 ? 16 / ((1 + kMT) * MM::kChunks) : 1;
    const int64_t nfull = K / MM::kKStep;
    const int64_t nsteps = (K + MM::kKStep - 1) / MM::kKStep;
    const int64_t per_w = (nfull / 4 / kU) * kU;
    int64_t st0 = wave * per_w;
    for (int64_t it = 0; it < per_w; it += kU, st0 += kU) {
        v4i fw[kU][MM::kChunks], fx[kU][kMT][MM::kChunks];
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int c = 0; c < MM::kChunks; ++c) {
                const int64_t k = (st0 + u) * MM::kKStep + (frag_grp * MM::kChunks + c) * 16;
                fw[u][c] = *reinterpret_cast<const v4i*>(wrow + k);
#pragma unroll
                for (int i = 0; i < kMT; ++i) fx[u][i][c] = *reinterpret_cast<const v4i*>(xrow[i] + k);
            }
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
            for (int i = 0; i < kMT; ++i) acc[i] = MM::run(fw[u], fx[u][i], acc[i]);
    }
    for (int64_t st = 4 * per_w + wave; st < nsteps; st += 4) {
        v4i fw[MM::kChunks], fx[kMT][MM::kChunks];
#pragma unroll
        for (int c = 0; c < MM::kChunks; ++c) {
            const int64_t k = st * MM::kKStep + (frag_grp * MM::kChunks + c) * 16;
            const bool ok = k < K;
            fw[c] = ok ? *reinterpret_cast<const v4i*>(wrow + k) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                fx[i][c] = ok ? *reinterpret_cast<const v4i*>(xrow[i] + k) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i) acc[i] = MM::run(fw, fx[i], acc[i]);
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
            store_block<MM, kOutAcc>(a, static_cast<int64_t>(i) * 16, n0, lane, M, N, x_scale, w_scale,
                                     tensor_scales != 0, y, out_acc, N, N);
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Decode kernel (M <= 16, K = 8 * kS * kKStep; used for E4M3 at K = 8192, the INT8 decode shape
// takes the LDS kernel below): bound by reading W once.  A block has 8 waves; wave w owns the w-th
// eighth of K and holds its X fragments for that eighth in registers for the whole kernel, so X is
// read once per wave instead of once per output tile.  Block b owns the output columns
// [b cols, (b + 1) cols): cols is a multiple of 8 chosen so that every CU streams the same share of
// W (at N = 14336, 56 columns: three 16-column tiles and one of 8, whose other 8 rows re-read the
// last row, from cache, and are not stored).  W fragments of kDepth tiles are in flight per wave,
// and a buffer is refilled as soon as the matrix cores have consumed it.  kDepth is the block's
// tile count, up to 2 (E4M3 fragments are 32 bytes per lane), so that no buffer is loaded for a
// tile the block does not have.
// Each wave writes its partial sums per tile to LDS; after one barrier the partials are added
// (exact for INT8) and stored, so no store sits between two waits for loads.
// ------------------------------------------------------------------------------------------------
constexpr int kDecodeThreads = 512;       // 8 waves
constexpr int kDecodeMaxTiles = 8;        // columns per block <= 8 tiles of 16
#ifndef W8A8_DECODE_BLOCKS
#define W8A8_DECODE_BLOCKS 256
#endif
constexpr int kDecodeBlocks = W8A8_DECODE_BLOCKS;   // blocks the columns are spread over

template <int kS, int kDepth, typename MM, bool kOutAcc>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc, int tensor_scales, int cols) {
    using Acc = typename MM::Acc;
    static_assert(MM::kTile == 16, "16x16 blocks");
    constexpr int kC = MM::kChunks;
    constexpr int kWaves = kDecodeThreads / kWave;
    static_assert(kDepth >= 1 && kDepth * kC <= 4, "W tiles in flight per wave");
    __shared__ Acc part[kDecodeMaxTiles][kWaves][kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int frag_row = lane & 15, frag_grp = lane >> 4;
    const int64_t kw0 = static_cast<int64_t>(wave) * kS * MM::kKStep;   // this wave's eighth of K
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * cols;
    const int64_t c1 = c0 + cols < N ? c0 + cols : N;                   // this block's columns [c0, c1)
    const int nt = static_cast<int>((c1 - c0 + 15) / 16);              // 1 .. kDecodeMaxTiles

    v4i fx[kS][kC];
    {
        const int64_t m = frag_row < M ? frag_row : M - 1;
        const uint8_t* xr = xq + m * K + kw0;
#pragma unroll
        for (int s = 0; s < kS; ++s)
#pragma unroll
            for (int c = 0; c < kC; ++c)
                fx[s][c] = *reinterpret_cast<const v4i*>(xr + s * MM::kKStep + (frag_grp * kC + c) * 16);
    }
    v4i fw[kDepth][kS][kC];
    auto load_w = [&](v4i (&dst)[kS][kC], int t) {
        t = t < nt ? t : nt - 1;
        int64_t n = c0 + static_cast<int64_t>(t) * 16 + frag_row;
        n = n < c1 ? n : c1 - 1;
        const uint8_t* wr = wq + n * K + kw0;
#pragma unroll
        for (int s = 0; s < kS; ++s)
#pragma unroll
            for (int c = 0; c < kC; ++c)
                dst[s][c] = *reinterpret_cast<const v4i*>(wr + s * MM::kKStep + (frag_grp * kC + c) * 16);
    };
#pragma unroll
    for (int i = 0; i < kDepth; ++i) load_w(fw[i], i);
    // Fully unrolled, so that the compiler counts the loads in flight exactly: across a loop's back
    // edge, or after a branch that skips loads, it waits for more of them than needed.  The last
    // group of kDepth tiles has a copy of its own without refills; in the other groups every
    // buffer is refilled (with the last tile again when fewer tiles remain).
#pragma unroll
    for (int t0 = 0; t0 < kDecodeMaxTiles; t0 += kDepth) {
        auto product = [&](int i) {
            Acc acc = MM::zero();
#pragma unroll
            for (int s = 0; s < kS; ++s) acc = MM::run(fw[i][s], fx[s], acc);
            // past the last tile a buffer holds the last tile again: the same sums, rewritten
            part[t0 + i < nt ? t0 + i : nt - 1][wave][lane] = acc;
        };
        if (t0 + kDepth >= nt || t0 + kDepth >= kDecodeMaxTiles) {
#pragma unroll
            for (int i = 0; i < kDepth; ++i) product(i);
            break;
        }
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {      // buffer i holds tile t0 + i
            product(i);
            load_w(fw[i], t0 + i + kDepth);
            // keep the program order: the compiler would otherwise move the refills behind the
            // later tiles' products
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    // The block's outputs: wave w adds the partials of tiles w, w + 8, ... and stores them.
    for (int t = wave; t < nt; t += kWaves) {
        Acc acc = part[t][0][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) acc += part[t][w][lane];
        store_block<MM, kOutAcc>(acc, 0, c0 + static_cast<int64_t>(t) * 16, lane, M, N, x_scale, w_scale,
                                 tensor_scales != 0, y, out_acc, c1, N);
    }
}

// ------------------------------------------------------------------------------------------------
// INT8 decode kernel with W staged through LDS (M <= 16, K = 4096).  The kernel above loads W
// fragments straight into registers, and the matrix-core layout puts 16 different rows in 16
// consecutive lanes, so each load instruction touches 16 rows x 64 bytes: read that way the
// weights stream from HBM at about two thirds of what a contiguous read of the same bytes gets.
// Here a block copies each 16-row tile of W (16 x 4096 bytes) into LDS with direct global -> LDS
// copies of 1 KB of one row per wave instruction, and the waves read their fragments from LDS.
// Within each 256-byte group of a row the 16-byte chunks are stored at chunk ^ (row % 16), which
// the copies produce by permuting their source addresses inside the group, so that the 16 rows of
// a fragment read fall in 16 different bank groups.  Two tile buffers (128 KB): the copies of tile
// t + 1 are in flight while tile t is multiplied, and tile t + 2 is copied into t's buffer once
// every wave has read it.  Column ranges, partial sums and stores are as in the kernel above (each
// wave owns an eighth of K and keeps its X fragments for it in registers; the 8 partials are added
// in LDS at the end).
// ------------------------------------------------------------------------------------------------
constexpr int kDecodeLdsK = 4096;

template <bool kOutAcc>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_lds_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc, int tensor_scales, int cols) {
    using MM = MmaI8x16;
    using Acc = MM::Acc;
    constexpr int kWaves = kDecodeThreads / kWave;
    constexpr int kS = kDecodeLdsK / kWaves / MM::kKStep;             // 8 instructions per wave and tile
    constexpr int kTileBytes = 16 * kDecodeLdsK;
    constexpr int kCopies = kTileBytes / 1024 / kWaves;               // 8 copies per wave and tile
    __shared__ __attribute__((aligned(1024))) uint8_t buf[2][kTileBytes];
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = threadIdx.x % kWave;
    const int frag_row = lane & 15, frag_grp = lane >> 4;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * cols;
    const int64_t c1 = c0 + cols < N ? c0 + cols : N;
    const int nt = static_cast<int>((c1 - c0 + 15) / 16);              // 1 .. kDecodeMaxTiles

    // Copy i of this wave of a 16-row tile whose row r starts at src + row_off(r): row
    // r = (kCopies wave + i) / 4 of the tile, quarter q of the row; lane l fills stored chunk
    // 64 q + l, which holds logical chunk (64 q + l) ^ r.
    auto copy_rows = [&](const uint8_t* src, auto row_off, uint8_t* dst, auto stream) {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int inst = kCopies * wave + i;
            const int r = inst >> 2, q = inst & 3;
            const uint32_t off = row_off(r) + static_cast<uint32_t>(((64 * q + lane) ^ r) * 16);
            const uint32_t l = lds_addr(dst) + static_cast<uint32_t>(r * kDecodeLdsK + q * 1024);
            if constexpr (decltype(stream)::value) copy_sv_nt(src, off, l);    // W: read once
            else copy_sv(src, off, l);
        }
    };
    // W rows from the block's own first row, so that offsets stay within the block's columns
    // (at most 2 kDecodeMaxTiles x 8 rows of 4 KB) for any N.
    const uint8_t* const wblk = wq + c0 * K;
    auto copy_tile = [&](int t, uint8_t* dst) {        // rows past c1 re-read row c1 - 1
        copy_rows(wblk, [&](int r) {
            int64_t n = static_cast<int64_t>(t) * 16 + r;
            n = n < c1 - c0 ? n : c1 - c0 - 1;
            return static_cast<uint32_t>(n * K);
        }, dst, std::true_type{});
    };
    // Fragment of row frag_row, K step s of this wave's eighth, from a tile in LDS.
    auto frag = [&](const uint8_t* b, int s) {
        const int chunk = (wave * kS + s) * (MM::kKStep / 16) + frag_grp;
        return *reinterpret_cast<const v4i*>(b + frag_row * kDecodeLdsK + ((chunk ^ frag_row) << 4));
    };
    // X goes through LDS too, next to tile 0: every global read of the kernel is then one of these
    // copies, whose waits are explicit (a plain load would make the compiler's own wait for it
    // count the copies issued after it, and wait for them as well).  X rows past M re-read row M - 1.
    copy_rows(xq, [&](int r) { return static_cast<uint32_t>((r < M ? r : M - 1) * K); }, buf[1], std::false_type{});
    copy_tile(0, buf[0]);
    wait_copies<kCopies>();                           // X has landed; tile 0 may be in flight
    block_barrier();
    v4i fx[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s) fx[s] = frag(buf[1], s);
    wait_lds_reads();
    block_barrier();                                  // every wave has read X: buffer 1 is free
    if (nt > 1) copy_tile(1, buf[1]);
    Acc acc[kDecodeMaxTiles];
#pragma unroll
    for (int t = 0; t < kDecodeMaxTiles; ++t) acc[t] = MM::zero();
    // Fully unrolled (at most kDecodeMaxTiles tiles) so that acc[t] has compile-time indices.
#pragma unroll
    for (int t = 0; t < kDecodeMaxTiles; ++t) {
        if (t >= nt) break;
        if (t + 1 < nt) wait_copies<kCopies>();       // tile t landed; tile t + 1 may be in flight
        else wait_copies<0>();
        block_barrier();
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            const v4i w = frag(buf[t & 1], s);
            acc[t] = MM::run(&w, &fx[s], acc[t]);
        }
        wait_lds_reads();
        block_barrier();                              // every wave has read buffer t & 1
        if (t + 2 < nt) copy_tile(t + 2, buf[t & 1]);
    }
    // The partial sums of the 8 waves meet in LDS (the tile buffers are free): wave w adds and
    // stores tiles w, w + 8, ...
    Acc* part = reinterpret_cast<Acc*>(&buf[0][0]);   // [tile][wave][lane]
#pragma unroll
    for (int t = 0; t < kDecodeMaxTiles; ++t)
        if (t < nt) part[(t * kWaves + wave) * kWave + lane] = acc[t];
    wait_lds_reads();
    block_barrier();
    for (int t = wave; t < nt; t += kWaves) {
        Acc a = part[t * kWaves * kWave + lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) a += part[(t * kWaves + w) * kWave + lane];
        store_block<MM, kOutAcc>(a, 0, c0 + static_cast<int64_t>(t) * 16, lane, M, N, x_scale, w_scale,
                                 tensor_scales != 0, y, out_acc, c1, N);
    }
}

// The same weight stream for 16 < M <= 16 kMT rows (INT8, K = 4096): every wave keeps the X
// fragments of its eighth of K for all kMT row tiles in registers (kMT 8 16-byte fragments), so a
// weight tile in LDS feeds kMT matrix-core instructions per fragment read.  X is staged through the
// two tile buffers first, two row tiles at a time; then the weight tiles stream as in
// gemm_decode_lds_kernel, at most kDecodeMultiTiles of them per block.
constexpr int kDecodeMultiTiles = 4;

template <int kMT, bool kOutAcc>
__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_lds_multi_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ x_scale, const uint8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ y,
    void* __restrict__ out_acc, int tensor_scales, int cols) {
    using MM = MmaI8x16;
    using Acc = MM::Acc;
    static_assert(kMT >= 2 && kMT % 2 == 0, "row tiles are staged two at a time");
    constexpr int kWaves = kDecodeThreads / kWave;
    constexpr int kS = kDecodeLdsK / kWaves / MM::kKStep;             // 8 instructions per wave and tile
    constexpr int kTileBytes = 16 * kDecodeLdsK;
    constexpr int kCopies = kTileBytes / 1024 / kWaves;               // 8 copies per wave and tile
    static_assert(kDecodeMultiTiles * kWaves * kWave * kMT * static_cast<int>(sizeof(Acc)) <= 2 * kTileBytes,
                  "the partial sums fit in the tile buffers");
    __shared__ __attribute__((aligned(1024))) uint8_t buf[2][kTileBytes];
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int lane = threadIdx.x % kWave;
    const int frag_row = lane & 15, frag_grp = lane >> 4;
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * cols;
    const int64_t c1 = c0 + cols < N ? c0 + cols : N;
    const int nt = static_cast<int>((c1 - c0 + 15) / 16);              // 1 .. kDecodeMultiTiles

    // Copies of a 16-row tile as in gemm_decode_lds_kernel (chunks of each 256-byte group stored
    // at chunk ^ (row mod 16)); `stream` marks the weight copies nontemporal.
    auto copy_rows = [&](const uint8_t* src, auto row_off, uint8_t* dst, auto stream) {
#pragma unroll
        for (int i = 0; i < kCopies; ++i) {
            const int inst = kCopies * wave + i;
            const int r = inst >> 2, q = inst & 3;
            const uint32_t off = row_off(r) + static_cast<uint32_t>(((64 * q + lane) ^ r) * 16);
            const uint32_t l = lds_addr(dst) + static_cast<uint32_t>(r * kDecodeLdsK + q * 1024);
            if constexpr (decltype(stream)::value) copy_sv_nt(src, off, l);
            else copy_sv(src, off, l);
        }
    };
    const uint8_t* const wblk = wq + c0 * K;
    auto copy_tile = [&](int t, uint8_t* dst) {
        copy_rows(wblk, [&](int r) {
            int64_t n = static_cast<int64_t>(t) * 16 + r;
            n = n < c1 - c0 ? n : c1 - c0 - 1;
            return static_cast<uint32_t>(n * K);
        }, dst, std::true_type{});
    };
    auto frag = [&](const uint8_t* b, int s) {
        const int chunk = (wave * kS + s) * (MM::kKStep / 16) + frag_grp;
        return *reinterpret_cast<const v4i*>(b + frag_row * kDecodeLdsK + ((chunk ^ frag_row) << 4));
    };
    // X: row tiles 2p and 2p + 1 through the two buffers; rows past M re-read row M - 1.
    v4i fx[kMT][kS];
#pragma unroll
    for (int p = 0; p < kMT / 2; ++p) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int mt = 2 * p + h;
            copy_rows(xq, [&](int r) {
                const int64_t m = static_cast<int64_t>(mt) * 16 + r;
                return static_cast<uint32_t>((m < M ? m : M - 1) * K);
            }, buf[h], std::false_type{});
        }
        wait_copies<0>();
        block_barrier();
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int s = 0; s < kS; ++s) fx[2 * p + h][s] = frag(buf[h], s);
        wait_lds_reads();
        block_barrier();                  // both buffers are free again
    }
    copy_tile(0, buf[0]);
    if (nt > 1) copy_tile(1, buf[1]);
    Acc acc[kDecodeMultiTiles][kMT];
#pragma unroll
    for (int t = 0; t < kDecodeMultiTiles; ++t)
#pragma unroll
        for (int i = 0; i < kMT; ++i) acc[t][i] = MM::zero();
#pragma unroll
    for (int t = 0; t < kDecodeMultiTiles; ++t) {
        if (t >= nt) break;
        if (t + 1 < nt) wait_copies<kCopies>();       // tile t landed; tile t + 1 may be in flight
        else wait_copies<0>();
        block_barrier();
#pragma unroll
        for (int s = 0; s < kS; ++s) {
            const v4i w = frag(buf[t & 1], s);
#pragma unroll
            for (int i = 0; i < kMT; ++i) acc[t][i] = MM::run(&w, &fx[i][s], acc[t][i]);
        }
        wait_lds_reads();
        block_barrier();                              // every wave has read buffer t & 1
        if (t + 2 < nt) copy_tile(t + 2, buf[t & 1]);
    }
    // Partial sums of the 8 waves through LDS: [tile][row tile][wave][lane]; wave w adds and stores
    // the (tile, row tile) pairs w, w + 8, ...
    Acc* part = reinterpret_cast<Acc*>(&buf[0][0]);
#pragma unroll
    for (int t = 0; t < kDecodeMultiTiles; ++t)
#pragma unroll
        for (int i = 0; i < kMT; ++i)
            if (t < nt) part[((t * kMT + i) * kWaves + wave) * kWave + lane] = acc[t][i];
    wait_lds_reads();
    block_barrier();
    for (int ti = wave; ti < nt * kMT; ti += kWaves) {
        Acc a = part[ti * kWaves * kWave + lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) a += part[(ti * kWaves + w) * kWave + lane];
        const int t = ti / kMT, i = ti % kMT;
        store_block<MM, kOutAcc>(a, static_cast<int64_t>(i) * 16, c0 + static_cast<int64_t>(t) * 16, lane, M, N,
                                 x_scale, w_scale, tensor_scales != 0, y, out_acc, c1, N);
    }
}

template <typename M16, typename MT, bool kOutAcc>
hipError_t gemm_dispatch(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale,
                         int64_t M, int64_t N, int64_t K, uint16_t* y, void* out_acc, int tensor, hipStream_t st) {
    if (M <= 16 && K == 8 * 8 * M16::kKStep) {
        // decode shape: X in registers; each block an equal range of columns (a multiple of 8), one
        // block per CU while that keeps a block's range within kDecodeMaxTiles tiles
        const int64_t units = (N + 7) / 8;
        int64_t per = (units + kDecodeBlocks - 1) / kDecodeBlocks;
        if (per > 2 * kDecodeMaxTiles) per = 2 * kDecodeMaxTiles;
        const int cols = static_cast<int>(per * 8);
        const int64_t grid = (N + cols - 1) / cols;
        const int tiles = (cols + 15) / 16;
        const dim3 g(static_cast<unsigned>(grid)), b(kDecodeThreads);
        if constexpr (M16::kChunks == 1) {              // INT8 (K = 4096): W through LDS
            static_assert(8 * 8 * M16::kKStep == kDecodeLdsK, "the INT8 decode shape is K = 4096");
            hipLaunchKernelGGL((gemm_decode_lds_kernel<kOutAcc>), g, b, 0, st, xq, x_scale, wq, w_scale, M, N, K, y,
                               out_acc, tensor, cols);
        } else if (tiles == 1) {                        // E4M3 (K = 8192): fragments straight to registers
            hipLaunchKernelGGL((gemm_decode_kernel<8, 1, M16, kOutAcc>), g, b, 0, st, xq, x_scale, wq, w_scale, M, N, K,
                               y, out_acc, tensor, cols);
        } else {
            hipLaunchKernelGGL((gemm_decode_kernel<8, 2, M16, kOutAcc>), g, b, 0, st, xq, x_scale, wq, w_scale, M, N, K,
                               y, out_acc, tensor, cols);
        }
        return hipGetLastError();
    }
    if constexpr (M16::kChunks == 1) {
        if (M <= 64 && K == kDecodeLdsK) {
            // INT8, 16 < M <= 64, K = 4096: the weight stream of the decode kernel with 2 or 4 row
            // tiles of X in registers; each block an equal range of columns (at most 4 tiles).
            const int64_t units = (N + 7) / 8;
            int64_t per = (units + kDecodeBlocks - 1) / kDecodeBlocks;
            if (per > 2 * kDecodeMultiTiles) per = 2 * kDecodeMultiTiles;
            const int cols = static_cast<int>(per * 8);
            const dim3 g(static_cast<unsigned>((N + cols - 1) / cols)), b(kDecodeThreads);
            if (M <= 32)
                hipLaunchKernelGGL((gemm_decode_lds_multi_kernel<2, kOutAcc>), g, b, 0, st, xq, x_scale, wq, w_scale, M,
                                   N, K, y, out_acc, tensor, cols);
            else
                hipLaunchKernelGGL((gemm_decode_lds_multi_kernel<4, kOutAcc>), g, b, 0, st, xq, x_scale, wq, w_scale, M,
                                   N, K, y, out_acc, tensor, cols);
            return hipGetLastError();
        }
    }
    if (M <= 16 || (M <= 32 && N <= 8192)) {
        // A block per 16 output columns streams W once; X is re-read per block from L2, which is
        // cheap while M and N are small.
        dim3 grid(static_cast<unsigned>((N + 15) / 16));
        if (M <= 16)
            hipLaunchKernelGGL((gemm_small_m_kernel<1, M16, kOutAcc>), grid, dim3(kThreads), 0, st, xq, x_scale, wq,
                               w_scale, M, N, K, y, out_acc, tensor);
        else
            hipLaunchKernelGGL((gemm_small_m_kernel<2, M16, kOutAcc>), grid, dim3(kThreads), 0, st, xq, x_scale, wq,
                               w_scale, M, N, K, y, out_acc, tensor);
        return hipGetLastError();
    }
    // Tiles: the largest tile that still gives at least kFill tiles (about three quarters of the 256
    // CUs, one tile each); with fewer, a CU's per-tile K loop is the whole kernel's time, so smaller
    // tiles finish sooner.  The smallest (64 x 64) is the fallback.
    constexpr int64_t kFill = 192;
    const int group_m = 4;
    auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    // One launch over the output columns [n_off, n_off + ncols): the weight rows, column scales and
    // outputs of that range, the output rows keeping their full stride N.
    auto launch = [&](auto kernel, int bm, int bn, int threads, int64_t n_off, int64_t ncols) {
        const int tiles_m = static_cast<int>((M + bm - 1) / bm);
        const int tiles_n = static_cast<int>((ncols + bn - 1) / bn);
        const float* ws = (w_scale != nullptr && !tensor) ? w_scale + n_off : w_scale;
        uint16_t* yo = y != nullptr ? y + n_off : nullptr;
        void* acc = out_acc != nullptr ? static_cast<void*>(static_cast<uint8_t*>(out_acc) + n_off * 4) : nullptr;
        hipLaunchKernelGGL(kernel, dim3(tiles_m * tiles_n), dim3(threads), 0, st, xq, x_scale, wq + n_off * K, ws, M,
                           ncols, K, yo, acc, tiles_m, tiles_n, group_m, tensor, N);
    };
    if (tiles(256, 256) >= 512) {
        // Enough 256 x 256 tiles for two rounds over 256 CUs: 4 waves of 128 x 128 outputs, half the
        // LDS reads and two thirds of the copies per matrix-core instruction of the smaller tile.
        // A last round less than half full (MLP-up 8192 x 11008: 1376 tiles, 5.4 rounds) is moved to
        // a second launch: the first n1 tile columns in whole rounds of 256 x 256 tiles, the rest of
        // the columns in one round of 256 x 128 tiles (the last round then takes a 256 x 128 tile's
        // time instead of a 256 x 256 tile's).
        constexpr int64_t kCUs = 256;
        const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256, rem = (tm * tn) % kCUs;
        int64_t n1 = 0;
        if (rem != 0 && rem < kCUs / 2) {
            for (int64_t c = tn - 1; c >= 1 && n1 == 0; --c)
                if ((tm * c) % kCUs == 0) n1 = c;
            if (n1 > 0 && tm * ((N - 256 * n1 + 127) / 128) > kCUs) n1 = 0;
        }
        if (n1 > 0) {
            launch(gemm_tile_kernel<256, 256, 2, 2, 2, 1, MT, kOutAcc>, 256, 256, 4 * kWave, 0, 256 * n1);
            launch(gemm_tile_kernel<256, 128, 4, 2, 3, 2, MT, kOutAcc>, 256, 128, 8 * kWave, 256 * n1, N - 256 * n1);
        } else {
            launch(gemm_tile_kernel<256, 256, 2, 2, 2, 1, MT, kOutAcc>, 256, 256, 4 * kWave, 0, N);
        }
    } else if (tiles(256, 128) >= kFill) {
        launch(gemm_tile_kernel<256, 128, 4, 2, 3, 2, MT, kOutAcc>, 256, 128, 8 * kWave, 0, N);
    } else if (tiles(128, 128) >= kFill) {
        launch(gemm_tile_kernel<128, 128, 2, 2, 3, 1, MT, kOutAcc>, 128, 128, 4 * kWave, 0, N);
    } else if (tiles(64, 128) >= kFill) {
        launch(gemm_tile_kernel<64, 128, 1, 4, 3, 1, MT, kOutAcc>, 64, 128, 4 * kWave, 0, N);
    } else {
        launch(gemm_tile_kernel<64, 64, 2, 2, 3, 1, MT, kOutAcc>, 64, 64, 4 * kWave, 0, N);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, bool fp8,
                       bool tensor_scales, int64_t M, int64_t N, int64_t K, uint16_t* y, void* out_acc,
                       hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (out_acc) {
        if (fp8) return gemm_dispatch<MmaF8x16, MmaF8x32, true>(xq, nullptr, wq, nullptr, M, N, K, nullptr, out_acc, 0, st);
        return gemm_dispatch<MmaI8x16, MmaI8x32, true>(xq, nullptr, wq, nullptr, M, N, K, nullptr, out_acc, 0, st);
    }
    const int t = tensor_scales ? 1 : 0;
    if (fp8) return gemm_dispatch<MmaF8x16, MmaF8x32, false>(xq, x_scale, wq, w_scale, M, N, K, y, nullptr, t, st);
    return gemm_dispatch<MmaI8x16, MmaI8x32, false>(xq, x_scale, wq, w_scale, M, N, K, y, nullptr, t, st);
}

}  // namespace w8a8
