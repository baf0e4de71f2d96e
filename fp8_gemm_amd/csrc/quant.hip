// Activation smooth + per-token quantize, and the weight quantize-and-transpose.
// ("Weight-Activation Quantization", section 3: divide activation channel j by s_j, multiply
// weight channel j by s_j, then both smoothed operands are quantized to 8 bits; section 2:
// symmetric INT8 with scale = absmax / 127; section 4: E4M3 with scale = absmax / 448.)
#include <algorithm>

#include "device.h"
#include "launch.h"

namespace w8a8 {

namespace {

// ---- activations: a row held in the registers of one, two or four waves --------------------------
//
// A block of kActWaves waves quantizes whole rows: kSplit consecutive waves share a row, and each
// group takes `rows_per_wave` rows in turn.  The block first stages s and its correctly rounded
// reciprocals in LDS, so that every X / s and every X~ / scale is a five-operation correctly
// rounded division (div_by_rcp) instead of a full one.  A row is read once from HBM into registers
// (kChunks 16-byte chunks of 8 elements per lane), the lanes of the kSplit waves owning
// interleaved chunks, so that each load instruction of a wave reads 512 consecutive elements; it is
// divided by s, reduced to its maximum with a wave butterfly and, across the row's waves, through
// LDS, and quantized from registers.
//
// Fast-division guards (outside them the full division is used, with identical results):
//   - every s[j] of the block in [2^-20, 2^20];
//   - the row scale in [2^-60, 2^60].
// Then every element whose code can be nonzero, and the row maximum, has X~ >= 2^-10 * scale >=
// 2^-70 and X >= 2^-90, so all quotients and remainders are normal numbers and exact; elements
// below that bound give code 0 on either path.  The row scale is only known after the quotients,
// so a block in which a row's scale comes out of that range (or zero) after fast divisions is
// quantized again with full divisions, which rewrites the same codes and scales.
constexpr int kActWaves = 8;

// LDS layout of s and 1/s: for chunk c (elements 8c .. 8c + 7), the low halves 8c .. 8c + 3 of all
// chunks come first, then the high halves, so that the 16-byte reads of consecutive lanes are
// consecutive (free of bank conflicts).
__device__ __forceinline__ int lds_half(int64_t j, int64_t nchunk) {
    const int64_t c = j >> 3, e = j & 7;
    return static_cast<int>((e >> 2) * nchunk * 4 + c * 4 + (e & 3));
}

template <bool kFast, bool kSmooth, bool kFp8, int kChunks>
__device__ __forceinline__ float smooth_chunks(float (&v)[kChunks][8], const float* sh_s, const float* sh_r,
                                               int lane_c, int stride, int64_t nchunk) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        int64_t c = lane_c + static_cast<int64_t>(stride) * i;
        c = c < nchunk ? c : nchunk - 1;
        {
            if constexpr (kSmooth) {
                const float4 s0 = *reinterpret_cast<const float4*>(sh_s + c * 4);
                const float4 s1 = *reinterpret_cast<const float4*>(sh_s + (nchunk + c) * 4);
                const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                if constexpr (kFast) {
                    const float4 r0 = *reinterpret_cast<const float4*>(sh_r + c * 4);
                    const float4 r1 = *reinterpret_cast<const float4*>(sh_r + (nchunk + c) * 4);
                    const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[i][e] = div_by_rcp<kFp8>(v[i][e], sv[e], rv[e]);
                } else {
                    // The rare full-division path: one division at a time (interleaving 8 or 32 of
                    // them would set the kernel's register count).
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        v[i][e] = div_rn(v[i][e], sv[e]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
        }
        // Each chunk's s and 1 / s are read from LDS where they are used: hoisting the reads of all
        // chunks would hold 16 registers per chunk at once.
        if constexpr (kSmooth) __builtin_amdgcn_sched_barrier(0);
    }
    return amax;
}

template <bool kFp8, bool kFast, int kChunks>
__device__ __forceinline__ void store_codes(const float (&v)[kChunks][8], float sc, float rsc, int lane_c,
                                            int stride, int64_t nchunk, uint8_t* __restrict__ qrow) {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        const int64_t c = lane_c + static_cast<int64_t>(stride) * i;
        if (c < nchunk) {
            float qv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (kFast) {
                    qv[e] = div_by_rcp<kFp8>(v[i][e], sc, rsc);
                } else {
                    qv[e] = div_rn(v[i][e], sc);
                    __builtin_amdgcn_sched_barrier(0);     // one full division at a time, as above
                }
            }
            const uint32_t lo = pack_codes4<kFp8>(qv[0], qv[1], qv[2], qv[3]);
            const uint32_t hi = pack_codes4<kFp8>(qv[4], qv[5], qv[6], qv[7]);
            *reinterpret_cast<uint2*>(qrow + c * 8) = make_uint2(lo, hi);
        }
    }
}

// The body of a block (index bx) of kActWaves waves.  sh: kSmooth: s then 1/s, each K floats
// (lds_half order); xchg: kSplit > 1: the parts' maxima of a row.
template <bool kBf16, bool kFp8, int kChunks, bool kSmooth, int kSplit, bool kOneRow>
__device__ __forceinline__ void quant_act_body(const void* __restrict__ x, const float* __restrict__ s, int64_t M,
                                               int64_t K, int rows_per_wave, uint8_t* __restrict__ q,
                                               float* __restrict__ scale, int64_t bx, float* sh,
                                               float (*xchg)[kActWaves]) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t nchunk = K / 8;
    float* const sh_s = sh;
    float* const sh_r = sh + K;
    // A row is handled by kSplit consecutive waves, which take interleaved 512-element blocks of it.
    constexpr int kRowsPerPass = kActWaves / kSplit;
    const int slot = wave / kSplit;
    const int part = wave % kSplit;
    const int lane_c = part * kWave + lane;     // first chunk of this wave's share
    constexpr int kStride = kSplit * kWave;
    // Loads of the chunks of one row (all unconditional: chunks past the row end re-read the last
    // chunk, which changes no maximum and is never stored), all issued before any conversion.
    auto load_row = [&](Raw8<kBf16> (&raw)[kChunks], int64_t rrow) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            int64_t c = lane_c + static_cast<int64_t>(kStride) * i;
            c = c < nchunk ? c : nchunk - 1;
            raw[i] = load_raw8<kBf16>(x, rrow * K + c * 8);
        }
    };
    // s is staged in LDS with its reciprocals.  kOneRow (rows_per_wave == 1, several waves per row;
    // with one wave per row the compiler keeps the early row in scratch memory): the wave's one row is
    // requested right after the s loads, so that it is in flight while the reciprocals are formed
    // (the loads complete in order, so the wait for s does not wait for the row).
    // K <= kSplit * kChunks * 512: at most kSplit * kChunks elements of s per thread, loaded
    // together (indices past K re-read s[K - 1] and are not stored).
    constexpr int kPer = kSmooth ? kSplit * kChunks : 1;
    float sv[kPer];
    if constexpr (kSmooth) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t j = threadIdx.x + static_cast<int64_t>(i) * (kActWaves * kWave);
            sv[i] = s[j < K ? j : K - 1];
        }
    }
    Raw8<kBf16> first[kChunks];
    if constexpr (kOneRow) {
        const int64_t row = bx * kRowsPerPass + slot;
        load_row(first, row < M ? row : M - 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    bool fast_s = true;
    if constexpr (kSmooth) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t j = threadIdx.x + static_cast<int64_t>(i) * (kActWaves * kWave);
            if (j < K) {
                const int h = lds_half(j, nchunk);
                sh_s[h] = sv[i];
                sh_r[h] = div_rn(1.0f, sv[i]);
                fast_s = fast_s && in_pow2_range<-20, 20>(sv[i]);
            }
        }
        fast_s = __syncthreads_and(fast_s);
    }
    // One pass over the block's rows; X / s by div_by_rcp when fast.  Returns whether a row of this
    // wave came out with a scale outside [2^-60, 2^60] (or zero) after fast divisions: the guard
    // above does not hold there, so the block then takes a second pass with full divisions, in
    // which the same lanes rewrite the same codes and scales.
    auto rows_pass = [&](bool fast) {
        bool redo = false;
        const int nrows = kOneRow ? 1 : rows_per_wave;
        for (int rr = 0; rr < nrows; ++rr) {
            const int64_t row = (bx * nrows + rr) * kRowsPerPass + slot;
            const bool live = row < M;
            if (kSplit == 1 && !live) break;
            const int64_t rrow = live ? row : M - 1;
            Raw8<kBf16> raw[kChunks];
            if (kOneRow && fast) {
#pragma unroll
                for (int i = 0; i < kChunks; ++i) raw[i] = first[i];
            } else {
                load_row(raw, rrow);
            }
            float v[kChunks][8];
#pragma unroll
            for (int i = 0; i < kChunks; ++i) unpack8<kBf16>(raw[i], v[i]);
            float amax = fast ? smooth_chunks<true, kSmooth, kFp8>(v, sh_s, sh_r, lane_c, kStride, nchunk)
                              : smooth_chunks<false, kSmooth, kFp8>(v, sh_s, sh_r, lane_c, kStride, nchunk);
            amax = wave_max(amax);
            if constexpr (kSplit > 1) {
                if (lane == 0) xchg[rr & 1][wave] = amax;
                __syncthreads();
#pragma unroll
                for (int p = 0; p < kSplit; ++p) amax = fmaxf(amax, xchg[rr & 1][slot * kSplit + p]);
            }
            if (!live) continue;
            const float sc = div_rn(amax, qmax<kFp8>());
            const bool sc_fast = in_pow2_range<-60, 60>(sc);
            if (fast && kSmooth && !sc_fast) {
                redo = true;
                continue;                       // written by the second pass
            }
            if (lane == 0 && part == 0) scale[row] = sc;
            uint8_t* const qrow = q + row * K;
            if (sc == 0.0f) {                   // a zero scale gives zero codes
#pragma unroll
                for (int i = 0; i < kChunks; ++i) {
                    const int64_t c = lane_c + static_cast<int64_t>(kStride) * i;
                    if (c < nchunk) *reinterpret_cast<uint2*>(qrow + c * 8) = make_uint2(0u, 0u);
                }
            } else if (sc_fast) {
                store_codes<kFp8, true>(v, sc, div_rn(1.0f, sc), lane_c, kStride, nchunk, qrow);
            } else {
                store_codes<kFp8, false>(v, sc, 0.0f, lane_c, kStride, nchunk, qrow);
            }
        }
        return redo;
    };
    const bool redo = rows_pass(fast_s);
    if (kSmooth && fast_s) {                    // fast_s is uniform over the block
        if (__syncthreads_or(redo)) rows_pass(false);
    }
}

template <bool kBf16, bool kFp8, int kChunks, bool kSmooth, int kSplit, bool kOneRow>
__global__ __launch_bounds__(kActWaves * kWave) void quant_act_kernel(
    const void* __restrict__ x, const float* __restrict__ s, int64_t M, int64_t K, int rows_per_wave,
    uint8_t* __restrict__ q, float* __restrict__ scale) {
    extern __shared__ float sh[];
    __shared__ float xchg[2][kActWaves];
    quant_act_body<kBf16, kFp8, kChunks, kSmooth, kSplit, kOneRow>(x, s, M, K, rows_per_wave, q, scale, blockIdx.x,
                                                                   sh, xchg);
}

// Few rows: one block per row, so that the grid is as wide as the batch, and one round trip to
// memory.  Each thread owns kC chunks of 8 elements and loads its chunks of X and of
// s together (no staging of s: each s element is used once per block); X / s is a full division
// (a reciprocal would be used only once).  The row maximum goes through LDS; the codes then take
// the row scale's reciprocal under the same guard as the many-row kernel.  Chunks past the row
// re-read the last one, which changes no maximum and is not stored.
constexpr int kRowThreads = 512;

template <bool kBf16, bool kFp8, int kC, bool kSmooth>
__global__ __launch_bounds__(kRowThreads) void quant_act_row_kernel(const void* __restrict__ x,
                                                                    const float* __restrict__ s, int64_t K,
                                                                    uint8_t* __restrict__ q,
                                                                    float* __restrict__ scale) {
    __shared__ float red[kRowThreads / kWave];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nwaves = blockDim.x / kWave;
    const int64_t row = blockIdx.x;
    const int64_t nchunk = K / 8;
    Raw8<kBf16> raw[kC];
    float4 sr[kC][2];
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        int64_t c = threadIdx.x + static_cast<int64_t>(i) * blockDim.x;
        c = c < nchunk ? c : nchunk - 1;
        raw[i] = load_raw8<kBf16>(x, row * K + c * 8);
        if constexpr (kSmooth) {
            sr[i][0] = *reinterpret_cast<const float4*>(s + c * 8);
            sr[i][1] = *reinterpret_cast<const float4*>(s + c * 8 + 4);
        }
    }
    float v[kC][8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kC; ++i) {
        unpack8<kBf16>(raw[i], v[i]);
        if constexpr (kSmooth) {
            const float sv[8] = {sr[i][0].x, sr[i][0].y, sr[i][0].z, sr[i][0].w,
                                 sr[i][1].x, sr[i][1].y, sr[i][1].z, sr[i][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = div_rn(v[i][e], sv[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    }
    amax = wave_max(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = red[0];
    for (int w = 1; w < nwaves; ++w) amax = fmaxf(amax, red[w]);
    const float sc = div_rn(amax, qmax<kFp8>());
    if (threadIdx.x == 0) scale[row] = sc;
    uint8_t* const qrow = q + row * K;
    if (sc == 0.0f) {                           // a zero scale gives zero codes
#pragma unroll
        for (int i = 0; i < kC; ++i) {
            const int64_t c = threadIdx.x + static_cast<int64_t>(i) * blockDim.x;
            if (c < nchunk) *reinterpret_cast<uint2*>(qrow + c * 8) = make_uint2(0u, 0u);
        }
    } else if (in_pow2_range<-60, 60>(sc)) {
        store_codes<kFp8, true>(v, sc, div_rn(1.0f, sc), threadIdx.x, blockDim.x, nchunk, qrow);
    } else {
        store_codes<kFp8, false>(v, sc, 0.0f, threadIdx.x, blockDim.x, nchunk, qrow);
    }
}

// Rows longer than the register-resident variants (K > 8192): two passes over the row (the second
// mostly hits the cache), full divisions.
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
        if (sc != 0.0f) {                       // a zero scale gives zero codes
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
// A block of 256 threads owns a tile of kTJ = 256 rows (j) x kTN = 64 columns (n) of W (small
// enough for four blocks per CU).  Loads are coalesced along n: a wave instruction reads 8 rows x
// 128 bytes (bf16).  Each thread handles 8 columns x
// 4 consecutive rows at a time, forms W~ = s[j] * W[j, n] and the codes with the column scales, and
// packs the 4 codes of one column (rows j .. j + 3) into one LDS word; the tile is stored transposed,
// one row of kTJ / 4 words per column n, and written back as 16-byte pieces of wq rows (contiguous
// along j).
//
// LDS word of (column c, row group g = j / 4): c * kTStride + (g ^ (8 * ((c / 8) % 8))).  The row
// stride kTStride = 72 = 8 (mod 64) and the xor make the 64 words one wave writes at a time (8 row
// groups x 8 column chunks) fall in 64 different banks; a 16-byte read of 4 consecutive words
// returns 4 consecutive row groups (the xor only moves whole aligned groups of 8).
//
// The column scales max_j |W~[j, n]| / Q are final when this kernel runs (the column pass divides
// its maxima by Q).  Codes use div_by_rcp with each column's correctly rounded 1 / scale when every
// column scale of the block lies in [2^-60, 2^60] or is 0 (codes 0); then every W~ whose code can
// be nonzero is at least 2^-70 and its quotient and remainders are normal.  Otherwise the block
// divides in full.
constexpr int kTJ = 256;
constexpr int kTN = 64;
constexpr int kTStride = kTJ / 4 + 8;
constexpr int kItems = (kTJ / 4) * (kTN / 8) / 256;   // (row group, column chunk) items per thread
static_assert(kItems >= 1 && kTN % 64 == 0, "8 column chunks per wave instruction");

template <bool kBf16>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
    if constexpr (kBf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(base)[i]) << 16);
    else return static_cast<const float*>(base)[i];
}

// Loads of one (row group, column chunk) item: rows j .. j + 3, columns n .. n + 7.  Unconditional
// (rows past K and columns past N re-read the last ones; their codes land in tile positions that
// are never stored), so that all of a thread's loads are in flight at once.
template <bool kBf16, bool kVec>
struct WeightItem {
    Raw8<kBf16> raw[4];       // kVec
    float val[kVec ? 1 : 4][kVec ? 1 : 8];
};

template <bool kBf16, bool kVec>
__device__ __forceinline__ void load_item(const void* __restrict__ w, int64_t K, int64_t N, int64_t j, int64_t n,
                                          WeightItem<kBf16, kVec>& it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t jr = (j + i < K) ? j + i : K - 1;
        if constexpr (kVec) {
            it.raw[i] = load_raw8<kBf16>(w, jr * N + (n < N ? n : N - 8));
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) it.val[i][e] = load1<kBf16>(w, jr * N + (n + e < N ? n + e : N - 1));
        }
    }
}

template <bool kBf16, bool kFp8, bool kVec, bool kFast>
__device__ __forceinline__ void code_item(const WeightItem<kBf16, kVec>& it, const float (&sj)[4],
                                          const float* col_scale, const float* col_rcp, int cl0,
                                          uint32_t* __restrict__ tile, int g) {
    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (kVec) {
            unpack8<kBf16>(it.raw[i], v[i]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = it.val[i][e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = cl0 + e;
        const float sc = col_scale[c];
        float qv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ws = sj[i] * v[i][e];
            qv[i] = kFast ? div_by_rcp<kFp8>(ws, sc, col_rcp[c]) : div_rn(ws, sc);
        }
        const uint32_t word = (sc != 0.0f) ? pack_codes4<kFp8>(qv[0], qv[1], qv[2], qv[3]) : 0u;
        tile[c * kTStride + (g ^ (8 * ((c >> 3) & 7)))] = word;
    }
}

// LDS of one weight tile.
struct WeightTileLds {
    uint32_t tile[kTN * kTStride];
    float col_scale[kTN], col_rcp[kTN], row_s[kTJ];
};

// The body of one tile (bx, by) = (column tile, row tile), run by 256 threads with index tid.  Its
// barriers are block-wide, so every thread of the block runs it (a second tile of a 512-thread
// block, or an inactive one that loads and codes a valid tile and stores nothing).
// kStream: nontemporal stores of the codes, for the weight preparation on its own, whose codes are
// read later, by GEMMs of later calls (cached stores would only displace W from the caches); the
// one-call preparation, whose GEMM follows at once, keeps them cached.
template <bool kBf16, bool kFp8, bool kVec, bool kStream>
__device__ __forceinline__ void weight_tile_body(const void* __restrict__ w, int64_t K, int64_t N,
                                                 const float* __restrict__ s, const float* __restrict__ w_scale,
                                                 int64_t scale_step, uint8_t* __restrict__ wq, int64_t bx, int64_t by,
                                                 int tid, bool active, WeightTileLds& L) {
    uint32_t* const tile = L.tile;
    float* const col_scale = L.col_scale;
    float* const col_rcp = L.col_rcp;
    float* const row_s = L.row_s;
    const int64_t n0 = bx * kTN;
    const int64_t j0 = by * kTJ;
    const int wave = tid / kWave, lane = tid % kWave;
    const int cl = lane & 7, rl = lane >> 3;
    // The column scale and s element of this thread, then the tile's loads, all issued before the
    // staging and its barrier so that the tile is in flight meanwhile.
    const int64_t n_t = n0 + tid, j_t = j0 + tid;
    const float sc_t = (tid < kTN && n_t < N) ? w_scale[n_t * scale_step] : 0.0f;
    const float s_t = (s && j_t < K) ? s[j_t] : 1.0f;
    // kTJ / 4 row groups x kTN / 8 column chunks, kItems (group, chunk) items per thread.  Item it of
    // wave w is combination b = kItems w + it: column chunk cc = cl + 8 (b / (kTJ / 32)), row group
    // g = rl + 8 (b % (kTJ / 32)).
    WeightItem<kBf16, kVec> items[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int b = wave * kItems + it;
        const int cc = cl + 8 * (b / (kTJ / 32)), g = rl + 8 * (b % (kTJ / 32));
        load_item<kBf16, kVec>(w, K, N, j0 + 4 * g, n0 + 8 * cc, items[it]);
    }
    bool fast = true;
    if (tid < kTN) {
        col_scale[tid] = sc_t;
        col_rcp[tid] = div_rn(1.0f, sc_t);
        fast = sc_t == 0.0f || in_pow2_range<-60, 60>(sc_t);
    }
    row_s[tid] = s_t;
    fast = __syncthreads_and(fast);
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int b = wave * kItems + it;
        const int cc = cl + 8 * (b / (kTJ / 32)), g = rl + 8 * (b % (kTJ / 32));
        const float sj[4] = {row_s[4 * g], row_s[4 * g + 1], row_s[4 * g + 2], row_s[4 * g + 3]};
        if (fast) code_item<kBf16, kFp8, kVec, true>(items[it], sj, col_scale, col_rcp, 8 * cc, tile, g);
        else code_item<kBf16, kFp8, kVec, false>(items[it], sj, col_scale, col_rcp, 8 * cc, tile, g);
    }
    __syncthreads();
    // Row n0 + c of wq gets 16-byte piece t (tile rows 16 t .. 16 t + 15 = row groups 4 t .. 4 t + 3,
    // stored at word 4 (t ^ 2 ((c / 8) % 8))).  16 consecutive threads read one column's 256 bytes.
    for (int idx = tid; idx < kTN * (kTJ / 16); idx += 256) {
        const int c = idx / (kTJ / 16), t = idx % (kTJ / 16);
        const int64_t n = n0 + c, j = j0 + 16 * t;
        const uint4 u = *reinterpret_cast<const uint4*>(&tile[c * kTStride + 4 * (t ^ (2 * ((c >> 3) & 7)))]);
        if (active && n < N && j < K) {                                                  // K % 16 == 0
            if constexpr (kStream) {
                typedef unsigned int v4u __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(v4u{u.x, u.y, u.z, u.w}, reinterpret_cast<v4u*>(wq + n * K + j));
            } else {
                *reinterpret_cast<uint4*>(wq + n * K + j) = u;
            }
        }
    }
}

template <bool kBf16, bool kFp8, bool kVec>
__global__ __launch_bounds__(256) void quant_weight_t_kernel(const void* __restrict__ w, int64_t K, int64_t N,
                                                             const float* __restrict__ s,
                                                             const float* __restrict__ w_scale, int64_t scale_step,
                                                             uint8_t* __restrict__ wq) {
    __shared__ WeightTileLds L;
    weight_tile_body<kBf16, kFp8, kVec, true>(w, K, N, s, w_scale, scale_step, wq, blockIdx.x, blockIdx.y, threadIdx.x, true,
                                        L);
}

// ---- the activation and weight codes of one layer in one launch -------------------------------
// Both need only s and the final weight scales, so blocks [0, nq) quantize activations (as
// quant_act_kernel) and the others code two weight tiles each (as quant_weight_t_kernel, waves 0-3
// and 4-7); tile 2b + 1 past the last tile is inactive.  One dynamic LDS buffer serves either role.
template <bool kBf16, bool kFp8, int kChunks, int kSplit, bool kOneRow>
__global__ __launch_bounds__(kActWaves * kWave) void quant_pair_kernel(
    const void* __restrict__ x, const float* __restrict__ s, int64_t M, int64_t K, int rows_per_wave,
    uint8_t* __restrict__ xq, float* __restrict__ x_scale, const void* __restrict__ w, int64_t N,
    const float* __restrict__ w_scale, uint8_t* __restrict__ wq, unsigned nq, unsigned wtx, unsigned ntiles) {
    extern __shared__ float4 lds4[];
    if (blockIdx.x < nq) {
        float* const sh = reinterpret_cast<float*>(lds4);
        float (*xchg)[kActWaves] = reinterpret_cast<float (*)[kActWaves]>(sh + 2 * K);
        quant_act_body<kBf16, kFp8, kChunks, true, kSplit, kOneRow>(x, s, M, K, rows_per_wave, xq, x_scale,
                                                                    blockIdx.x, sh, xchg);
    } else {
        const int half = threadIdx.x / 256;
        WeightTileLds* const L = reinterpret_cast<WeightTileLds*>(lds4) + half;
        const unsigned t = 2 * (blockIdx.x - nq) + half;
        const bool active = t < ntiles;
        const unsigned tc = active ? t : ntiles - 1;
        weight_tile_body<kBf16, kFp8, true, false>(w, K, N, s, w_scale, 1, wq, tc % wtx, tc / wtx, threadIdx.x % 256, active,
                                            *L);
    }
}

// ---- RMS norm with the smoothing folded into its gain, then per-token quantize --------------------
// ("Weight-Activation Quantization", s3 step 1: the SmoothQuant transform is done offline; the
// W8A16-vs-W8A8 lesson, s2: no runtime overhead.)  X~[j] = (h[j] * r) * g'[j] with
// g' = g / s folded once, r = 1 / sqrt(mean(h^2) + eps), then the per-token quantize of X~: one HBM
// pass over the residual stream h, which replaces the norm kernel's output and the activation
// quantize's read of it.
//
// The row is register-resident as in quant_act_kernel (kSplit waves per row).  The float mean
// square must not depend on the order of the sum.  Each square of a float is exact in double, and a
// plain double sum of them through at most 41 additions (32 per lane, 6 across the wave, 3 across
// the parts) is within 41 * 2^-53 < 2^-47 of the exact sum.  The mean is taken as certified when
// both ends of a 2^-44 band around the estimate round to the same float: the exactly rounded mean
// lies in the band, so it is that float.  Otherwise (about one row in 2^19) the sum is redone in
// double-double (error-free TwoSum additions, within about 2^-100 of the exact sum in any order)
// and the mean taken from it, as a sequential exact sum would give it.

// (hi, lo) + x for |lo| <= ulp(hi) / 2.
__device__ __forceinline__ void dd_add(double& hi, double& lo, double x) {
    const double s = hi + x;
    const double bb = s - hi;
    const double e = (hi - (s - bb)) + (x - bb) + lo;
    hi = s + e;
    lo = e - (hi - s);
}

// (hi, lo) + (h2, l2).
__device__ __forceinline__ void dd_merge(double& hi, double& lo, double h2, double l2) {
    const double s = hi + h2;
    const double bb = s - hi;
    const double e = (hi - (s - bb)) + (h2 - bb) + lo + l2;
    hi = s + e;
    lo = e - (hi - s);
}

// The float mean of a sum estimate within 2^-47 of the exact sum, or -1 when the band around it
// straddles a float rounding boundary.  inv_k = 1/K in double (relative error 2^-53).
__device__ __forceinline__ float certified_mean(double sum, double inv_k) {
    const double q = sum * inv_k;
    const float lo = static_cast<float>(q - q * 0x1p-44);
    const float hi = static_cast<float>(q + q * 0x1p-44);
    return lo == hi ? lo : -1.0f;
}

// The float mean of a signed sum of K terms, into out; false when it cannot be certified.  When
// every term is a multiple of 2^qexp and abs_sum <= 2^(52 + qexp) (a factor 2 of margin over 2^53
// for the rounding of abs_sum itself), every partial sum is exact in double, so sum is the exact
// sum and the correctly rounded sum / K is the value the exact mean rounds to (inputs with few
// significant bits, as bf16, often land exactly on a float tie, and this decides it).  Otherwise
// the estimate is within 2^-47 of abs_sum from the exact sum and the band test applies.
__device__ __forceinline__ bool certified_mean_signed(double sum, double abs_sum, int qexp, int64_t K, float& out) {
    if (abs_sum <= __builtin_ldexp(1.0, 52 + qexp)) {
        out = static_cast<float>(sum / static_cast<double>(K));
        return true;
    }
    const double inv_k = 1.0 / static_cast<double>(K);
    const double q = sum * inv_k;
    const double err = abs_sum * inv_k * 0x1p-44;
    const float lo = static_cast<float>(q - err);
    const float hi = static_cast<float>(q + err);
    out = lo;
    return lo == hi;
}

// The row's mean of v (kSquare: of v^2) from the double-double sum of this lane's terms: a
// butterfly across the wave, then (kSplit > 1) an exchange across the row's waves.  Called by
// every wave of the block.
template <int kChunks, int kSplit, bool kSquare = true>
__device__ __forceinline__ float dd_mean(const float (&v)[kChunks][8], int lane_c, int64_t nchunk, int64_t K,
                                         int lane, int wave, int slot, double (*xhi)[kActWaves],
                                         double (*xlo)[kActWaves], int buf) {
    constexpr int kStride = kSplit * kWave;
    double hi = 0.0, lo = 0.0;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
        if (lane_c + static_cast<int64_t>(kStride) * i < nchunk) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dd_add(hi, lo, kSquare ? static_cast<double>(v[i][e]) * static_cast<double>(v[i][e])
                                       : static_cast<double>(v[i][e]));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double h2 = __shfl_xor(hi, off, kWave), l2 = __shfl_xor(lo, off, kWave);
        dd_merge(hi, lo, h2, l2);
    }
    if constexpr (kSplit > 1) {
        if (lane == 0) {
            xhi[buf][wave] = hi;
            xlo[buf][wave] = lo;
        }
        __syncthreads();
        hi = xhi[buf][slot * kSplit];
        lo = xlo[buf][slot * kSplit];
#pragma unroll
        for (int p = 1; p < kSplit; ++p) dd_merge(hi, lo, xhi[buf][slot * kSplit + p], xlo[buf][slot * kSplit + p]);
    }
    return static_cast<float>((hi + lo) / static_cast<double>(K));
}

// Norm kinds: RMS norm without or with a gain, and LayerNorm (gain g' and bias b', staged as 1
// and 0 where not given).
constexpr int kRmsNorm = 0, kRmsNormGain = 1, kLayerNorm = 2;

// LayerNorm ("Weight-Activation Quantization", s3 step 1 with the norm before the layer a
// LayerNorm: 1/s folded into both gain and bias): mu = the float mean of the exact sum of h, d =
// h - mu in fp32, var = the float mean of the exact sum of d^2, r = 1 / sqrt(var + eps), X~ =
// (d * r) * g' + b' rounded after each operation.  The mean's sum has signed terms: its plain
// double estimate is exact when the row's values are multiples of a quantum small enough, and is
// otherwise certified against a band of 2^-44 of the sum of |h| (the error bound of the 41
// additions is 41 * 2^-53 of it), with the same double-double fallback.
template <bool kBf16, bool kFp8, int kChunks, int kMode, int kSplit>
__global__ __launch_bounds__(kActWaves * kWave) void norm_quant_kernel(
    const void* __restrict__ h, const float* __restrict__ g, const float* __restrict__ b, float eps, int64_t M,
    int64_t K, int rows_per_wave, uint8_t* __restrict__ q, float* __restrict__ scale) {
    constexpr bool kGain = kMode != kRmsNorm, kLayer = kMode == kLayerNorm;
    extern __shared__ float sh_g[];             // kGain: g', K floats; kLayer: then b', K floats (lds_half order)
    __shared__ double xsum[2][kActWaves], xhi[2][kActWaves], xlo[2][kActWaves];
    __shared__ double xmsum[2][kActWaves], xmabs[2][kActWaves], xmhi[2][kActWaves], xmlo[2][kActWaves];
    __shared__ int xmexp[2][kActWaves];
    __shared__ float xmax[2][kActWaves];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t nchunk = K / 8;
    float* const sh_b = sh_g + K;
    if constexpr (kGain) {
        constexpr int kPer = kSplit * kChunks;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t j = threadIdx.x + static_cast<int64_t>(i) * blockDim.x;
            if (j < K) {
                const int hj = lds_half(j, nchunk);
                sh_g[hj] = (!kLayer || g) ? g[j] : 1.0f;
                if constexpr (kLayer) sh_b[hj] = b ? b[j] : 0.0f;
            }
        }
        __syncthreads();
    }
    constexpr int kRowsPerPass = kActWaves / kSplit;
    const int slot = wave / kSplit;
    const int part = wave % kSplit;
    const int lane_c = part * kWave + lane;
    constexpr int kStride = kSplit * kWave;
    for (int rr = 0; rr < rows_per_wave; ++rr) {
        const int64_t row = (static_cast<int64_t>(blockIdx.x) * rows_per_wave + rr) * kRowsPerPass + slot;
        const bool live = row < M;
        if (kSplit == 1 && !live) break;
        const int64_t rrow = live ? row : M - 1;
        Raw8<kBf16> raw[kChunks];
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            int64_t c = lane_c + static_cast<int64_t>(kStride) * i;
            c = c < nchunk ? c : nchunk - 1;
            raw[i] = load_raw8<kBf16>(h, rrow * K + c * 8);
        }
        float v[kChunks][8];
#pragma unroll
        for (int i = 0; i < kChunks; ++i) unpack8<kBf16>(raw[i], v[i]);
        const double inv_k = 1.0 / static_cast<double>(K);
        if constexpr (kLayer) {
            // The mean, then v becomes d = v - mu (fp32).
            // Sum, sum of |h| and the smallest exponent of a nonzero h (frexp: |h| = m 2^e, m in
            // [1/2, 1)); a nonzero input is then a multiple of 2^(e - kMant).
            constexpr int kMant = kBf16 ? 8 : 24;
            double msum = 0.0, mabs = 0.0;
            int mexp = 1 << 20;
#pragma unroll
            for (int i = 0; i < kChunks; ++i) {
                if (lane_c + static_cast<int64_t>(kStride) * i < nchunk) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const double d = static_cast<double>(v[i][e]);
                        msum += d;
                        mabs += __builtin_fabs(d);
                        mexp = min(mexp, v[i][e] != 0.0f ? __builtin_amdgcn_frexp_expf(v[i][e]) : (1 << 20));
                    }
                }
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                msum += __shfl_xor(msum, off, kWave);
                mabs += __shfl_xor(mabs, off, kWave);
                mexp = min(mexp, __shfl_xor(mexp, off, kWave));
            }
            float mu;
            if constexpr (kSplit == 1) {
                if (!certified_mean_signed(msum, mabs, mexp - kMant, K, mu))
                    mu = dd_mean<kChunks, 1, false>(v, lane_c, nchunk, K, lane, wave, slot, xmhi, xmlo, rr & 1);
            } else {
                if (lane == 0) {
                    xmsum[rr & 1][wave] = msum;
                    xmabs[rr & 1][wave] = mabs;
                    xmexp[rr & 1][wave] = mexp;
                }
                __syncthreads();
                bool straddle = false;
                mu = 0.0f;
#pragma unroll
                for (int t = 0; t < kRowsPerPass; ++t) {
                    double st = xmsum[rr & 1][t * kSplit], sa = xmabs[rr & 1][t * kSplit];
                    int se = xmexp[rr & 1][t * kSplit];
#pragma unroll
                    for (int p = 1; p < kSplit; ++p) {
                        st += xmsum[rr & 1][t * kSplit + p];
                        sa += xmabs[rr & 1][t * kSplit + p];
                        se = min(se, xmexp[rr & 1][t * kSplit + p]);
                    }
                    float mt;
                    straddle |= !certified_mean_signed(st, sa, se - kMant, K, mt);
                    if (t == slot) mu = mt;
                }
                if (straddle)
                    mu = dd_mean<kChunks, kSplit, false>(v, lane_c, nchunk, K, lane, wave, slot, xmhi, xmlo, rr & 1);
            }
#pragma unroll
            for (int i = 0; i < kChunks; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) v[i][e] = __fsub_rn(v[i][e], mu);
        }
        // Sum of squares over this lane's chunks (re-read chunks past the row end do not count): a
        // plain double sum of exact squares, the same in every lane after the xor butterfly.
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            if (lane_c + static_cast<int64_t>(kStride) * i < nchunk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double d = static_cast<double>(v[i][e]);
                    sum = __builtin_fma(d, d, sum);
                }
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, kWave);
        float ms;
        if constexpr (kSplit == 1) {
            ms = certified_mean(sum, inv_k);
            if (ms < 0.0f) ms = dd_mean<kChunks, 1>(v, lane_c, nchunk, K, lane, wave, slot, xhi, xlo, rr & 1);
        } else {
            // Every wave certifies every row of the pass, so the fallback (which has a barrier) is
            // taken by the whole block or not at all.
            if (lane == 0) xsum[rr & 1][wave] = sum;
            __syncthreads();
            bool straddle = false;
            ms = 0.0f;
#pragma unroll
            for (int t = 0; t < kRowsPerPass; ++t) {
                double st = xsum[rr & 1][t * kSplit];
#pragma unroll
                for (int p = 1; p < kSplit; ++p) st += xsum[rr & 1][t * kSplit + p];
                const float mt = certified_mean(st, inv_k);
                straddle |= mt < 0.0f;
                if (t == slot) ms = mt;
            }
            if (straddle) ms = dd_mean<kChunks, kSplit>(v, lane_c, nchunk, K, lane, wave, slot, xhi, xlo, rr & 1);
        }
        const float r = div_rn(1.0f, __builtin_sqrtf(ms + eps));
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            int64_t c = lane_c + static_cast<int64_t>(kStride) * i;
            c = c < nchunk ? c : nchunk - 1;
            float gv[8] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
            if constexpr (kGain) {
                const float4 g0 = *reinterpret_cast<const float4*>(sh_g + c * 4);
                const float4 g1 = *reinterpret_cast<const float4*>(sh_g + (nchunk + c) * 4);
                gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w;
                gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
            }
            if constexpr (kLayer) {
                const float4 b0 = *reinterpret_cast<const float4*>(sh_b + c * 4);
                const float4 b1 = *reinterpret_cast<const float4*>(sh_b + (nchunk + c) * 4);
                const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // Each operation rounded on its own: the compiler must not fuse the multiply
                    // and the add.
#pragma clang fp contract(off)
                    const float t = (v[i][e] * r) * gv[e];
                    v[i][e] = t + bv[e];
                    amax = fmaxf(amax, fabsf(v[i][e]));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    v[i][e] = (v[i][e] * r) * gv[e];
                    amax = fmaxf(amax, fabsf(v[i][e]));
                }
            }
        }
        amax = wave_max(amax);
        if constexpr (kSplit > 1) {
            if (lane == 0) xmax[rr & 1][wave] = amax;
            __syncthreads();
#pragma unroll
            for (int p = 0; p < kSplit; ++p) amax = fmaxf(amax, xmax[rr & 1][slot * kSplit + p]);
        }
        if (!live) continue;
        const float sc = div_rn(amax, qmax<kFp8>());
        if (lane == 0 && part == 0) scale[row] = sc;
        uint8_t* const qrow = q + row * K;
        if (sc == 0.0f) {                       // a zero scale gives zero codes
#pragma unroll
            for (int i = 0; i < kChunks; ++i) {
                const int64_t c = lane_c + static_cast<int64_t>(kStride) * i;
                if (c < nchunk) *reinterpret_cast<uint2*>(qrow + c * 8) = make_uint2(0u, 0u);
            }
        } else if (in_pow2_range<-60, 60>(sc)) {
            store_codes<kFp8, true>(v, sc, div_rn(1.0f, sc), lane_c, kStride, nchunk, qrow);
        } else {
            store_codes<kFp8, false>(v, sc, 0.0f, lane_c, kStride, nchunk, qrow);
        }
    }
}

template <bool kBf16, bool kFp8, int kChunks, int kSplit>
void norm_quant_launch(const void* h, const float* g, const float* b, bool layer, float eps, int64_t M, int64_t K,
                       uint8_t* xq, float* xs, hipStream_t st) {
    const int64_t rows_per_pass = kActWaves / kSplit;
    const int64_t rows_per_block_pass = rows_per_pass * 512;
    const int rpw = static_cast<int>(std::max<int64_t>(1, (M + rows_per_block_pass - 1) / rows_per_block_pass));
    const int64_t rows_per_block = rows_per_pass * rpw;
    dim3 grid(static_cast<unsigned>((M + rows_per_block - 1) / rows_per_block)), block(kActWaves * kWave);
    if (layer)
        hipLaunchKernelGGL((norm_quant_kernel<kBf16, kFp8, kChunks, kLayerNorm, kSplit>), grid, block,
                           2 * static_cast<size_t>(K) * sizeof(float), st, h, g, b, eps, M, K, rpw, xq, xs);
    else if (g)
        hipLaunchKernelGGL((norm_quant_kernel<kBf16, kFp8, kChunks, kRmsNormGain, kSplit>), grid, block,
                           static_cast<size_t>(K) * sizeof(float), st, h, g, b, eps, M, K, rpw, xq, xs);
    else
        hipLaunchKernelGGL((norm_quant_kernel<kBf16, kFp8, kChunks, kRmsNorm, kSplit>), grid, block, 0, st, h, g, b,
                           eps, M, K, rpw, xq, xs);
}

template <bool kBf16, bool kFp8>
hipError_t norm_quant_dispatch(const void* h, const float* g, const float* b, bool layer, float eps, int64_t M,
                               int64_t K, uint8_t* xq, float* xs, hipStream_t st) {
    const int64_t per_lane = (K / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) norm_quant_launch<kBf16, kFp8, 1, 1>(h, g, b, layer, eps, M, K, xq, xs, st);
    else if (per_lane <= 2) norm_quant_launch<kBf16, kFp8, 2, 1>(h, g, b, layer, eps, M, K, xq, xs, st);
    else if (per_lane <= 4) norm_quant_launch<kBf16, kFp8, 4, 1>(h, g, b, layer, eps, M, K, xq, xs, st);
    else if (per_lane <= 8) norm_quant_launch<kBf16, kFp8, 4, 2>(h, g, b, layer, eps, M, K, xq, xs, st);
    else if (per_lane <= 16) norm_quant_launch<kBf16, kFp8, 4, 4>(h, g, b, layer, eps, M, K, xq, xs, st);
    else return hipErrorInvalidValue;       // K > 8192: refused by the C ABI before this point
    return hipGetLastError();
}

__global__ void fold_gain_kernel(const float* __restrict__ g, const float* __restrict__ s, int64_t K,
                                 float* __restrict__ out) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j < K) out[j] = div_rn(g ? g[j] : 1.0f, s ? s[j] : 1.0f);
}

template <bool kBf16, bool kFp8, int kChunks, int kSplit>
void quant_act_launch(const void* x, int64_t M, int64_t K, const float* s, uint8_t* xq, float* xs, hipStream_t st) {
    // Rows per wave: one, or more once there are enough rows for two blocks per CU on 256 CUs.
    const int64_t rows_per_pass = kActWaves / kSplit;
    const int64_t rows_per_block_pass = rows_per_pass * 512;
    const int rpw = static_cast<int>(std::max<int64_t>(1, (M + rows_per_block_pass - 1) / rows_per_block_pass));
    const int64_t rows_per_block = rows_per_pass * rpw;
    dim3 grid(static_cast<unsigned>((M + rows_per_block - 1) / rows_per_block)), block(kActWaves * kWave);
    if (s) {
        const size_t lds = 2 * static_cast<size_t>(K) * sizeof(float);
        // One row per wave group: the early-row form (instantiated for kSplit > 1 only).
        if (rpw == 1 && kSplit > 1)
            hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, kChunks, true, kSplit, kSplit != 1>), grid, block, lds,
                               st, x, s, M, K, rpw, xq, xs);
        else
            hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, kChunks, true, kSplit, false>), grid, block, lds, st, x, s,
                               M, K, rpw, xq, xs);
    } else {
        hipLaunchKernelGGL((quant_act_kernel<kBf16, kFp8, kChunks, false, kSplit, false>), grid, block, 0, st, x, s, M,
                           K, rpw, xq, xs);
    }
}

template <bool kBf16, bool kFp8, int kC>
void quant_act_rows_launch(const void* x, int64_t M, int64_t K, const float* s, uint8_t* xq, float* xs,
                           hipStream_t st) {
    const int64_t nchunk = K / 8;
    const int64_t per_thread_waves = (nchunk + kC * kWave - 1) / (kC * kWave);       // 1 .. 8
    const dim3 grid(static_cast<unsigned>(M)), block(static_cast<unsigned>(per_thread_waves * kWave));
    if (s) hipLaunchKernelGGL((quant_act_row_kernel<kBf16, kFp8, kC, true>), grid, block, 0, st, x, s, K, xq, xs);
    else hipLaunchKernelGGL((quant_act_row_kernel<kBf16, kFp8, kC, false>), grid, block, 0, st, x, s, K, xq, xs);
}

// Batches of up to this many rows take one block per row (K = 4096, bf16: 3.2 / 3.5 / 4.0 / 6.2 µs
// at 16 / 256 / 512 / 1024 rows against 3.2 / 5.6 / 5.7 / 6.8 µs for the many-row kernel; at 2048
// rows 9.6 against 9.1 µs, where re-reading s per row and the full divisions cost more than the
// wider grid gains).
constexpr int64_t kRowKernelMaxM = 1024;

template <bool kBf16, bool kFp8>
hipError_t quant_act_dispatch(const void* x, int64_t M, int64_t K, const float* s, uint8_t* xq, float* xs,
                              hipStream_t st) {
    if (M <= kRowKernelMaxM && K <= 8 * kRowThreads * 2) {
        if (K <= 8 * kRowThreads) quant_act_rows_launch<kBf16, kFp8, 1>(x, M, K, s, xq, xs, st);
        else quant_act_rows_launch<kBf16, kFp8, 2>(x, M, K, s, xq, xs, st);
        return hipGetLastError();
    }
    const int64_t per_lane = (K / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) quant_act_launch<kBf16, kFp8, 1, 1>(x, M, K, s, xq, xs, st);
    else if (per_lane <= 2) quant_act_launch<kBf16, kFp8, 2, 1>(x, M, K, s, xq, xs, st);
    else if (per_lane <= 4) quant_act_launch<kBf16, kFp8, 4, 1>(x, M, K, s, xq, xs, st);
    // K in (2048, 8192]: two or four waves per row (more, smaller waves interleave the loads and
    // the arithmetic of different rows better than one wave holding the whole row).
    else if (per_lane <= 8) quant_act_launch<kBf16, kFp8, 4, 2>(x, M, K, s, xq, xs, st);
    else if (per_lane <= 16) quant_act_launch<kBf16, kFp8, 4, 4>(x, M, K, s, xq, xs, st);
    else hipLaunchKernelGGL((quant_act_long_kernel<kBf16, kFp8>), dim3(static_cast<unsigned>((M + 3) / 4)), dim3(256), 0,
                            st, x, s, M, K, xq, xs);
    return hipGetLastError();
}

template <bool kBf16, bool kFp8, int kChunks, int kSplit>
void quant_pair_launch(const void* x, int64_t M, int64_t K, const float* s, uint8_t* xq, float* xs, const void* w,
                       int64_t N, const float* w_scale, uint8_t* wq, hipStream_t st) {
    const int64_t rows_per_pass = kActWaves / kSplit;
    const int64_t rows_per_block_pass = rows_per_pass * 512;
    const int rpw = static_cast<int>(std::max<int64_t>(1, (M + rows_per_block_pass - 1) / rows_per_block_pass));
    const int64_t rows_per_block = rows_per_pass * rpw;
    const int64_t nq = (M + rows_per_block - 1) / rows_per_block;
    const int64_t wtx = (N + kTN - 1) / kTN;
    const int64_t ntiles = wtx * ((K + kTJ - 1) / kTJ);
    const size_t lds = std::max(2 * static_cast<size_t>(K) * sizeof(float) + 2 * kActWaves * sizeof(float),
                                2 * sizeof(WeightTileLds));
    const dim3 grid(static_cast<unsigned>(nq + (ntiles + 1) / 2)), block(kActWaves * kWave);
    if (rpw == 1 && kSplit > 1)          // the early-row form, as in quant_act_launch
        hipLaunchKernelGGL((quant_pair_kernel<kBf16, kFp8, kChunks, kSplit, kSplit != 1>), grid, block, lds, st, x, s, M, K,
                           rpw, xq, xs, w, N, w_scale, wq, static_cast<unsigned>(nq), static_cast<unsigned>(wtx),
                           static_cast<unsigned>(ntiles));
    else
        hipLaunchKernelGGL((quant_pair_kernel<kBf16, kFp8, kChunks, kSplit, false>), grid, block, lds, st, x, s, M, K,
                           rpw, xq, xs, w, N, w_scale, wq, static_cast<unsigned>(nq), static_cast<unsigned>(wtx),
                           static_cast<unsigned>(ntiles));
}

// K <= 8192, N % 8 == 0, M, N >= 1.
template <bool kBf16, bool kFp8>
hipError_t quant_pair_dispatch(const void* x, int64_t M, int64_t K, const float* s, uint8_t* xq, float* xs,
                               const void* w, int64_t N, const float* w_scale, uint8_t* wq, hipStream_t st) {
    const int64_t per_lane = (K / 8 + kWave - 1) / kWave;
    if (per_lane <= 1) quant_pair_launch<kBf16, kFp8, 1, 1>(x, M, K, s, xq, xs, w, N, w_scale, wq, st);
    else if (per_lane <= 2) quant_pair_launch<kBf16, kFp8, 2, 1>(x, M, K, s, xq, xs, w, N, w_scale, wq, st);
    else if (per_lane <= 4) quant_pair_launch<kBf16, kFp8, 4, 1>(x, M, K, s, xq, xs, w, N, w_scale, wq, st);
    else if (per_lane <= 8) quant_pair_launch<kBf16, kFp8, 4, 2>(x, M, K, s, xq, xs, w, N, w_scale, wq, st);
    else if (per_lane <= 16) quant_pair_launch<kBf16, kFp8, 4, 4>(x, M, K, s, xq, xs, w, N, w_scale, wq, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool kBf16, bool kFp8>
hipError_t quant_weight_dispatch(const void* w, int64_t K, int64_t N, const float* s, const float* w_scale,
                                 int64_t scale_step, uint8_t* wq, hipStream_t st) {
    dim3 grid(static_cast<unsigned>((N + kTN - 1) / kTN), static_cast<unsigned>((K + kTJ - 1) / kTJ));
    if (N % 8 == 0)
        hipLaunchKernelGGL((quant_weight_t_kernel<kBf16, kFp8, true>), grid, dim3(256), 0, st, w, K, N, s, w_scale,
                           scale_step, wq);
    else
        hipLaunchKernelGGL((quant_weight_t_kernel<kBf16, kFp8, false>), grid, dim3(256), 0, st, w, K, N, s, w_scale,
                           scale_step, wq);
    return hipGetLastError();
}

// ---- per-tensor quantize ("Weight-Activation Quantization", s4 "Per-Tensor Scaling for FP8") ----
//
// One scale for the whole tensor, scale = amax_in[0] / Q, so the kernel is a plain stream of
// 16-byte chunks: 8 elements in, 8 codes out.  Block b streams its own contiguous range of chunks,
// kU chunks in flight per thread.  Under delayed scaling amax_in is an earlier tensor's maximum and values beyond Q * scale
// saturate; kTrack merges this tensor's maximum into amax_out in the same pass (an atomic maximum
// per block, skipped when amax_out already holds as much).  Division: the fast exact form when the
// scale is in [2^-60, 2^60], else the full one.  Elements are first clamped to +-2 Q scale, which
// changes no code (both quotients saturate) and keeps the fast form's intermediates finite.
template <bool kBf16, bool kFp8, bool kTrack>
__global__ __launch_bounds__(256) void quant_tensor_kernel(const void* __restrict__ a, int64_t nchunk,
                                                           const float* __restrict__ amax_in, uint8_t* __restrict__ q,
                                                           float* __restrict__ scale_out,
                                                           float* __restrict__ amax_out) {
    constexpr int kU = 4;
    const float sc = div_rn(amax_in[0], qmax<kFp8>());
    if (blockIdx.x == 0 && threadIdx.x == 0) scale_out[0] = sc;
    const bool fast = in_pow2_range<-60, 60>(sc);
    const float rsc = fast ? div_rn(1.0f, sc) : 0.0f;
    const float lim = 2.0f * qmax<kFp8>() * sc;
    const int64_t lo = block_range_lo(nchunk), hi = block_range_hi(nchunk);
    float m = 0.0f;
    for (int64_t c0 = lo + threadIdx.x; c0 < hi; c0 += kU * blockDim.x) {
        Raw8<kBf16> raw[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t c = c0 + u * blockDim.x;
            raw[u] = load_raw8<kBf16>(a, (c < hi ? c : hi - 1) * 8);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int64_t c = c0 + u * blockDim.x;
            float v[8];
            unpack8<kBf16>(raw[u], v);
            if constexpr (kTrack) {
#pragma unroll
                for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
            }
            if (c >= hi) continue;
            uint32_t clo = 0, chi = 0;
            if (sc != 0.0f) {                   // a zero scale gives zero codes
                float qv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = fminf(fmaxf(v[e], -lim), lim);
                    qv[e] = fast ? div_by_rcp<kFp8>(t, sc, rsc) : div_rn(t, sc);
                }
                clo = pack_codes4<kFp8>(qv[0], qv[1], qv[2], qv[3]);
                chi = pack_codes4<kFp8>(qv[4], qv[5], qv[6], qv[7]);
            }
            *reinterpret_cast<uint2*>(q + c * 8) = make_uint2(clo, chi);
        }
    }
    if constexpr (kTrack) {
        __shared__ float part[4];
        m = wave_max(m);
        const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
        if (lane == 0) part[wave] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            const float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
            if (b > *amax_out) atomic_max_nonneg(amax_out, b);
        }
    }
}

template <bool kBf16, bool kFp8>
hipError_t quant_tensor_dispatch(const void* a, int64_t n, const float* amax_in, uint8_t* q, float* scale_out,
                                 float* amax_out, hipStream_t st) {
    const int64_t nchunk = n / 8;       // n == 0: one block, which only writes the scale
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((nchunk + 256 * 4 - 1) / (256 * 4), 4096));
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (amax_out)
        hipLaunchKernelGGL((quant_tensor_kernel<kBf16, kFp8, true>), grid, block, 0, st, a, nchunk, amax_in, q,
                           scale_out, amax_out);
    else
        hipLaunchKernelGGL((quant_tensor_kernel<kBf16, kFp8, false>), grid, block, 0, st, a, nchunk, amax_in, q,
                           scale_out, amax_out);
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

hipError_t launch_norm_quant_act(const void* h, bool bf16, int64_t M, int64_t K, const float* g, const float* b,
                                 bool layer, float eps, bool fp8, uint8_t* xq, float* x_scale, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (bf16) return fp8 ? norm_quant_dispatch<true, true>(h, g, b, layer, eps, M, K, xq, x_scale, st)
                         : norm_quant_dispatch<true, false>(h, g, b, layer, eps, M, K, xq, x_scale, st);
    return fp8 ? norm_quant_dispatch<false, true>(h, g, b, layer, eps, M, K, xq, x_scale, st)
               : norm_quant_dispatch<false, false>(h, g, b, layer, eps, M, K, xq, x_scale, st);
}

hipError_t launch_fold_norm_gain(const float* g, const float* s, int64_t K, float* out, hipStream_t st) {
    if (K <= 0) return hipSuccess;
    hipLaunchKernelGGL(fold_gain_kernel, dim3(static_cast<unsigned>((K + 255) / 256)), dim3(256), 0, st, g, s, K, out);
    return hipGetLastError();
}

hipError_t launch_quant_weight_t(const void* w, bool bf16, int64_t K, int64_t N, const float* s,
                                 const float* w_scale, bool tensor_scale, bool fp8, uint8_t* wq, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    const int64_t step = tensor_scale ? 0 : 1;
    if (bf16) return fp8 ? quant_weight_dispatch<true, true>(w, K, N, s, w_scale, step, wq, st)
                         : quant_weight_dispatch<true, false>(w, K, N, s, w_scale, step, wq, st);
    return fp8 ? quant_weight_dispatch<false, true>(w, K, N, s, w_scale, step, wq, st)
               : quant_weight_dispatch<false, false>(w, K, N, s, w_scale, step, wq, st);
}

hipError_t launch_quant_pair(const void* x, bool bf16, int64_t M, int64_t K, const float* s, bool fp8, uint8_t* xq,
                             float* x_scale, const void* w, int64_t N, const float* w_scale, uint8_t* wq,
                             hipStream_t st) {
    if (bf16) return fp8 ? quant_pair_dispatch<true, true>(x, M, K, s, xq, x_scale, w, N, w_scale, wq, st)
                         : quant_pair_dispatch<true, false>(x, M, K, s, xq, x_scale, w, N, w_scale, wq, st);
    return fp8 ? quant_pair_dispatch<false, true>(x, M, K, s, xq, x_scale, w, N, w_scale, wq, st)
               : quant_pair_dispatch<false, false>(x, M, K, s, xq, x_scale, w, N, w_scale, wq, st);
}

hipError_t launch_quant_tensor(const void* a, bool bf16, int64_t n, const float* amax_in, bool fp8, uint8_t* q,
                               float* scale_out, float* amax_out, hipStream_t st) {
    if (n < 0) return hipSuccess;
    if (bf16) return fp8 ? quant_tensor_dispatch<true, true>(a, n, amax_in, q, scale_out, amax_out, st)
                         : quant_tensor_dispatch<true, false>(a, n, amax_in, q, scale_out, amax_out, st);
    return fp8 ? quant_tensor_dispatch<false, true>(a, n, amax_in, q, scale_out, amax_out, st)
               : quant_tensor_dispatch<false, false>(a, n, amax_in, q, scale_out, amax_out, st);
}


}  // namespace w8a8
