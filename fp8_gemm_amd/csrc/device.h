// Device-side helpers shared by the libw8a8 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// ---- element loads: 8 consecutive elements of a float32 or bf16 row as float32 ---------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 elements as loaded, before conversion: one 16-byte load for bf16, two for float32.  Loading
// raw chunks first and converting later lets a wave keep many loads in flight with few registers.
template <bool kBf16>
struct Raw8 {
    uint4 u[kBf16 ? 1 : 2];
};

template <bool kBf16>
__device__ __forceinline__ Raw8<kBf16> load_raw8(const void* base, int64_t elem) {
    Raw8<kBf16> r;
    if constexpr (kBf16) {
        r.u[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    } else {
        const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
        r.u[0] = p[0];
        r.u[1] = p[1];
    }
    return r;
}

template <bool kBf16>
__device__ __forceinline__ void unpack8(const Raw8<kBf16>& r, float (&v)[8]) {
    if constexpr (kBf16) {
        const uint4 u = r.u[0];
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    } else {
        const uint4 a = r.u[0], b = r.u[1];
        v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
        v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
    }
}

template <bool kBf16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
    if constexpr (kBf16) {
        uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
        v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        float4 a = p[0], b = p[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// ---- streams over a whole tensor ----------------------------------------------------------------
// Block b of the grid takes the contiguous range [lo, hi) of n items, ceil(n / gridDim.x) each (the
// last blocks may get fewer or none).  A block's loads in flight then fall on a few neighbouring
// DRAM pages: in-bounds probes of 512 MB read at 6.1 TB/s this way, against 4.5-5.1 TB/s for a
// grid-stride walk at 1024-8192 blocks.
__device__ __forceinline__ int64_t block_range_lo(int64_t n) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    return min(static_cast<int64_t>(blockIdx.x) * per, n);
}
__device__ __forceinline__ int64_t block_range_hi(int64_t n) {
    const int64_t per = (n + gridDim.x - 1) / gridDim.x;
    return min(static_cast<int64_t>(blockIdx.x + 1) * per, n);
}

// ---- reductions ------------------------------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Maximum of non-negative floats: their bit patterns order like unsigned integers, so the
// result of concurrent updates is exact and independent of their order.
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
    atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// ---- quantization ------------------------------------------------------------------------------

// IEEE fp32 division, correctly rounded (not a reciprocal multiply).
__device__ __forceinline__ float div_rn(float a, float b) { return __fdiv_rn(a, b); }

// a / b correctly rounded from rb = div_rn(1, b), in five operations instead of a full division
// (Markstein, IBM J. Res. Dev. 34(1), 1990; Muller et al., "Handbook of Floating-Point
// Arithmetic", the theorem on FMA-based division).  q0 = a * rb is within 1.5 ulp of a / b; the
// first correction makes it faithful (within 1 ulp), and with a faithful quotient and the
// correctly rounded reciprocal the second correction returns the correctly rounded a / b.  The
// remainders are exact when nothing underflows: callers use this only where |b| and the quotients
// that can affect a result lie well inside the normal range, and fall back to div_rn elsewhere.
// The corrections turn a zero quotient into +0; kZeroSign restores the sign of a zero quotient
// from q0 (needed where the sign of zero reaches a result, as in E4M3 codes).  Host-callable so
// that the same arithmetic can be checked against IEEE division on the CPU.
template <bool kZeroSign = true>
__host__ __device__ __forceinline__ float div_by_rcp(float a, float b, float rb) {
    const float q0 = a * rb;
    const float r0 = __builtin_fmaf(-q0, b, a);
    const float q1 = __builtin_fmaf(r0, rb, q0);
    const float r1 = __builtin_fmaf(-q1, b, a);
    const float q = __builtin_fmaf(r1, rb, q1);
    return kZeroSign ? __builtin_copysignf(q, q0) : q;
}

// Divisors for which div_by_rcp is used: 2^lo <= |b| <= 2^hi.
template <int kLo, int kHi>
__host__ __device__ __forceinline__ bool in_pow2_range(float b) {
    const float m = fabsf(b);
    return m >= __builtin_ldexpf(1.0f, kLo) && m <= __builtin_ldexpf(1.0f, kHi);
}

// Symmetric INT8 code of v / scale: round half to even, clamp to [-127, 127].
__device__ __forceinline__ int int8_code(float q) {
    float r = __builtin_rintf(q);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
}

// Two OCP E4M3 ("fn": bias 7, largest 448, subnormals m * 2^-9) codes from the conversion
// instruction v_cvt_pk_fp8_f32, which on gfx950 rounds to the nearest E4M3 value with ties to
// even and keeps the sign of zero.  q0 goes to byte 2 kHi and q1 to byte 2 kHi + 1 of old, whose
// other two bytes are kept.  Inputs are clamped to +-448 first, so nothing overflows.  An in-bounds
// probe matched torch's float8_e4m3fn cast on every representable value, every midpoint between
// two of them, the neighbouring floats of both, subnormals and signed zeros.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3_pair(float q0, float q1, uint32_t old) {
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(q0, -448.0f), 448.0f),
                                                                 fminf(fmaxf(q1, -448.0f), 448.0f),
                                                                 static_cast<int>(old), kHi));
}

// Code of a quotient q = v / scale (already divided).
template <bool kFp8>
__device__ __forceinline__ uint32_t code_of_q(float q) {
    if constexpr (kFp8) {
        return e4m3_pair<false>(q, 0.0f, 0u) & 0xFFu;
    } else {
        return static_cast<uint32_t>(int8_code(q)) & 0xFFu;
    }
}

template <bool kFp8>
__device__ __forceinline__ uint32_t code_of(float xs, float scale) {
    return code_of_q<kFp8>(div_rn(xs, scale));
}

// Four codes of quotients packed into a word, q[0] in the low byte.
// INT8: q is clamped to [-127, 127] (clamping before rounding gives the same integer as rounding
// before clamping) and 1.5 * 2^23 is added: the sum's spacing is 1, so the addition rounds q to
// an integer with ties to even, and the low byte of the sum's bit pattern is that integer in two's
// complement.  Two byte permutes and an or gather the four low bytes.
template <bool kFp8>
__device__ __forceinline__ uint32_t pack_codes4(float q0, float q1, float q2, float q3) {
    if constexpr (kFp8) {
        return e4m3_pair<true>(q2, q3, e4m3_pair<false>(q0, q1, 0u));
    } else {
        auto rounded = [](float q) { return __float_as_uint(fminf(fmaxf(q, -127.0f), 127.0f) + 12582912.0f); };
        // v_perm_b32 selectors: 0-3 pick bytes of the second operand, 4-7 of the first, 0x0c gives 0.
        const uint32_t lo = __builtin_amdgcn_perm(rounded(q1), rounded(q0), 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(rounded(q3), rounded(q2), 0x04000c0cu);
        return lo | hi;
    }
}

template <bool kFp8>
__device__ __forceinline__ constexpr float qmax() { return kFp8 ? 448.0f : 127.0f; }

// Two finite floats rounded to bf16 (nearest, ties to even) and packed, a in the low half:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{a, b}), bf16x2));
}

// Store a block's bf16 output tiles t = t0, t0 + G, ... (rows m < M <= 16, 16 columns each) from
// LDS: ybuf[j] holds tile t0 + j G.  16-byte stores where the row allows them.
__device__ __forceinline__ void store_tiles_bf16(const uint16_t (*ybuf)[16][16], int ntiles_block, int t0, int G,
                                            int64_t M, int64_t N, uint16_t* __restrict__ y) {
    const int rows = static_cast<int>(M);
    const bool vec_ok = (N % 8) == 0;
    for (int i = threadIdx.x; i < ntiles_block * rows * 2; i += blockDim.x) {
        const int j = i / (rows * 2), m = (i / 2) % rows, h = i % 2;
        const int64_t n = (static_cast<int64_t>(t0) + static_cast<int64_t>(j) * G) * 16 + 8 * h;
        const uint4 v = *reinterpret_cast<const uint4*>(&ybuf[j][m][8 * h]);
        uint16_t* dst = y + m * N + n;
        if (vec_ok && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = static_cast<uint16_t>(w4[e / 2] >> (16 * (e % 2)));
        }
    }
}

}  // namespace w8a8
