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

// Symmetric INT8 code of v / scale: round half to even, clamp to [-127, 127].
__device__ __forceinline__ int int8_code(float q) {
    float r = __builtin_rintf(q);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return static_cast<int>(r);
}

// OCP E4M3 ("fn") code of q, |q| <= 448 (callers clamp first), round to nearest even.
// Normal range (|q| >= 2^-6): keep 3 of the 23 fp32 mantissa bits with round-half-even on the
// bit pattern (a carry moves into the exponent, which is the correct result), then rebias the
// exponent from 127 to 7.  Below 2^-6 the E4M3 spacing is 2^-9, so the code is rint(|q| * 2^9)
// (0..8, where 8 is the smallest normal, 2^-6, whose code is also 8).
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    uint32_t u = __float_as_uint(q);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t mag;
    if (a >= 0x3C800000u) {
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        mag = r - (120u << 3);
    } else {
        mag = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
    }
    return sign | mag;
}

template <bool kFp8>
__device__ __forceinline__ uint32_t code_of(float xs, float scale) {
    if constexpr (kFp8) {
        float q = div_rn(xs, scale);
        q = fminf(fmaxf(q, -448.0f), 448.0f);
        return e4m3_code(q);
    } else {
        return static_cast<uint32_t>(int8_code(div_rn(xs, scale))) & 0xFFu;
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

}  // namespace w8a8
