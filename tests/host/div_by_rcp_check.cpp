// Host check of the five-operation division of the quantize kernels (w8a8::div_by_rcp in
// fp8_gemm_amd/csrc/device.h, the same source the kernels compile) against IEEE binary32
// division.  "Weight-Activation Quantization", section 3: each activation channel is divided by
// its smoothing factor; the quantized value is the smoothed value divided by its scale.  Both are
// fp32 divisions, and the kernels replace them by div_by_rcp where the divisor and the quotients
// that can reach a result lie inside guarded ranges.  This program checks that replacement bit for
// bit on those ranges:
//   - divisors |b| in [2^-20, 2^20] (smoothing factors) and [2^-60, 2^60] (row and column scales);
//   - dividends with |a| >= 2^-90 and quotients |a / b| in [2^-70, 2^100];
//   - random pairs (uniform exponent, uniform mantissa, random signs), and adversarial pairs whose
//     exact quotient lies within a few ulps of a rounding midpoint or of a representable value,
//     and powers of two, extreme mantissas and signed zeros.
// Usage: div_by_rcp_check <random pairs> <seed>.  Prints the counts; exit status 1 on a mismatch.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "device.h"

namespace {

uint64_t splitmix64(uint64_t& s) {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

float bits(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}
uint32_t ubits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

// A float with the given unbiased exponent and random mantissa and sign.
float make(uint64_t r, int e) {
    const uint32_t mant = static_cast<uint32_t>(r) & 0x7FFFFFu;
    const uint32_t sign = static_cast<uint32_t>(r >> 32) & 0x80000000u;
    return bits(sign | (static_cast<uint32_t>(e + 127) << 23) | mant);
}

bool in_domain(float a, float b, int blo, int bhi) {
    const double ab = fabs(static_cast<double>(b));
    if (ab < ldexp(1.0, blo) || ab > ldexp(1.0, bhi)) return false;
    if (a == 0.0f) return true;
    if (fabs(static_cast<double>(a)) < ldexp(1.0, -90)) return false;
    const double q = fabs(static_cast<double>(a) / static_cast<double>(b));
    return q >= ldexp(1.0, -70) && q <= ldexp(1.0, 100);
}

// 0 when div_by_rcp(a, b, 1/b) equals a / b bit for bit (both zero signs included).
int check(float a, float b) {
    const float rb = 1.0f / b;
    const float want = a / b;
    const float got = w8a8::div_by_rcp<true>(a, b, rb);
    if (ubits(want) == ubits(got)) return 0;
    static int shown = 0;
    if (shown++ < 10)
        fprintf(stderr, "mismatch a=%a b=%a want=%a got=%a\n", static_cast<double>(a), static_cast<double>(b),
                static_cast<double>(want), static_cast<double>(got));
    return 1;
}

}  // namespace

int main(int argc, char** argv) {
    const long long n = argc > 1 ? atoll(argv[1]) : 1000000;
    const uint64_t seed = argc > 2 ? strtoull(argv[2], nullptr, 10) : 1;
    const int ranges[2][2] = {{-20, 20}, {-60, 60}};
    long long tested = 0, bad = 0;

    // Random pairs, split over threads by index (each pair from its own counter).
#pragma omp parallel for reduction(+ : tested, bad) schedule(static)
    for (long long i = 0; i < n; ++i) {
        uint64_t s = seed * 0x100000000ull + static_cast<uint64_t>(i);
        const int* rg = ranges[i & 1];
        const uint64_t r1 = splitmix64(s), r2 = splitmix64(s), r3 = splitmix64(s);
        const int eb = rg[0] + static_cast<int>(r3 % static_cast<uint64_t>(rg[1] - rg[0]));
        const float b = make(r2, eb);
        const int lo = eb - 70 < -90 ? -90 : eb - 70, hi = eb + 100 > 127 ? 127 : eb + 100;
        const int ea = lo + static_cast<int>((r3 >> 32) % static_cast<uint64_t>(hi - lo));
        const float a = make(r1, ea);
        if (!in_domain(a, b, rg[0], rg[1])) continue;
        ++tested;
        bad += check(a, b);
    }

    // Adversarial pairs: a = b * q rounded, for q at or beside a midpoint of two floats or a float.
    long long adv = 0;
#pragma omp parallel for reduction(+ : adv, bad) schedule(static)
    for (long long i = 0; i < n / 8 + 1; ++i) {
        uint64_t s = (seed + 7) * 0x100000000ull + static_cast<uint64_t>(i);
        const int* rg = ranges[i & 1];
        const uint64_t r1 = splitmix64(s), r2 = splitmix64(s), r3 = splitmix64(s);
        const int eb = rg[0] + static_cast<int>(r3 % static_cast<uint64_t>(rg[1] - rg[0]));
        const float b = make(r2, eb);
        const float q = make(r1, -60 + static_cast<int>((r3 >> 32) % 150));
        const double half_ulp = ldexp(1.0, ilogb(q) - 24);
        const double mid = static_cast<double>(q) + (q < 0 ? -half_ulp : half_ulp);
        const double targets[3] = {mid, static_cast<double>(q), mid * (1.0 + ldexp(1.0, -40))};
        for (double t : targets) {
            const float a0 = static_cast<float>(t * static_cast<double>(b));
            for (int d = -2; d <= 2; ++d) {
                const float a = bits(ubits(a0) + static_cast<uint32_t>(d));
                if (!isfinite(a) || !in_domain(a, b, rg[0], rg[1])) continue;
                ++adv;
                bad += check(a, b);
            }
        }
    }

    // Powers of two, extreme mantissas and signed zeros.
    long long edge = 0;
    const uint32_t mants[4] = {0u, 1u, 0x400000u, 0x7FFFFFu};
    for (const auto& rg : ranges)
        for (int eb = rg[0]; eb <= rg[1]; ++eb)
            for (uint32_t mb : mants)
                for (int ea = -90; ea <= 127; ++ea)
                    for (uint32_t ma : mants)
                        for (int sg = 0; sg < 4; ++sg) {
                            const float b = bits((sg & 1 ? 0x80000000u : 0u) | (static_cast<uint32_t>(eb + 127) << 23) | mb);
                            const float a = bits((sg & 2 ? 0x80000000u : 0u) | (static_cast<uint32_t>(ea + 127) << 23) | ma);
                            if (in_domain(a, b, rg[0], rg[1])) { ++edge; bad += check(a, b); }
                            if (ea == -90 && ma == 0) {       // signed zeros
                                ++edge;
                                bad += check(sg & 2 ? -0.0f : 0.0f, b);
                            }
                        }
    printf("random %lld adversarial %lld edge %lld mismatches %lld\n", tested, adv, edge, bad);
    return bad ? 1 : 0;
}
