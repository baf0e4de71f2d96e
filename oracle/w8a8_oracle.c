/*
 * Plain CPU oracle for the W8A8 linear layer: SmoothQuant smoothing, symmetric per-token /
 * per-output-channel quantization (INT8, or OCP FP8 E4M3), the integer GEMM and the dequantize.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the GPU library: it is
 * loaded by the tests, by the package's smoke check and by the benchmark's CPU-baseline leg,
 * never by the library itself.  It shares no code, header or table with the HIP kernels.
 *
 * Sources (web pages; sections as titled on each page):
 *   [WAQ]  "Weight-Activation Quantization" (infra.bea.ai inference guide)
 *            s2 "The Problem: Activation Outliers"  - symmetric INT8, scale = absmax / 127
 *            s3 "SmoothQuant: The Smoothing Trick"  - Y = XW = (X S^-1)(S W); divide activation
 *                                                    channel j by s_j, multiply weight channel j
 *                                                    by s_j; two-step pipeline; s_j formula
 *            s4 "FP8 W8A8"                          - E4M3 for weights/activations, range +-448,
 *                                                    codes round x / scale to E4M3, scale = max|x| / 448
 *   [ACT]  "Define activation quantization..." (zenaique flashcard) - per-token / per-channel
 *            scaling of activations and weights.
 *
 * Readings where the pages leave a step open (each is listed with its reason in the design notes):
 *   - division is IEEE fp32 division, not a multiply by a reciprocal (the page divides the activation
 *     channels by their factors);
 *   - the rounding of quantize() is round-half-to-even; INT8 codes are clamped to [-127, 127];
 *   - X gets one scale per row (token), W~ one scale per output channel (column of W [K, N]);
 *   - "channel j" of s_j is the contraction index: column j of X, row j of W [K, N];
 *   - a zero maximum gives s_j = 1; a row/column with scale 0 (all zero, or a maximum whose
 *     quotient by 127 or 448 underflows) gets codes 0;
 *   - alpha = 0.5 is evaluated as sqrtf(ax) / sqrtf(aw) (two correctly rounded roots and one
 *     division); other alpha use pow in double, rounded once to float;
 *   - dequantize is y = ((float)acc * sx[m]) * sw[n], rounded to bf16 (nearest even); the
 *     reference value y64 = acc * sx * sw is also returned in double;
 *   - E4M3 is the OCP "fn" flavour: bias 7, largest finite 448, subnormals m * 2^-9, no
 *     infinities; values are clamped to [-448, 448] before rounding;
 *   - per-tensor scaling (s4) uses one scale max|x| / Q for a whole tensor, without smoothing;
 *     under delayed scaling the maximum is an earlier tensor's, and values beyond Q * s saturate;
 *   - W8A16 (weight-only) multiplies 16-bit X by q * sw; the per-channel scale factors out of the
 *     sum, and the reference is that sum in double (the dequantized weight is not rounded first);
 *   - with the smoothing folded offline into the layer before, that layer is an RMS norm
 *     (x * r) * g with r = 1 / sqrt(mean(x^2) + eps), the mean taken in double and rounded to
 *     float once, and 1/s folded into its gain g' = g / s; or a LayerNorm
 *     ((x - mu) * r) * g' + b' with mu and the variance about it each rounded to float once, and
 *     1/s folded into both gain and bias.
 *
 * Arithmetic: IEEE binary32/binary64, round-to-nearest-even, compiled without fast-math and
 * without FMA contraction.  Every loop is the definition written out; the only parallelism is an
 * optional OpenMP split over independent output rows, which does not change any result.
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_INT8 0
#define ORACLE_FP8_E4M3 1

/* Element i of an input stored as float32 or as bfloat16 bit patterns.  Widening bf16 to f32 is
 * exact: the 16 bits are the high half of the float32. */
static float load_elem(const void* p, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return ((const float*)p)[i];
    uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

int oracle_rounding_is_nearest(void) { return fegetround() == FE_TONEAREST; }

/* Threads the OpenMP loops below may use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------------------
 * Calibration maxima, [WAQ] s3 "Choosing the Smoothing Factor": max|X_j| over the tokens of
 * activation channel j, and max|W_j| over the outputs fed by weight channel j.
 * ------------------------------------------------------------------------------------------- */
void oracle_absmax_cols(const void* x, int dtype, int64_t M, int64_t K, float* ax) {
    for (int64_t j = 0; j < K; ++j) {
        float m = 0.0f;
        for (int64_t i = 0; i < M; ++i) {
            float a = fabsf(load_elem(x, dtype, i * K + j));
            if (a > m) m = a;
        }
        ax[j] = m;
    }
}

void oracle_absmax_rows(const void* w, int dtype, int64_t K, int64_t N, float* aw) {
    for (int64_t j = 0; j < K; ++j) {
        float m = 0.0f;
        for (int64_t n = 0; n < N; ++n) {
            float a = fabsf(load_elem(w, dtype, j * N + n));
            if (a > m) m = a;
        }
        aw[j] = m;
    }
}

/* s_j = max|X_j|^alpha / max|W_j|^(1 - alpha), [WAQ] s3. */
float oracle_smooth_factor(float ax, float aw, double alpha) {
    if (ax == 0.0f || aw == 0.0f) return 1.0f;
    if (alpha == 0.5) return sqrtf(ax) / sqrtf(aw);
    if (alpha == 1.0) return ax;
    if (alpha == 0.0) return 1.0f / aw;
    return (float)(pow((double)ax, alpha) / pow((double)aw, 1.0 - alpha));
}

void oracle_smooth_factors(const float* ax, const float* aw, int64_t K, double alpha, float* s) {
    for (int64_t j = 0; j < K; ++j) s[j] = oracle_smooth_factor(ax[j], aw[j], alpha);
}

/* X~[i, j] = X[i, j] / s_j: each activation channel j divided by s_j ([WAQ] s3).  s == NULL means s = 1. */
void oracle_smooth_act(const void* x, int dtype, int64_t M, int64_t K, const float* s, float* xs) {
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < K; ++j) {
            float v = load_elem(x, dtype, i * K + j);
            xs[i * K + j] = s ? v / s[j] : v;
        }
}

/* W~[j, n] = s_j W[j, n]: each weight channel (row j of W [K, N]) multiplied by s_j ([WAQ] s3). */
void oracle_smooth_weight(const void* w, int dtype, int64_t K, int64_t N, const float* s, float* ws) {
    for (int64_t j = 0; j < K; ++j)
        for (int64_t n = 0; n < N; ++n) {
            float v = load_elem(w, dtype, j * N + n);
            ws[j * N + n] = s ? s[j] * v : v;
        }
}

/* ---------------------------------------------------------------------------------------------
 * OCP FP8 E4M3 ([WAQ] s4: 3 mantissa bits, range +-448).  Code layout: sign, 4 exponent bits with
 * bias 7, 3 mantissa bits.  Exponent field 0 holds subnormals m * 2^-9; 0x7F / 0xFF are NaN and
 * there is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448 (code 0x7E).
 * ------------------------------------------------------------------------------------------- */
double oracle_e4m3_decode(uint8_t c) {
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round |v| <= 448 to the nearest E4M3 value, ties to the even mantissa, and return its code. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);              /* a = f * 2^e2 with f in [0.5, 1): a lies in [2^(e2-1), 2^e2) */
    int e = e2 - 1;
    if (e < -6) e = -6;         /* below the smallest normal 2^-6 the spacing stays 2^-9 */
    double quantum = ldexp(1.0, e - 3);         /* spacing of E4M3 values in this binade */
    double r = nearbyint(a / quantum) * quantum;  /* a / quantum is exact (power-of-two divisor) */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6))                     /* subnormal: r = m * 2^-9, m in 1..7 */
        return sign | (uint8_t)(r / ldexp(1.0, -9));
    int re2;
    double f = frexp(r, &re2);                  /* r = f * 2^re2, f in [0.5, 1) */
    int E = re2 - 1 + 7;                        /* biased exponent */
    int m = (int)((2.0 * f - 1.0) * 8.0);       /* exact: r has at most 4 significant bits */
    return sign | (uint8_t)((E << 3) | m);
}

/* ---------------------------------------------------------------------------------------------
 * Symmetric quantization of each row of a float32 matrix V [R, C] with one scale per row:
 *   INT8 ([WAQ] s2):  scale = max|v| / 127,  q = clamp(round_half_even(v / scale), -127, 127)
 *   E4M3 ([WAQ] s4):  scale = max|v| / 448,  q = e4m3(clamp(v / scale, -448, 448))
 * A row whose scale is zero (its maximum is zero, or so small that max / Q rounds to zero) gets
 * all-zero codes: v / scale is not defined there.  Codes are stored as bytes.
 * ------------------------------------------------------------------------------------------- */
void oracle_quantize_rows(const float* v, int64_t R, int64_t C, int qtype, uint8_t* q, float* scale) {
    const float qmax = (qtype == ORACLE_INT8) ? 127.0f : 448.0f;
    for (int64_t r = 0; r < R; ++r) {
        const float* row = v + r * C;
        float amax = 0.0f;
        for (int64_t c = 0; c < C; ++c)
            if (fabsf(row[c]) > amax) amax = fabsf(row[c]);
        float sc = amax / qmax;
        scale[r] = sc;
        for (int64_t c = 0; c < C; ++c) {
            uint8_t code;
            if (sc == 0.0f) {
                code = 0;
            } else if (qtype == ORACLE_INT8) {
                float t = nearbyintf(row[c] / sc);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                code = (uint8_t)(int8_t)t;
            } else {
                float t = row[c] / sc;
                if (t > 448.0f) t = 448.0f;
                if (t < -448.0f) t = -448.0f;
                code = oracle_e4m3_encode(t);
            }
            q[r * C + c] = code;
        }
    }
}

/* Activation path at inference ([WAQ] s3 step 2, per-token scales [ACT]):
 * X~ = X / s (per channel), then per-row quantization.  q: [M, K] codes, sx: [M]. */
int oracle_quant_act(const void* x, int dtype, int64_t M, int64_t K, const float* s, int qtype,
                     uint8_t* q, float* sx) {
    float* xs = (float*)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xs) return -1;
    oracle_smooth_act(x, dtype, M, K, s, xs);
    oracle_quantize_rows(xs, M, K, qtype, q, sx);
    free(xs);
    return 0;
}

/* Weight path ([WAQ] s3 step 1 then step 2, per-output-channel scales [ACT]):
 * W~ = s * W (per channel j), then one scale per output column n of W~ [K, N].
 * The codes are returned transposed, q: [N, K] (row n holds output channel n), sw: [N]. */
int oracle_fold_quant_weight(const void* w, int dtype, int64_t K, int64_t N, const float* s, int qtype,
                             uint8_t* q, float* sw) {
    float* ws = (float*)malloc(sizeof(float) * (size_t)(K * N > 0 ? K * N : 1));
    float* wt = (float*)malloc(sizeof(float) * (size_t)(K * N > 0 ? K * N : 1));
    if (!ws || !wt) { free(ws); free(wt); return -1; }
    oracle_smooth_weight(w, dtype, K, N, s, ws);
    for (int64_t j = 0; j < K; ++j)
        for (int64_t n = 0; n < N; ++n) wt[n * K + j] = ws[j * N + n];
    oracle_quantize_rows(wt, N, K, qtype, q, sw);
    free(ws);
    free(wt);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * INT8 GEMM ([WAQ] s3 step 2: the product of the two code matrices, then dequantized):
 *   acc[m, n] = sum_k qx[m, k] * qw[n, k], exact in integers.
 * With |codes| <= 127, |acc| <= K * 127^2, which fits int32 for K <= 133144; the sum is kept
 * in int64 and the function returns -1 if any result would not fit int32.
 * ------------------------------------------------------------------------------------------- */
int oracle_gemm_i32(const int8_t* qx, const int8_t* qw, int64_t M, int64_t N, int64_t K, int32_t* acc) {
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        const int8_t* a = qx + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* b = qw + n * K;
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k) t += (int64_t)a[k] * (int64_t)b[k];
            if (t > INT32_MAX || t < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)t;
        }
    }
    return bad ? -1 : 0;
}

/* Round a finite float to bfloat16, nearest with ties to even; returns the bit pattern. */
uint16_t oracle_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Dequantize ([WAQ] s3 step 2; per-token x per-channel scales factor out of the sum over k):
 *   y64[m, n] = acc * sx[m] * sw[n] in double (the reference value), and
 *   y_bf16    = bf16(((float)acc * sx[m]) * sw[n]) (the fp32 dequantize, then bf16). */
void oracle_dequant_i32(const int32_t* acc, const float* sx, const float* sw, int64_t M, int64_t N,
                        double* y64, uint16_t* y_bf16) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int32_t a = acc[m * N + n];
            if (y64) y64[m * N + n] = (double)a * (double)sx[m] * (double)sw[n];
            if (y_bf16) {
                float y = ((float)a * sx[m]) * sw[n];
                y_bf16[m * N + n] = oracle_bf16_rne(y);
            }
        }
}

/* ---------------------------------------------------------------------------------------------
 * FP8 GEMM + dequantize ([WAQ] s4: x^ = s * q).  Every finite E4M3 value is an integer multiple
 * of 2^-9 with |multiple| <= 448 * 2^9, so each product of two decoded codes is an integer
 * multiple of 2^-18 and a sum of K of them is held exactly in int64 (K <= 2^26).  The oracle
 * therefore computes the exact dot product, then:
 *   y64[m, n]  = dot * sx[m] * sw[n]                     (double; the reference value)
 *   mag64[m,n] = sum_k |dec(qx) dec(qw)| * sx[m] * sw[n]  (for a floating-point error bound)
 * ------------------------------------------------------------------------------------------- */
int oracle_gemm_fp8(const uint8_t* qx, const uint8_t* qw, int64_t M, int64_t N, int64_t K,
                    const float* sx, const float* sw, double* y64, double* mag64) {
    int64_t lut[256];
    for (int c = 0; c < 256; ++c) {
        double d = oracle_e4m3_decode((uint8_t)c);
        lut[c] = isnan(d) ? 0 : (int64_t)ldexp(d, 9);   /* decoded value in units of 2^-9 */
    }
    int bad = 0;
    for (int64_t i = 0; i < M * K; ++i) bad |= ((qx[i] & 0x7F) == 0x7F);
    for (int64_t i = 0; i < N * K; ++i) bad |= ((qw[i] & 0x7F) == 0x7F);
    if (bad || K > ((int64_t)1 << 26)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const uint8_t* a = qx + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t* b = qw + n * K;
            int64_t t = 0, u = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t p = lut[a[k]] * lut[b[k]];
                t += p;
                u += p < 0 ? -p : p;
            }
            double scale = (double)sx[m] * (double)sw[n];
            if (y64) y64[m * N + n] = ldexp((double)t, -18) * scale;
            if (mag64) mag64[m * N + n] = ldexp((double)u, -18) * scale;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Per-tensor scaling ([WAQ] s4 "Per-Tensor Scaling for FP8": codes of x / s in E4M3, x^ = s q with
 * s = max|x| / 448; [WAQ] s2 gives the same per-tensor recipe for INT8 with 127).  One scale
 * serves a whole tensor.  Under delayed scaling ([WAQ] s4, the FP8-vs-INT8 table: the scale comes
 * from the previous step's maximum) the maximum is an earlier tensor's, so values beyond Q * s
 * occur; x / s is clamped to [-Q, Q] before rounding, i.e. they saturate.
 * ------------------------------------------------------------------------------------------- */

/* max |a[i]| over n elements (float32 or bf16). */
float oracle_absmax_tensor(const void* a, int dtype, int64_t n) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        const float v = fabsf(load_elem(a, dtype, i));
        if (v > amax) amax = v;
    }
    return amax;
}

/* s = amax / Q (Q = 127 for INT8, 448 for E4M3), one IEEE fp32 division. */
float oracle_tensor_scale(float amax, int qtype) {
    return amax / ((qtype == ORACLE_INT8) ? 127.0f : 448.0f);
}

/* q[i] = code(clamp(a[i] / scale, -Q, Q)) for n elements; scale 0 gives codes 0 (a / 0 is not
 * defined).  INT8 rounds half to even; E4M3 as oracle_e4m3_encode. */
void oracle_quantize_tensor(const void* a, int dtype, int64_t n, float scale, int qtype, uint8_t* q) {
    for (int64_t i = 0; i < n; ++i) {
        const float v = load_elem(a, dtype, i);
        uint8_t code = 0;
        if (scale != 0.0f) {
            float t = v / scale;
            if (qtype == ORACLE_INT8) {
                t = nearbyintf(t);
                if (t > 127.0f) t = 127.0f;
                if (t < -127.0f) t = -127.0f;
                code = (uint8_t)(int8_t)t;
            } else {
                if (t > 448.0f) t = 448.0f;
                if (t < -448.0f) t = -448.0f;
                code = oracle_e4m3_encode(t);
            }
        }
        q[i] = code;
    }
}

/* Per-tensor weight quantization: s = max|W| / Q over all of W [K, N]; the codes of W / s are
 * returned transposed, q: [N, K] (row n holds output channel n). */
int oracle_quant_weight_tensor(const void* w, int dtype, int64_t K, int64_t N, int qtype, uint8_t* q,
                               float* scale) {
    uint8_t* t = (uint8_t*)malloc((size_t)(K * N > 0 ? K * N : 1));
    if (!t) return -1;
    const float sc = oracle_tensor_scale(oracle_absmax_tensor(w, dtype, K * N), qtype);
    oracle_quantize_tensor(w, dtype, K * N, sc, qtype, t);
    for (int64_t j = 0; j < K; ++j)
        for (int64_t n = 0; n < N; ++n) q[n * K + j] = t[j * N + n];
    *scale = sc;
    free(t);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * Weight-only W8A16 GEMM, the contrast the pages draw with W8A8 ([WAQ] s1 "Why Quantize
 * Activations Too?": weight-only quantization keeps the GEMM in 16-bit with one low-precision
 * operand; the W8A16-vs-W8A8 lesson, s1: the 8-bit weights are dequantized to 16-bit on the fly
 * and the multiply runs on 16-bit tensor cores).  The weights are per-output-channel INT8 codes
 * q [N, K] with scales sw [N] (the weight quantize of s2 without smoothing); X stays 16-bit.  The
 * dequantized weight q[n, k] * sw[n] has one scale per output channel, which factors out of the
 * sum over k:
 *   y64[m, n]   = sw[n] * sum_k x[m, k] * q[n, k]      (double; every product is exact)
 *   mag64[m, n] = sw[n] * sum_k |x[m, k] * q[n, k]|    (for a floating-point error bound)
 * ------------------------------------------------------------------------------------------- */
int oracle_gemm_w8a16(const void* x, int dtype, const int8_t* q, const float* sw, int64_t M, int64_t N, int64_t K,
                      double* y64, double* mag64) {
    double* xd = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xd) return -1;
    for (int64_t i = 0; i < M * K; ++i) xd[i] = (double)load_elem(x, dtype, i);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        const double* a = xd + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const int8_t* b = q + n * K;
            double t = 0.0, u = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = a[k] * (double)b[k];
                t += p;
                u += fabs(p);
            }
            if (y64) y64[m * N + n] = t * (double)sw[n];
            if (mag64) mag64[m * N + n] = u * (double)sw[n];
        }
    }
    free(xd);
    return 0;
}

/* ---------------------------------------------------------------------------------------------
 * The activation step with the smoothing folded into the layer before it ([WAQ] s3 step 1: the
 * SmoothQuant transform is done offline, during model preparation; the W8A16-vs-W8A8 lesson, s2:
 * the whole process happens offline, with no runtime overhead).  X is the output of an RMS norm
 * of the residual stream h (the norm of the Llama models the pages name), and 1/s is folded into
 * the norm's gain once, offline:
 *   g'[j] = g[j] / s[j]                                     (fp32 division)
 * then per row of h [M, K]:
 *   ms    = (float)((sum_j (double)h[j] * h[j]) / K)        (the sum carried in double-double)
 *   r     = 1 / sqrtf(ms + eps)                             (fp32 add, correctly rounded root, division)
 *   X~[j] = (h[j] * r) * g'[j]                              (fp32, two roundings, in this order)
 * and X~ is quantized per row as in oracle_quantize_rows.  g == NULL: g = 1.
 * The sum of squares (each square of a float is exact in double) is carried as an unevaluated
 * pair hi + lo with error-free additions (Knuth's TwoSum), so it is within about 2^-100 of the
 * exact sum whatever the order of the terms; rounded to double and divided by K, it gives a mean
 * that any summation order reproduces after the rounding to float.
 * ------------------------------------------------------------------------------------------- */
/* (hi, lo) + x for |lo| <= ulp(hi) / 2: TwoSum, then renormalization. */
static void dd_add(double* hi, double* lo, double x) {
    const double s = *hi + x;
    const double bb = s - *hi;
    const double e = (*hi - (s - bb)) + (x - bb) + *lo;
    *hi = s + e;
    *lo = e - (*hi - s);
}

void oracle_fold_norm_gain(const float* g, const float* s, int64_t K, float* gout) {
    for (int64_t j = 0; j < K; ++j) gout[j] = (g ? g[j] : 1.0f) / (s ? s[j] : 1.0f);
}

void oracle_rms_norm(const void* h, int dtype, int64_t M, int64_t K, const float* g, float eps, float* out) {
    for (int64_t m = 0; m < M; ++m) {
        double hi = 0.0, lo = 0.0;
        for (int64_t j = 0; j < K; ++j) {
            const double v = (double)load_elem(h, dtype, m * K + j);
            dd_add(&hi, &lo, v * v);
        }
        const float ms = (float)((hi + lo) / (double)K);
        const float r = 1.0f / sqrtf(ms + eps);
        for (int64_t j = 0; j < K; ++j) {
            const float v = load_elem(h, dtype, m * K + j);
            out[m * K + j] = (v * r) * (g ? g[j] : 1.0f);
        }
    }
}

int oracle_norm_quant_act(const void* h, int dtype, int64_t M, int64_t K, const float* g, float eps, int qtype,
                          uint8_t* q, float* sx) {
    float* xs = (float*)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xs) return -1;
    oracle_rms_norm(h, dtype, M, K, g, eps, xs);
    oracle_quantize_rows(xs, M, K, qtype, q, sx);
    free(xs);
    return 0;
}

/* ---- LayerNorm with the smoothing folded into its gain and bias ----------------------------
 * The same offline fold when the norm before the layer is a LayerNorm: both its gain and its bias
 * scale the output, so both are divided by s (b'[j] = b[j] / s[j], the division of
 * oracle_fold_norm_gain).  Per row of h [M, K]:
 *   mu    = (float)((sum_j (double)h[j]) / K)               (the sum carried in double-double)
 *   d[j]  = h[j] - mu                                       (fp32)
 *   var   = (float)((sum_j (double)d[j] * d[j]) / K)        (the sum carried in double-double)
 *   r     = 1 / sqrtf(var + eps)
 *   X~[j] = (d[j] * r) * g'[j] + b'[j]                      (fp32 multiply, multiply, add, in this
 *                                                            order; no fused multiply-add)
 * g == NULL: g = 1; b == NULL: b = 0.  The variance is taken about the rounded mean (two passes),
 * not as mean(h^2) - mu^2.
 * ------------------------------------------------------------------------------------------- */
void oracle_layer_norm(const void* h, int dtype, int64_t M, int64_t K, const float* g, const float* b, float eps,
                       float* out) {
    for (int64_t m = 0; m < M; ++m) {
        double hi = 0.0, lo = 0.0;
        for (int64_t j = 0; j < K; ++j) dd_add(&hi, &lo, (double)load_elem(h, dtype, m * K + j));
        const float mu = (float)((hi + lo) / (double)K);
        hi = 0.0;
        lo = 0.0;
        for (int64_t j = 0; j < K; ++j) {
            const float d = load_elem(h, dtype, m * K + j) - mu;
            dd_add(&hi, &lo, (double)d * (double)d);
        }
        const float var = (float)((hi + lo) / (double)K);
        const float r = 1.0f / sqrtf(var + eps);
        for (int64_t j = 0; j < K; ++j) {
            const float d = load_elem(h, dtype, m * K + j) - mu;
            const float t = (d * r) * (g ? g[j] : 1.0f);
            out[m * K + j] = t + (b ? b[j] : 0.0f);
        }
    }
}

int oracle_layer_norm_quant_act(const void* h, int dtype, int64_t M, int64_t K, const float* g, const float* b,
                                float eps, int qtype, uint8_t* q, float* sx) {
    float* xs = (float*)malloc(sizeof(float) * (size_t)(M * K > 0 ? M * K : 1));
    if (!xs) return -1;
    oracle_layer_norm(h, dtype, M, K, g, b, eps, xs);
    oracle_quantize_rows(xs, M, K, qtype, q, sx);
    free(xs);
    return 0;
}
