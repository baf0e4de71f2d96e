/*
 * A plain C99 caller of libw8a8 (no Python, no torch): the whole layer through the C ABI, as an
 * inference engine written in C would run it ("Weight-Activation Quantization", section 3: the
 * smoothing factors, the fold and quantization of the weights, the quantization of the activations,
 * and the dequantized 8-bit product).  Device memory comes from the HIP runtime directly.
 *
 * usage: layer_from_c <in> <out>
 *   in:  int64 M, K, N; float32 alpha; int32 qtype (0 INT8, 1 E4M3); X float32 [M, K]; W float32 [K, N]
 *   out: int32 status of each call (smooth_quant, gemm_dequant, a quant_act with K = 17); then
 *        ax, aw, s float32 [K]; wq [N, K] bytes; w_scale float32 [N]; xq [M, K] bytes;
 *        x_scale float32 [M]; y bf16 bits [M, N]
 * Exit status 0 when every HIP call succeeded (the library's statuses are written for the test).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "w8a8.h"

#define HIP_OK(call)                                                            \
    do {                                                                        \
        hipError_t e_ = (call);                                                 \
        if (e_ != hipSuccess) {                                                 \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));   \
            return 2;                                                           \
        }                                                                       \
    } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n; }
static int write_all(FILE* f, const void* p, size_t n) { return fwrite(p, 1, n, f) == n; }

int main(int argc, char** argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <in> <out>\n", argv[0]);
        return 1;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int64_t dims[3];
    float alpha;
    int32_t qtype;
    if (!read_all(in, dims, sizeof dims) || !read_all(in, &alpha, 4) || !read_all(in, &qtype, 4)) return 1;
    const int64_t M = dims[0], K = dims[1], N = dims[2];
    const size_t xb = (size_t)(M * K) * 4, wb = (size_t)(K * N) * 4;
    float* hx = (float*)malloc(xb);
    float* hw = (float*)malloc(wb);
    if (!hx || !hw || !read_all(in, hx, xb) || !read_all(in, hw, wb)) return 1;
    fclose(in);

    void *x, *w, *ax, *aw, *s, *wq, *sw, *xq, *sx, *y;
    HIP_OK(hipMalloc(&x, xb));
    HIP_OK(hipMalloc(&w, wb));
    HIP_OK(hipMalloc(&ax, (size_t)K * 4));
    HIP_OK(hipMalloc(&aw, (size_t)K * 4));
    HIP_OK(hipMalloc(&s, (size_t)K * 4));
    HIP_OK(hipMalloc(&wq, (size_t)(N * K)));
    HIP_OK(hipMalloc(&sw, (size_t)N * 4));
    HIP_OK(hipMalloc(&xq, (size_t)(M * K)));
    HIP_OK(hipMalloc(&sx, (size_t)M * 4));
    HIP_OK(hipMalloc(&y, (size_t)(M * N) * 2));
    HIP_OK(hipMemcpy(x, hx, xb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(w, hw, wb, hipMemcpyHostToDevice));
    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));

    const w8a8_qtype q = qtype ? W8A8_FP8_E4M3 : W8A8_INT8;
    int32_t status[3];
    status[0] = w8a8_smooth_quant(x, W8A8_F32, M, K, w, W8A8_F32, N, alpha, q, (float*)ax, (float*)aw,
                                  (float*)s, wq, (float*)sw, xq, (float*)sx, st);
    status[1] = w8a8_gemm_dequant(xq, (const float*)sx, wq, (const float*)sw, q, M, N, K, y, st);
    /* K = 17 is not a multiple of 16: refused on the host, nothing queued. */
    status[2] = w8a8_quant_act(x, W8A8_F32, 1, 17, NULL, q, xq, (float*)sx, st);
    HIP_OK(hipStreamSynchronize(st));
    fprintf(stderr, "statuses: %s, %s, %s\n", w8a8_status_string((w8a8_status)status[0]),
            w8a8_status_string((w8a8_status)status[1]), w8a8_status_string((w8a8_status)status[2]));

    FILE* out = fopen(argv[2], "wb");
    if (!out || !write_all(out, status, sizeof status)) return 1;
    struct { void* d; size_t n; } parts[] = {
        {ax, (size_t)K * 4}, {aw, (size_t)K * 4}, {s, (size_t)K * 4}, {wq, (size_t)(N * K)},
        {sw, (size_t)N * 4}, {xq, (size_t)(M * K)}, {sx, (size_t)M * 4}, {y, (size_t)(M * N) * 2}};
    for (size_t i = 0; i < sizeof parts / sizeof parts[0]; ++i) {
        void* h = malloc(parts[i].n);
        if (!h) return 1;
        HIP_OK(hipMemcpy(h, parts[i].d, parts[i].n, hipMemcpyDeviceToHost));
        if (!write_all(out, h, parts[i].n)) return 1;
        free(h);
    }
    fclose(out);
    HIP_OK(hipStreamDestroy(st));
    void* bufs[] = {x, w, ax, aw, s, wq, sw, xq, sx, y};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
    free(hx);
    free(hw);
    return 0;
}
