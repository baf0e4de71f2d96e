"""Parity of the one-call layer preparation, w8a8_smooth_quant (calibration maxima, smoothing
factors, weight fold + quantize, activation quantize: "Weight-Activation Quantization", s3 steps 1
and 2 and "Choosing the Smoothing Factor"), with the CPU oracle, through the C ABI.

Bar: ax, aw, s, weight codes and scales, activation codes and scales all bit-exact (INT8 and
E4M3, f32 and bf16 inputs).  Shapes cover every register layout of the activation rows (K up to
512, 1024, 2048, 4096, 8192), ragged M and N, an odd number of weight tiles (the second tile of the
last block is idle), zero channels (s = 1), several alpha, and the shapes that take the unfused
sequence (N % 8 != 0, K > 8192, X and W of different dtypes).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import announce, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def f():
    import fp8_gemm_amd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fp8_gemm_amd.w8a8_version()
    assert fp8_gemm_amd.lib_path() in open("/proc/self/maps").read(), "libw8a8.so is not loaded"
    return fp8_gemm_amd


def codes(a):
    return np.ascontiguousarray(a).view(np.uint8)


def inputs(M, K, N, xdt, wdt, seed):
    X = synth.random_matrix((M, K), seed=seed, outliers=max(1, K // 100))
    W = synth.random_matrix((K, N), seed=seed + 1, scale=0.02)
    X[:, K // 2] = 0.0                                  # ax = 0: s = 1
    W[K // 3, :] = 0.0                                  # aw = 0: s = 1
    if xdt == "bf16":
        X = synth.f32_to_bf16_bits(X)
    if wdt == "bf16":
        W = synth.f32_to_bf16_bits(W)
    return X, W


def check(f, X, W, alpha, qtype):
    r = f.w8a8_smooth_quant(dev(X), dev(W), alpha, qtype)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in r.items()}
    ax, aw, s = oracle.smooth_scales(X, W, alpha)
    np.testing.assert_array_equal(g["ax"], ax)
    np.testing.assert_array_equal(g["aw"], aw)
    np.testing.assert_array_equal(g["s"], s)
    qw, sw = oracle.fold_quant_weight(W, s, qtype)
    np.testing.assert_array_equal(g["w_scale"], sw)
    np.testing.assert_array_equal(codes(g["wq"]), codes(qw))
    qx, sx = oracle.quant_act(X, s, qtype)
    np.testing.assert_array_equal(g["x_scale"], sx)
    np.testing.assert_array_equal(codes(g["xq"]), codes(qx))


# (M, K, N): every activation register layout, ragged M and N, odd tile counts, a ragged last
# column block of the calibration (K % 512 != 0) at 2048 and 2049 rows, and more weight scales to
# zero than the calibration has threads (K = 64, N = 9000)
SHAPES = [(1, 16, 8), (5, 48, 72), (33, 512, 520), (70, 1040, 136), (129, 2064, 264), (64, 4096, 200),
          (19, 6160, 64), (40, 8192, 96), (3000, 256, 1032),
          (2048, 1040, 136), (2049, 528, 72), (127, 64, 9000)]


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_smooth_quant(f, qtype, M, K, N, dtype):
    announce(f"smooth_quant {qtype} {dtype} M={M} K={K} N={N}")
    X, W = inputs(M, K, N, dtype, dtype, seed=M + K + N)
    check(f, X, W, 0.5, qtype)


@pytest.mark.parametrize("alpha", [0.0, 0.3, 1.0])
def test_smooth_quant_alpha(f, alpha):
    """alpha is a float in the C ABI: the oracle gets the same float (0.3 as float32)."""
    announce(f"smooth_quant alpha={alpha}")
    X, W = inputs(77, 1024, 264, "bf16", "bf16", seed=5)
    check(f, X, W, float(np.float32(alpha)), "int8")


@pytest.mark.parametrize("M,K,N,xdt,wdt", [(37, 512, 77, "bf16", "bf16"), (9, 8208, 40, "bf16", "bf16"),
                                           (50, 1024, 128, "f32", "bf16")])
def test_smooth_quant_unfused_shapes(f, M, K, N, xdt, wdt):
    """N % 8 != 0, K > 8192 and mixed dtypes take the three separate calls: same results."""
    announce(f"smooth_quant unfused M={M} K={K} N={N} {xdt}/{wdt}")
    X, W = inputs(M, K, N, xdt, wdt, seed=M + N)
    check(f, X, W, 0.5, "int8")


def test_smooth_quant_prefill_shape(f):
    """The prefill workload (2048 x 4096 x 4096, bf16, outlier channels) at full size."""
    announce("smooth_quant prefill shape")
    X, W = synth.make_inputs("c2")
    check(f, X, W, 0.5, "int8")


def test_smooth_quant_repeated_calls(f):
    """ax and w_scale are rebuilt by every call (no maxima carried over from the previous one)."""
    announce("smooth_quant repeated calls")
    X1, W1 = inputs(64, 1024, 128, "bf16", "bf16", seed=11)
    X2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(X1) * np.float32(0.25))
    W2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(W1) * np.float32(0.5))
    out = f.w8a8_smooth_quant(dev(X1), dev(W1), 0.5, "int8")
    f.w8a8_smooth_quant(dev(X2), dev(W2), 0.5, "int8", out=out)
    torch.cuda.synchronize()
    ax, aw, s = oracle.smooth_scales(X2, W2, 0.5)
    np.testing.assert_array_equal(host(out["ax"]), ax)
    _, sw = oracle.fold_quant_weight(W2, s, "int8")
    np.testing.assert_array_equal(host(out["w_scale"]), sw)


@pytest.mark.parametrize("M,N", [(0, 64), (24, 0)])
def test_smooth_quant_empty(f, M, N):
    """No activation rows (ax = 0) or no weight columns (aw = 0): s = 1 everywhere, and the outputs
    that exist match the oracle."""
    announce(f"smooth_quant empty M={M} N={N}")
    K = 512
    X = synth.random_matrix((M, K), seed=3) if M else np.zeros((0, K), np.float32)
    W = synth.random_matrix((K, N), seed=4, scale=0.02) if N else np.zeros((K, 0), np.float32)
    X, W = synth.f32_to_bf16_bits(X), synth.f32_to_bf16_bits(W)
    r = f.w8a8_smooth_quant(dev(X), dev(W), 0.5, "int8")
    torch.cuda.synchronize()
    ax, aw, s = oracle.smooth_scales(X, W, 0.5)
    np.testing.assert_array_equal(host(r["ax"]), ax)
    np.testing.assert_array_equal(host(r["aw"]), aw)
    np.testing.assert_array_equal(host(r["s"]), s)
    assert np.all(s == 1.0)
    if N:
        qw, sw = oracle.fold_quant_weight(W, s, "int8")
        np.testing.assert_array_equal(host(r["w_scale"]), sw)
        np.testing.assert_array_equal(codes(host(r["wq"])), codes(qw))
    if M:
        qx, sx = oracle.quant_act(X, s, "int8")
        np.testing.assert_array_equal(host(r["x_scale"]), sx)
        np.testing.assert_array_equal(codes(host(r["xq"])), codes(qx))


@pytest.mark.parametrize("name", ["c1", "c3", "c4", "c5"])
def test_smooth_quant_large_workloads(f, name):
    """The tiny, MLP-up (INT8), decode and large FP8 workloads at full size (the prefill one has
    its own test), as the benchmark step runs them: maxima, s, weight codes and scales, activation
    codes and scales bit-exact."""
    wl = synth.workload(name)
    announce(f"smooth_quant {wl.name}")
    X, W = synth.make_inputs(wl, seed=0)
    check(f, X, W, wl.alpha, wl.qtype)


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("M,K,N,xdt,wdt", [(70, 1040, 136, "bf16", "bf16"), (129, 4096, 264, "f32", "f32"),
                                          (2048, 4096, 4096, "bf16", "bf16"), (16, 4096, 14336, "bf16", "bf16"),
                                          (33, 512, 100, "bf16", "bf16"),        # N % 8 != 0: two launches
                                          (40, 8208, 64, "bf16", "bf16"),        # K > 8192: two launches
                                          (24, 256, 48, "f32", "bf16")])         # mixed dtypes: two launches
def test_quant_pair(f, qtype, M, K, N, xdt, wdt):
    """w8a8_quant_pair given the oracle's s and weight scales: both operands' codes and the token
    scales bit-exact against the oracle, in one launch or two."""
    announce(f"quant_pair {qtype} M={M} K={K} N={N} {xdt}/{wdt}")
    X, W = inputs(M, K, N, xdt, wdt, 31)
    ax, aw, s = oracle.smooth_scales(X, W, 0.5)
    qw, sw = oracle.fold_quant_weight(W, s, qtype)
    qx, sx = oracle.quant_act(X, s, qtype)
    xq, x_scale, wq = f.w8a8_quant_pair(dev(X), dev(W), dev(s), dev(sw), qtype)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(x_scale), sx)
    np.testing.assert_array_equal(codes(host(xq)), codes(qx))
    np.testing.assert_array_equal(codes(host(wq)), codes(qw))


def test_quant_pair_empty_operand(f):
    """M = 0 writes only the weight codes; N = 0 only the activation codes."""
    X, W = inputs(20, 256, 64, "bf16", "bf16", 33)
    ax, aw, s = oracle.smooth_scales(X, W, 0.5)
    qw, sw = oracle.fold_quant_weight(W, s, "int8")
    qx, sx = oracle.quant_act(X, s, "int8")
    xq, x_scale, wq = f.w8a8_quant_pair(dev(X[:0]), dev(W), dev(s), dev(sw), "int8")
    np.testing.assert_array_equal(codes(host(wq)), codes(qw))
    xq, x_scale, wq = f.w8a8_quant_pair(dev(X), dev(W[:, :0]), dev(s), dev(sw[:0]), "int8")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes(host(xq)), codes(qx))
    np.testing.assert_array_equal(host(x_scale), sx)
