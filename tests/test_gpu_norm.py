"""Parity of the fused RMS norm + per-token quantize (the smoothing folded into the norm's gain:
"Weight-Activation Quantization", s3 step 1 done offline; the W8A16-vs-W8A8 lesson, s2) with the
CPU oracle, through the C ABI.

Bar: the folded gain, the scales and the codes bit-exact (INT8 and E4M3), f32 and bf16 inputs,
row lengths for every register layout (one wave per row up to four), ragged rows and row counts,
rows with outliers and rows spanning 2^40 in magnitude, zero rows, and the prefill shape.
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


def folded_gain(f, K, seed):
    g = synth.random_scales(K, seed=seed, lo=0.5, hi=2.0)
    s = synth.random_scales(K, seed=seed + 1, lo=0.05, hi=20.0)
    gf = f.w8a8_fold_norm_gain(dev(g), dev(s))
    torch.cuda.synchronize()
    gf = host(gf)
    np.testing.assert_array_equal(gf, oracle.fold_norm_gain(g, s))
    return gf


# (M, K): one wave per row (K <= 512, 1024, 2048), two (<= 4096), four (<= 8192); ragged tails
SHAPES = [(1, 16), (5, 48), (33, 512), (70, 1040), (129, 2064), (64, 4096), (19, 6160), (40, 8192)]


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_norm_quant_act(f, qtype, M, K, dtype):
    announce(f"norm_quant_act {qtype} {dtype} {M}x{K}")
    H = synth.random_matrix((M, K), seed=M * 13 + K, dtype=dtype, outliers=max(1, K // 100))
    gf = folded_gain(f, K, seed=K)
    for g, eps in ((gf, 1e-5), (None, 1e-6)):
        xq, sx = f.w8a8_norm_quant_act(dev(H), None if g is None else dev(g), eps, qtype)
        torch.cuda.synchronize()
        q_ref, sx_ref = oracle.norm_quant_act(H, g, eps, qtype)
        np.testing.assert_array_equal(host(sx), sx_ref)
        np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_norm_quant_act_wide_range_and_zero_rows(f, qtype):
    """Rows whose squares span 2^80 (the double-double sum must match the oracle's), an all-zero row
    (scale 0, codes 0), and eps = 0."""
    announce(f"norm_quant_act wide range {qtype}")
    rng = np.random.Generator(np.random.PCG64(77))
    H = rng.standard_normal((48, 4096)).astype(np.float32)
    H *= np.exp2(rng.integers(-20, 20, H.shape)).astype(np.float32)
    H[5] = 0.0
    gf = folded_gain(f, 4096, seed=78)
    xq, sx = f.w8a8_norm_quant_act(dev(H), dev(gf), 1e-5, qtype)
    torch.cuda.synchronize()
    q_ref, sx_ref = oracle.norm_quant_act(H, gf, 1e-5, qtype)
    np.testing.assert_array_equal(host(sx), sx_ref)
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))
    assert sx_ref[5] == 0 and np.all(q_ref[5] == 0)
    Hn = np.delete(H, 5, axis=0)
    xq, sx = f.w8a8_norm_quant_act(dev(Hn), dev(gf), 0.0, qtype)
    torch.cuda.synchronize()
    q_ref, sx_ref = oracle.norm_quant_act(Hn, gf, 0.0, qtype)
    np.testing.assert_array_equal(host(sx), sx_ref)
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("K", [128, 1024, 2048, 4096, 8192])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_norm_quant_act_mean_square_tie(f, qtype, K, dtype):
    """Rows whose mean square sits on a float rounding tie, or just past it by squares that a plain
    double sum drops (the rows normalize differently, so a mean taken from such a sum fails), among
    random rows: in the first and last pass of a block, and alone or in pairs within one pass."""
    announce(f"norm_quant_act mean square tie {qtype} {dtype} K={K}")
    M = 37
    H = synth.random_matrix((M, K), seed=K + 5, outliers=max(1, K // 100))
    tie = synth.mean_square_tie_rows(K)
    for r0 in (0, 6, 17, 35):
        H[r0:r0 + 2] = tie
    if dtype == "bf16":
        H = synth.f32_to_bf16_bits(H)
    gf = folded_gain(f, K, seed=K + 6)
    for g, eps in ((None, 0.0), (gf, 0.0), (gf, 1e-5)):
        xq, sx = f.w8a8_norm_quant_act(dev(H), None if g is None else dev(g), eps, qtype)
        torch.cuda.synchronize()
        q_ref, sx_ref = oracle.norm_quant_act(H, g, eps, qtype)
        np.testing.assert_array_equal(host(sx), sx_ref)
        np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))
        if g is None:
            assert sx_ref[0] != sx_ref[1]


def test_norm_quant_act_prefill_shape(f):
    """The prefill workload's activations as the residual stream (2048 x 4096, bf16, outlier
    channels), the smoothing factors of that workload folded into a random gain."""
    announce("norm_quant_act prefill shape")
    X, W = synth.make_inputs("c2")
    x, w = dev(X), dev(W)
    _, _, s = f.w8a8_smooth_scales(x, w, 0.5)
    g = synth.random_scales(X.shape[1], seed=79, lo=0.5, hi=2.0)
    gf = f.w8a8_fold_norm_gain(dev(g), s)
    xq, sx = f.w8a8_norm_quant_act(x, gf, 1e-5, "int8")
    torch.cuda.synchronize()
    gf_h = host(gf)
    np.testing.assert_array_equal(gf_h, oracle.fold_norm_gain(g, host(s)))
    q_ref, sx_ref = oracle.norm_quant_act(X, gf_h, 1e-5, "int8")
    np.testing.assert_array_equal(host(sx), sx_ref)
    np.testing.assert_array_equal(host(xq), q_ref)


# ---- LayerNorm with the smoothing folded into gain and bias ----------------------------------

@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_norm_quant_act(f, qtype, M, K, dtype):
    """Rows with a nonzero mean (an offset of 3 on top of the outlier-channel draw)."""
    announce(f"layer_norm_quant_act {qtype} {dtype} {M}x{K}")
    H = synth.random_matrix((M, K), seed=M * 17 + K, outliers=max(1, K // 100)) + np.float32(3.0)
    if dtype == "bf16":
        H = synth.f32_to_bf16_bits(H)
    gf = folded_gain(f, K, seed=K + 1)
    b = synth.random_scales(K, seed=K + 2, lo=-1.0, hi=1.0)
    s = synth.random_scales(K, seed=K + 3, lo=0.05, hi=20.0)
    bf = f.w8a8_fold_norm_gain(dev(b), dev(s))
    torch.cuda.synchronize()
    bf = host(bf)
    np.testing.assert_array_equal(bf, oracle.fold_norm_gain(b, s))
    for g, bb, eps in ((gf, bf, 1e-5), (None, None, 1e-6), (gf, None, 0.0)):
        xq, sx = f.w8a8_layer_norm_quant_act(dev(H), None if g is None else dev(g), None if bb is None else dev(bb),
                                             eps, qtype)
        torch.cuda.synchronize()
        q_ref, sx_ref = oracle.layer_norm_quant_act(H, g, bb, eps, qtype)
        np.testing.assert_array_equal(host(sx), sx_ref)
        np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_layer_norm_wide_range_constant_and_zero_rows(f, qtype):
    """Rows spanning 2^40 (d = h - mu not exact in fp32), a constant row (d = 0: X~ = b), an
    all-zero row, and eps = 0 for the rows that allow it."""
    announce(f"layer_norm_quant_act wide range {qtype}")
    rng = np.random.Generator(np.random.PCG64(81))
    H = rng.standard_normal((48, 4096)).astype(np.float32)
    H *= np.exp2(rng.integers(-20, 20, H.shape)).astype(np.float32)
    H[5] = 0.0
    H[9] = np.float32(-2.75)
    g = synth.random_scales(4096, seed=82, lo=0.5, hi=2.0)
    b = synth.random_scales(4096, seed=83, lo=-1.0, hi=1.0)
    xq, sx = f.w8a8_layer_norm_quant_act(dev(H), dev(g), dev(b), 1e-5, qtype)
    torch.cuda.synchronize()
    q_ref, sx_ref = oracle.layer_norm_quant_act(H, g, b, 1e-5, qtype)
    np.testing.assert_array_equal(host(sx), sx_ref)
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))
    Hn = np.delete(H, [5, 9], axis=0)
    xq, sx = f.w8a8_layer_norm_quant_act(dev(Hn), dev(g), None, 0.0, qtype)
    torch.cuda.synchronize()
    q_ref, sx_ref = oracle.layer_norm_quant_act(Hn, g, None, 0.0, qtype)
    np.testing.assert_array_equal(host(sx), sx_ref)
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("K", [128, 1024, 2048, 4096, 8192])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layer_norm_mean_and_variance_ties(f, qtype, K, dtype):
    """Rows whose mean, or whose variance, sits on a float rounding tie or just past it by terms a
    plain double sum drops, among random rows in several passes of a block.  With the gain
    g[0] = 2^-20 the entries at the mean set the scale, so a mean taken from a plain sum changes
    the scales of the mean pairs; the variance pairs normalize differently at eps = 0."""
    announce(f"layer_norm mean/variance ties {qtype} {dtype} K={K}")
    M = 41
    H = synth.random_matrix((M, K), seed=K + 9, outliers=max(1, K // 100))
    for r0 in (0, 7, 22):
        H[r0:r0 + 2] = synth.mean_tie_rows(K)
    for r0 in (3, 17, 39):
        H[r0:r0 + 2] = synth.variance_tie_rows(K)
    if dtype == "bf16":
        H = synth.f32_to_bf16_bits(H)
    g = np.ones(K, np.float32)
    g[0] = 2.0 ** -20
    for gg, eps in ((g, 0.0), (None, 0.0), (g, 1e-5)):
        xq, sx = f.w8a8_layer_norm_quant_act(dev(H), None if gg is None else dev(gg), None, eps, qtype)
        torch.cuda.synchronize()
        q_ref, sx_ref = oracle.layer_norm_quant_act(H, gg, None, eps, qtype)
        np.testing.assert_array_equal(host(sx), sx_ref)
        np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))
        if gg is not None and eps == 0.0:
            assert sx_ref[0] != sx_ref[1]


def test_layer_norm_prefill_shape(f):
    """The prefill workload's activations read as the residual stream, gain and bias folded."""
    announce("layer_norm_quant_act prefill shape")
    X, W = synth.make_inputs("c2")
    x, w = dev(X), dev(W)
    _, _, s = f.w8a8_smooth_scales(x, w, 0.5)
    g = synth.random_scales(X.shape[1], seed=84, lo=0.5, hi=2.0)
    b = synth.random_scales(X.shape[1], seed=85, lo=-0.5, hi=0.5)
    gf, bf = f.w8a8_fold_norm_gain(dev(g), s), f.w8a8_fold_norm_gain(dev(b), s)
    xq, sx = f.w8a8_layer_norm_quant_act(x, gf, bf, 1e-5, "int8")
    torch.cuda.synchronize()
    q_ref, sx_ref = oracle.layer_norm_quant_act(X, host(gf), host(bf), 1e-5, "int8")
    np.testing.assert_array_equal(host(sx), sx_ref)
    np.testing.assert_array_equal(host(xq), q_ref)
