"""Parity of the per-tensor path ("Weight-Activation Quantization", s4 "Per-Tensor Scaling for
FP8"; s2's per-tensor INT8) with the CPU oracle, through the C ABI.

Bar: tensor maxima, scales and codes bit-exact (INT8 and E4M3), under current scaling (the
tensor's own maximum) and delayed scaling (an earlier maximum: values beyond Q * scale
saturate); INT8 GEMM output bit-exact against the oracle's fp32 dequantize; E4M3 GEMM output
within 1e-2 relative plus the matrix cores' accumulation bound (gpu_util.fp8_accumulation_bound).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import announce, assert_rel_tol, dev, fp8_accumulation_bound, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def native_library():
    import fp8_gemm_amd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fp8_gemm_amd.w8a8_version()                  # loads the library
    assert fp8_gemm_amd.lib_path() in open("/proc/self/maps").read(), "libw8a8.so is not loaded"
    yield fp8_gemm_amd


@pytest.fixture
def f(native_library):
    return native_library


def inputs(M, K, dtype, seed, outliers=2):
    X = synth.random_matrix((M, K), seed=seed, outliers=outliers)
    return synth.f32_to_bf16_bits(X) if dtype == "bf16" else X


def codes(a):
    return np.ascontiguousarray(a).view(np.uint8)


SHAPES = [(1, 16), (7, 48), (64, 512), (300, 4112), (1031, 2064)]


@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_absmax(f, M, K, dtype):
    announce(f"absmax {dtype} {M}x{K}")
    X = inputs(M, K, dtype, seed=M + K)
    a = f.w8a8_absmax(dev(X))
    torch.cuda.synchronize()
    assert host(a)[0] == oracle.absmax_tensor(X)
    # accumulate keeps a larger value and takes a larger one
    big = torch.tensor([1e6], dtype=torch.float32, device="cuda")
    f.w8a8_absmax(dev(X), amax=big, accumulate=True)
    small = torch.tensor([1e-6], dtype=torch.float32, device="cuda")
    f.w8a8_absmax(dev(X), amax=small, accumulate=True)
    torch.cuda.synchronize()
    assert host(big)[0] == np.float32(1e6)
    assert host(small)[0] == oracle.absmax_tensor(X)


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("M,K", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quant_act_tensor_current(f, qtype, M, K, dtype):
    """Current scaling: the scale from this X's own maximum."""
    announce(f"quant_act_tensor current {qtype} {dtype} {M}x{K}")
    X = inputs(M, K, dtype, seed=3 * M + K)
    x = dev(X)
    amax = f.w8a8_absmax(x)
    xq, sc, _ = f.w8a8_quant_act_tensor(x, amax, qtype)
    torch.cuda.synchronize()
    q_ref, sc_ref = oracle.quant_tensor(X, oracle.absmax_tensor(X), qtype)
    assert host(sc)[0] == sc_ref
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_tensor_path_full_grids(f, qtype):
    """A tensor of 4099 x 8192 bf16 (33.6 M elements): the maximum and the codes run on their full
    grids (1024 and 4096 blocks), each block streaming its own contiguous range of chunks over
    several loop passes, with a shorter last range.  Maximum, scale, codes and the maximum tracked
    in the same pass bit-exact."""
    announce(f"tensor path full grids {qtype}")
    X = inputs(4099, 8192, "bf16", seed=23, outliers=20)
    x = dev(X)
    amax = f.w8a8_absmax(x)
    xq, sc, amax_out = f.w8a8_quant_act_tensor(x, amax, qtype, track=True)
    torch.cuda.synchronize()
    a_ref = oracle.absmax_tensor(X)
    assert host(amax)[0] == a_ref
    assert host(amax_out)[0] == a_ref
    q_ref, sc_ref = oracle.quant_tensor(X, a_ref, qtype)
    assert host(sc)[0] == sc_ref
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("factor", [0.25, 3.0])
def test_quant_act_tensor_delayed(f, qtype, factor):
    """Delayed scaling: the scale from an earlier maximum (smaller: values saturate; larger: none
    do), and this X's maximum returned in the same pass."""
    announce(f"quant_act_tensor delayed {qtype} x{factor}")
    X = inputs(517, 1040, "bf16", seed=41)
    x = dev(X)
    prev = np.float32(oracle.absmax_tensor(X) * np.float32(factor))
    xq, sc, amax_out = f.w8a8_quant_act_tensor(x, dev(np.array([prev], np.float32)), qtype, track=True)
    torch.cuda.synchronize()
    q_ref, sc_ref = oracle.quant_tensor(X, prev, qtype)
    assert host(sc)[0] == sc_ref
    np.testing.assert_array_equal(codes(host(xq)), codes(q_ref))
    assert host(amax_out)[0] == oracle.absmax_tensor(X)
    # accumulate: a larger value already in amax_out stays
    keep = torch.tensor([1e9], dtype=torch.float32, device="cuda")
    f.w8a8_quant_act_tensor(x, dev(np.array([prev], np.float32)), qtype, amax_out=keep, accumulate=True)
    torch.cuda.synchronize()
    assert host(keep)[0] == np.float32(1e9)


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_quant_act_tensor_extremes(f, qtype):
    """Scales outside the fast-division range, ratios up to 2^60 beyond the top code, subnormal
    and signed-zero elements, and a zero maximum."""
    announce(f"quant_act_tensor extremes {qtype}")
    rng = np.random.Generator(np.random.PCG64(7))
    X = rng.standard_normal((96, 256)).astype(np.float32)
    X *= np.exp2(rng.integers(-40, 40, X.shape)).astype(np.float32)
    X[0, :6] = [0.0, -0.0, 1e-40, -1e-40, 3e38, -3e38]
    x = dev(X)
    for prev in (oracle.absmax_tensor(X), np.float32(1e-30), np.float32(2.0 ** -70), np.float32(1e37),
                 np.float32(0.5), np.float32(0.0)):
        xq, sc, _ = f.w8a8_quant_act_tensor(x, dev(np.array([prev], np.float32)), qtype)
        torch.cuda.synchronize()
        q_ref, sc_ref = oracle.quant_tensor(X, prev, qtype)
        assert host(sc)[0] == sc_ref, prev
        np.testing.assert_array_equal(codes(host(xq)), codes(q_ref), err_msg=f"amax_in={prev!r}")


def test_quant_act_tensor_empty_writes_scale(f):
    amax = dev(np.array([448.0], np.float32))
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    _, sc, _ = f.w8a8_quant_act_tensor(x, amax, "fp8")
    torch.cuda.synchronize()
    assert host(sc)[0] == np.float32(1.0)


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("K,N,dtype", [(16, 8, "f32"), (64, 35, "bf16"), (528, 1000, "bf16"), (4096, 1027, "f32")])
def test_quant_weight_tensor(f, qtype, K, N, dtype):
    announce(f"quant_weight_tensor {qtype} {dtype} {K}x{N}")
    W = synth.random_matrix((K, N), seed=K + N, scale=0.02)
    W[K // 3, N // 2] = 0.75
    if dtype == "bf16":
        W = synth.f32_to_bf16_bits(W)
    wq, sc = f.w8a8_quant_weight_tensor(dev(W), qtype)
    torch.cuda.synchronize()
    q_ref, sc_ref = oracle.quant_weight_tensor(W, qtype)
    assert host(sc)[0] == sc_ref
    np.testing.assert_array_equal(codes(host(wq)), codes(q_ref))


# (M, N, K): decode kernel, small-M kernel, 256 x 128 tiles with ragged edges, 256 x 256 tiles
GEMM_SHAPES = [(5, 3000, 4096), (40, 600, 1024), (300, 520, 2064), (4100, 8200, 256)]


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_dequant_tensor(f, qtype, M, N, K):
    announce(f"gemm_dequant_tensor {qtype} {M}x{N}x{K}")
    if qtype == "fp8" and K == 4096 and M <= 16:
        K = 8192                                    # the E4M3 decode shape
    xq_h = synth.random_codes((M, K), seed=M, qtype=qtype)
    wq_h = synth.random_codes((N, K), seed=N, qtype=qtype)
    sx, sw = np.float32(3.1e-3), np.float32(7.3e-4)
    y = f.w8a8_gemm_dequant_tensor(dev(xq_h), dev(np.array([sx])), dev(wq_h), dev(np.array([sw])), qtype)
    torch.cuda.synchronize()
    y = host(y)
    rows = np.arange(M) if M <= 64 else np.unique(np.r_[0, M - 1, np.random.default_rng(1).integers(0, M, 48)])
    sxv, swv = np.full(len(rows), sx, np.float32), np.full(N, sw, np.float32)
    if qtype == "int8":
        acc = oracle.gemm_i32(xq_h[rows], wq_h)
        _, yb = oracle.dequant_i32(acc, sxv, swv)
        np.testing.assert_array_equal(y[rows], yb)
    else:
        y64, mag = oracle.gemm_fp8(xq_h[rows], wq_h, sxv, swv)
        assert_rel_tol(y[rows], y64, 1e-2, extra=fp8_accumulation_bound(K, mag))


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_layer_tensor_two_steps(f, qtype):
    """The per-tensor path over two steps: step 1 with current scaling, step 2 with delayed
    scaling from step 1's maximum (two different X of the prefill shape's width)."""
    announce(f"layer_tensor two steps {qtype}")
    X1, W = synth.make_inputs("c1", seed=0, M=200)
    X2, _ = synth.make_inputs("c1", seed=1, M=200)
    w = dev(W)
    g1 = f.w8a8_layer_tensor(dev(X1), w, qtype)
    g2 = f.w8a8_layer_tensor(dev(X2), w, qtype, amax_prev=g1["amax"])
    torch.cuda.synchronize()
    r1 = oracle.layer_tensor(X1, W, qtype)
    r2 = oracle.layer_tensor(X2, W, qtype, amax_x=r1["amax_x"])
    for g, r in ((g1, r1), (g2, r2)):
        assert host(g["w_scale"])[0] == r["sw"]
        np.testing.assert_array_equal(codes(host(g["wq"])), codes(r["qw"]))
        assert host(g["x_scale"])[0] == r["sx"]
        np.testing.assert_array_equal(codes(host(g["xq"])), codes(r["qx"]))
    assert host(g2["amax"])[0] == oracle.absmax_tensor(X2)
    for g, r in ((g1, r1), (g2, r2)):
        if qtype == "int8":
            np.testing.assert_array_equal(host(g["y"]), r["y_bf16"])
        else:
            assert_rel_tol(host(g["y"]), r["y64"], 1e-2, extra=fp8_accumulation_bound(W.shape[0], r["mag64"]))
