"""Parity of the HIP path with the CPU oracle on the five workloads (seeded synthetic inputs).

Bar: calibration maxima, smoothing factors (alpha = 0.5), codes, scales and int32 accumulators
bit-exact; bf16 output within 1e-2 relative of the oracle's exact dequantized value (INT8 also
bit-exact against the oracle's fp32 dequantize).  FP8: E4M3 codes and scales bit-exact; output
within 1e-2 relative plus the worst-case accumulation error of the matrix cores' E4M3 dot product
(gpu_util.fp8_accumulation_bound), and within 1e-2 relative in the Frobenius norm.
Every output of every workload is compared at full size; the oracle's GEMM runs over blocks of
rows so that its host memory stays bounded on the largest shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import announce, assert_rel_tol, bf16_to_f64, dev, fp8_accumulation_bound, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def native_library():
    import fp8_gemm_amd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fp8_gemm_amd.w8a8_version()                  # loads the library
    maps = open("/proc/self/maps").read()
    assert fp8_gemm_amd.lib_path() in maps, "libw8a8.so is not loaded"
    yield fp8_gemm_amd


def gpu_path(f, X, W, alpha, qtype):
    x, w = dev(X), dev(W)
    ax, aw, s = f.w8a8_smooth_scales(x, w, alpha)
    wq, sw = f.w8a8_fold_quant_weight(w, s, qtype)
    xq, sx = f.w8a8_quant_act(x, s, qtype)
    y = f.w8a8_gemm_dequant(xq, sx, wq, sw, qtype)
    out = dict(ax=ax, aw=aw, s=s, wq=wq, sw=sw, xq=xq, sx=sx, y=y)
    if qtype == "int8":
        out["acc"] = f.w8a8_gemm_i32(xq, wq)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}


def check_prep(g, X, W, alpha, qtype):
    ax, aw, s = oracle.smooth_scales(X, W, alpha)
    np.testing.assert_array_equal(g["ax"], ax)
    np.testing.assert_array_equal(g["aw"], aw)
    np.testing.assert_array_equal(g["s"], s)
    qw, sw = oracle.fold_quant_weight(W, s, qtype)
    np.testing.assert_array_equal(g["sw"], sw)
    np.testing.assert_array_equal(g["wq"].view(np.uint8), qw.view(np.uint8))
    qx, sx = oracle.quant_act(X, s, qtype)
    np.testing.assert_array_equal(g["sx"], sx)
    np.testing.assert_array_equal(g["xq"].view(np.uint8), qx.view(np.uint8))
    return qx, sx, qw, sw


ROW_BLOCK = 512     # rows of the oracle GEMM per block on the large workloads


def row_blocks(M):
    for r0 in range(0, M, ROW_BLOCK):
        yield r0, min(M, r0 + ROW_BLOCK)


@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c3"])
def test_int8_layer(native_library, name):
    wl = synth.workload(name)
    announce(f"int8 layer {wl.name} M={wl.M} K={wl.K} N={wl.N}")
    X, W = synth.make_inputs(wl, seed=0)
    g = gpu_path(native_library, X, W, wl.alpha, "int8")
    qx, sx, qw, sw = check_prep(g, X, W, wl.alpha, "int8")
    for r0, r1 in row_blocks(wl.M):
        acc = oracle.gemm_i32(qx[r0:r1], qw)
        np.testing.assert_array_equal(g["acc"][r0:r1], acc, err_msg=f"rows {r0}..{r1}")
        y64, yb = oracle.dequant_i32(acc, sx[r0:r1], sw)
        assert_rel_tol(g["y"][r0:r1], y64, 1e-2)
        np.testing.assert_array_equal(g["y"][r0:r1], yb, err_msg=f"rows {r0}..{r1}")


@pytest.mark.timeout(900)
def test_fp8_layer_large(native_library):
    wl = synth.workload("c5")
    announce(f"fp8 layer {wl.name} M={wl.M} K={wl.K} N={wl.N}")
    X, W = synth.make_inputs(wl, seed=0)
    g = gpu_path(native_library, X, W, wl.alpha, "fp8")
    qx, sx, qw, sw = check_prep(g, X, W, wl.alpha, "fp8")
    del X, W
    err2 = ref2 = 0.0
    for r0, r1 in row_blocks(wl.M):
        y64, mag = oracle.gemm_fp8(qx[r0:r1], qw, sx[r0:r1], sw)
        assert_rel_tol(g["y"][r0:r1], y64, 1e-2, extra=fp8_accumulation_bound(wl.K, mag))
        y = bf16_to_f64(g["y"][r0:r1])
        err2 += float(np.sum((y - y64) ** 2))
        ref2 += float(np.sum(y64 ** 2))
        announce(f"fp8 layer rows {r0}..{r1} of {wl.M} within bound")
    assert np.sqrt(err2 / ref2) <= 1e-2


def test_fp8_layer_small(native_library):
    """The FP8 variant on the tiny and prefill shapes (not only the large one), full outputs."""
    for name in ("c1", "c2"):
        wl = synth.workload(name)
        X, W = synth.make_inputs(wl, seed=1, M=min(wl.M, 512))
        g = gpu_path(native_library, X, W, wl.alpha, "fp8")
        qx, sx, qw, sw = check_prep(g, X, W, wl.alpha, "fp8")
        y64, mag = oracle.gemm_fp8(qx, qw, sx, sw)
        assert_rel_tol(g["y"], y64, 1e-2, extra=fp8_accumulation_bound(wl.K, mag))
