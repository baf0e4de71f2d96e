"""Parity of the weight-only W8A16 GEMM ("Weight-Activation Quantization", s1; the W8A16-vs-W8A8
lesson, s1) with the CPU oracle, through the C ABI.

Bar:
  - integer-valued X (|x| <= 31, so every partial sum of the fp32 accumulation is an exact integer
    below 2^24): the output is bit-exact against bf16((float)(sum_k x q) * sw[n]), i.e. the oracle's
    integer GEMM and fp32 dequantize with an activation scale of 1;
  - real bf16 X: within 1e-2 relative of the oracle's double-precision value plus the worst-case
    accumulation error of the matrix cores (gpu_util.fp8_accumulation_bound, which also covers an
    fp32 accumulation of exact products).
Shapes cover the decode kernel (M <= 16, K = 4096), the small-M kernel (up to 128 rows on narrow
layers), and the tiled kernel with 64 x 64, 128 x 128 and 256 x 256 tiles (ragged M and N, fewer
rows than one tile, a K that ends in half a 32-wide step, a grid that does not divide into the 8
XCDs), 64 x 64 tiles with K split among 4 groups of waves (at most 256 tiles) and among 2 (at most
512), and 128 x 128 tiles with K split among 2 (160 to 256 tiles), whose partial sums meet in LDS.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import announce, assert_rel_tol, dev, fp8_accumulation_bound, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def f():
    import fp8_gemm_amd
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fp8_gemm_amd.w8a8_version()
    assert fp8_gemm_amd.lib_path() in open("/proc/self/maps").read(), "libw8a8.so is not loaded"
    return fp8_gemm_amd


# (M, K, N): decode kernel; general kernel with one row block, with four, several row blocks
SHAPES = [(1, 4096, 1000), (7, 4096, 4100), (16, 4096, 96), (5, 528, 77), (40, 1040, 300), (300, 4096, 130),
          (129, 2064, 517), (17, 48, 33), (100, 528, 8200), (1000, 1040, 1000), (2050, 272, 4100),
          (4096, 4096, 4096),
          (3000, 1040, 4200), (2600, 272, 5100),   # 256 x 256 tiles: ragged M, N and K, 220 blocks
          (64, 4096, 9000), (400, 1040, 4104),     # 64 x 64 tiles with K split 4 and 2 ways
          (1000, 1040, 3000), (300, 2064, 9000)]   # 128 x 128 tiles with K split 2 ways


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8a16_integer_inputs_exact(f, M, K, N):
    announce(f"w8a16 integer M={M} K={K} N={N}")
    rng = np.random.Generator(np.random.PCG64(M * 31 + N))
    Xi = rng.integers(-31, 32, (M, K)).astype(np.float32)
    q = synth.random_codes((N, K), seed=N + K)
    sw = synth.random_scales(N, seed=N)
    y = f.w8a8_gemm_w8a16(dev(synth.f32_to_bf16_bits(Xi)), dev(q), dev(sw))
    torch.cuda.synchronize()
    acc = oracle.gemm_i32(Xi.astype(np.int8), q)
    _, yb = oracle.dequant_i32(acc, np.ones(M, np.float32), sw)
    np.testing.assert_array_equal(host(y), yb)


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8a16_real_inputs(f, M, K, N):
    announce(f"w8a16 real M={M} K={K} N={N}")
    X = synth.random_matrix((M, K), seed=M + K, dtype="bf16", outliers=max(1, K // 100))
    W = synth.random_matrix((K, N), seed=K + N, dtype="bf16", scale=0.02)
    wq, sw = f.w8a8_fold_quant_weight(dev(W), None, "int8")      # weight-only: no smoothing
    y = f.w8a8_gemm_w8a16(dev(X), wq, sw)
    torch.cuda.synchronize()
    q_ref, sw_ref = oracle.fold_quant_weight(W, None, "int8")
    np.testing.assert_array_equal(host(wq), q_ref)
    np.testing.assert_array_equal(host(sw), sw_ref)
    y64, mag = oracle.gemm_w8a16(X, q_ref, sw_ref)
    assert_rel_tol(host(y), y64, 1e-2, extra=fp8_accumulation_bound(K, mag))
    fro = np.linalg.norm(synth.bf16_bits_to_f32(host(y)).astype(np.float64) - y64) / np.linalg.norm(y64)
    assert fro <= 1e-2


def test_w8a16_rejects_wrong_types(f):
    x = torch.zeros((4, 32), dtype=torch.float32, device="cuda")
    q = torch.zeros((8, 32), dtype=torch.int8, device="cuda")
    with pytest.raises(TypeError):
        f.w8a8_gemm_w8a16(x, q, torch.ones(8, device="cuda"))
