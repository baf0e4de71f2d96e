"""The path inside a HIP graph.  The whole layer (smoothing scales, weight folding and quantization,
activation quantization, GEMM with its epilogue; and the per-tensor E4M3 layer) is captured once and
replayed several times, with new inputs copied in, other eager work and synchronizations between
the replays, and the outputs overwritten before each replay.  Every replay must give the bytes
that the eager calls give on the same inputs (the kernels are deterministic), and the INT8 output
must match the oracle.  The library clears its buffers with a fill kernel, never a memset node."""
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
    return fp8_gemm_amd


def _inputs(M, K, N, seed):
    X = synth.random_matrix((M, K), seed=seed, dtype="bf16", outliers=max(1, K // 200))
    W = synth.random_matrix((K, N), seed=seed + 1, dtype="bf16", scale=0.02)
    return X, W


def _snapshot(r):
    return {k: host(v).copy() for k, v in r.items()}


@pytest.mark.parametrize("qtype,M,K,N,fused", [
    ("int8", 5, 4096, 1000, False),      # decode-shaped GEMM
    ("int8", 300, 512, 700, True),       # tiled GEMM, one-pass smooth + quantize
    ("fp8", 3, 8192, 520, False),
    ("fp8", 200, 1024, 264, True),
])
def test_layer_graph_replays(f, qtype, M, K, N, fused):
    announce(f"graph layer M={M} K={K} N={N} {qtype} fused={fused}")
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    inputs = [_inputs(M, K, N, seed) for seed in (101, 202, 303)]
    eager = []
    for X, W in inputs:
        x.copy_(dev(X))
        w.copy_(dev(W))
        eager.append(_snapshot(f.w8a8_layer(x, w, 0.5, qtype, fused=fused)))
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f.w8a8_layer(x, w, 0.5, qtype, fused=fused)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = f.w8a8_layer(x, w, 0.5, qtype, fused=fused)
    torch.cuda.synchronize()

    other = dev(inputs[0][0][: min(M, 4)])
    for rep, i in enumerate((1, 0, 2, 1)):
        X, W = inputs[i]
        x.copy_(dev(X))
        w.copy_(dev(W))
        for v in out.values():                       # stale bytes must not survive a replay
            v.view(torch.uint8).fill_(0x5A)
        f.w8a8_quant_act(other, None, qtype)         # eager work of the library between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(out)
        for k, ref in eager[i].items():
            np.testing.assert_array_equal(got[k].view(np.uint8), ref.view(np.uint8),
                                          err_msg=f"replay {rep} (inputs {i}): {k}")
    if qtype == "int8":
        X, W = inputs[1]
        s = eager[1]["s"]
        qw, sw = oracle.fold_quant_weight(W, s, qtype)
        qx, sx = oracle.quant_act(X, s, qtype)
        _, yb = oracle.dequant_i32(oracle.gemm_i32(qx, qw), sx, sw)
        np.testing.assert_array_equal(eager[1]["y"], yb)


def test_tensor_layer_graph_replays(f):
    """The per-tensor E4M3 layer (absmax fill + atomic maximum, then quantize and GEMM) in a graph."""
    M, K, N = 64, 1024, 520
    announce(f"graph tensor layer M={M} K={K} N={N}")
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    inputs = [_inputs(M, K, N, seed) for seed in (7, 8)]
    eager = []
    for X, W in inputs:
        x.copy_(dev(X))
        w.copy_(dev(W))
        eager.append(_snapshot(f.w8a8_layer_tensor(x, w, "fp8")))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f.w8a8_layer_tensor(x, w, "fp8")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = f.w8a8_layer_tensor(x, w, "fp8")
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 0, 1)):
        X, W = inputs[i]
        x.copy_(dev(X))
        w.copy_(dev(W))
        for v in out.values():
            v.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(out)
        for k, ref in eager[i].items():
            np.testing.assert_array_equal(got[k].view(np.uint8), ref.view(np.uint8),
                                          err_msg=f"replay {rep} (inputs {i}): {k}")
