"""The layer from a plain C99 program (tests/c_caller/layer_from_c.c): no Python and no torch in the
caller, device memory from the HIP runtime, every call through include/w8a8.h.  Its outputs are
checked against the oracle like the binding's: maxima, smoothing factors, codes and scales bit-exact,
the bf16 output bit-exact against the oracle's dequantize (INT8) or within 1e-2 relative plus the
matrix cores' accumulation bound (E4M3); a K that is not a multiple of 16 is refused with
W8A8_ERR_UNSUPPORTED ("Weight-Activation Quantization", section 3, the whole layer; section 4, E4M3)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from gpu_util import announce, assert_rel_tol, fp8_accumulation_bound

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_caller", "layer_from_c")


@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_layer_from_c(tmp_path, qtype):
    assert os.path.exists(EXE), "the C caller is not built: run __graft_entry__.build()"
    M, K, N, alpha = 70, 1040, 136, 0.5
    announce(f"C caller {qtype} M={M} K={K} N={N}")
    X = synth.random_matrix((M, K), seed=81, dtype="f32", outliers=10)
    W = synth.random_matrix((K, N), seed=82, dtype="f32", scale=0.02)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as fh:
        fh.write(np.array([M, K, N], np.int64).tobytes())
        fh.write(np.array([alpha], np.float32).tobytes())
        fh.write(np.array([1 if qtype == "fp8" else 0], np.int32).tobytes())
        fh.write(np.ascontiguousarray(X, np.float32).tobytes())
        fh.write(np.ascontiguousarray(W, np.float32).tobytes())
    r = subprocess.run([EXE, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    buf = open(out, "rb").read()
    pos = 0

    def take(dtype, n):
        nonlocal pos
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a

    status = take(np.int32, 3)
    assert list(status) == [0, 0, 2]            # OK, OK, W8A8_ERR_UNSUPPORTED
    ax, aw, s = take(np.float32, K), take(np.float32, K), take(np.float32, K)
    wq, sw = take(np.uint8, N * K).reshape(N, K), take(np.float32, N)
    xq, sx = take(np.uint8, M * K).reshape(M, K), take(np.float32, M)
    y = take(np.uint16, M * N).reshape(M, N)
    assert pos == len(buf)
    ref = oracle.layer(X, W, alpha, qtype)
    np.testing.assert_array_equal(ax, ref["ax"])
    np.testing.assert_array_equal(aw, ref["aw"])
    np.testing.assert_array_equal(s, ref["s"])
    np.testing.assert_array_equal(wq, ref["qw"].view(np.uint8))
    np.testing.assert_array_equal(sw, ref["sw"])
    np.testing.assert_array_equal(xq, ref["qx"].view(np.uint8))
    np.testing.assert_array_equal(sx, ref["sx"])
    if qtype == "int8":
        np.testing.assert_array_equal(y, ref["y_bf16"])
    else:
        assert_rel_tol(y, ref["y64"], 1e-2, extra=fp8_accumulation_bound(K, ref["mag64"]))
