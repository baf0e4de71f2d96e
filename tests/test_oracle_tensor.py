"""Pins of the oracle's per-tensor scaling ("Weight-Activation Quantization", s4 "Per-Tensor
Scaling for FP8", and the per-tensor INT8 example of s2), of its weight-only W8A16 GEMM (s1 and
the W8A16-vs-W8A8 lesson) and of its RMS norm with the smoothing folded into the gain (s3 step 1,
offline) against things other than themselves: the page's outlier row, library
routines with the same semantics (numpy float32 division and round-half-even, torch's
float8_e4m3fn cast, numpy float64 matmul), closed forms and invariants.

Each test names the kind of mistake it is there to catch.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32(a):
    return np.asarray(a, dtype=np.float32)


def int8_ref(v, scale):
    """numpy's float32 division, round-half-even and clip: the INT8 recipe of s2 with saturation."""
    t = (f32(v) / np.float32(scale)).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int8)


def e4m3_ref(v, scale):
    """torch's E4M3 cast of the fp32 quotient clamped to +-448 (the section 4 conversion of x / s)."""
    with np.errstate(over="ignore"):
        t = (f32(v) / np.float32(scale)).astype(np.float32)
    t = np.clip(t, -448, 448)
    return torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_absmax_tensor_matches_numpy():
    """Catches: a maximum over one axis only, a signed instead of absolute maximum, bf16 read as
    something else."""
    X = synth.random_matrix((37, 96), seed=3, outliers=2)
    assert oracle.absmax_tensor(X) == np.max(np.abs(X))
    Xb = synth.f32_to_bf16_bits(X)
    assert oracle.absmax_tensor(Xb) == np.max(np.abs(synth.bf16_bits_to_f32(Xb)))
    neg = -np.abs(X)
    assert oracle.absmax_tensor(neg) == np.max(np.abs(X))
    assert oracle.absmax_tensor(np.zeros((3, 16), np.float32)) == 0


def test_tensor_scale_closed_form():
    """s = amax / Q as one fp32 division; catches Q = 128 / 127 mixed up, or amax * Q."""
    for amax in (80.0, 1.0, 3.7e-3, 448.0 * 2.0 ** -7):
        assert oracle.tensor_scale(amax, "int8") == np.float32(amax) / np.float32(127)
        assert oracle.tensor_scale(amax, "fp8") == np.float32(amax) / np.float32(448)
    assert oracle.tensor_scale(448.0 * 2.0 ** -7, "fp8") == np.float32(2.0 ** -7)


def test_outlier_rows_per_tensor():
    """s2's example as a tensor: the outlier row sets the one scale (80 / 127, printed 0.63) for
    every row, and every small value of both rows maps to a code of at most 1 (all 0 under
    round-half-even).  Catches: per-row scales where one tensor scale is meant."""
    g = golden("outlier_row_per_tensor.json")
    row = f32(g["row"])
    small_row = f32([0.3, -0.2, 0.1, 0.25, -0.3, 0.15, 0.05, -0.1])
    X = np.stack([row, small_row])
    q, sc = oracle.quant_tensor(X, oracle.absmax_tensor(X), "int8")
    assert round(float(sc), g["scale_printed_decimals"]) == g["scale_printed"]
    assert sc == np.float32(80.0) / np.float32(127.0)
    small = [i for i in range(len(row)) if i not in g["outlier_positions"]]
    assert np.all(np.abs(q[0, small]) <= g["small_values_max_abs_code"])
    assert np.all(q[1] == 0)                        # the whole second row is destroyed
    # per-row scaling keeps the second row (the motivation for per-token scales)
    q_rows, _ = oracle.quantize_rows(X, "int8")
    assert np.max(np.abs(q_rows[1])) == 127


def test_int8_tensor_matches_numpy():
    """Catches: multiply by a reciprocal instead of dividing, round-half-away, a missing clamp."""
    X = synth.random_matrix((48, 160), seed=21, outliers=3)
    amax = oracle.absmax_tensor(X)
    q, sc = oracle.quant_tensor(X, amax, "int8")
    np.testing.assert_array_equal(q, int8_ref(X, sc))
    assert np.max(np.abs(q)) == 127


def test_fp8_tensor_matches_torch():
    """Catches: a wrong E4M3 flavour (FNUZ, 240), lost signs of zero, a scale off by a factor."""
    X = synth.random_matrix((40, 128), seed=22, outliers=2)
    X[0, :4] = [0.0, -0.0, 1e-30, -1e-30]
    amax = oracle.absmax_tensor(X)
    q, sc = oracle.quant_tensor(X, amax, "fp8")
    np.testing.assert_array_equal(q, e4m3_ref(X, sc))
    dec = np.vectorize(oracle.e4m3_decode)(q)
    assert np.max(np.abs(dec)) == 448.0
    # a power-of-two scale: codes are the E4M3 cast of x * 2^-k itself
    X2 = X / np.float32(amax) * np.float32(448.0 * 2.0 ** -5)
    q2, sc2 = oracle.quant_tensor(X2, oracle.absmax_tensor(X2), "fp8")
    assert sc2 == np.float32(2.0 ** -5)
    ref = torch.from_numpy((X2 * np.float32(32.0)).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(q2, ref.view(torch.uint8).numpy())


def test_dequantized_tensor_within_half_spacing():
    """x^ = s q (s4): every value decodes to within half an E4M3 spacing of x / s (relative 2^-4
    for normal codes, 2^-10 absolute in the subnormal range).  Catches: truncation instead of
    rounding, a scale applied twice."""
    X = synth.random_matrix((32, 128), seed=23, outliers=2)
    q, sc = oracle.quant_tensor(X, oracle.absmax_tensor(X), "fp8")
    dec = np.vectorize(oracle.e4m3_decode)(q).astype(np.float64)
    t = X.astype(np.float64) / float(sc)
    bound = np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(dec - t) <= bound * (1 + 1e-12))


def test_delayed_scaling_saturates():
    """Delayed scaling (s4 table): the scale comes from an earlier, smaller maximum, so values
    beyond Q s clamp to the top code and the rest round as usual.  Catches: wrap-around instead of
    saturation, the scale recomputed from the current tensor."""
    X = synth.random_matrix((24, 128), seed=24, outliers=2)
    amax = oracle.absmax_tensor(X)
    prev = np.float32(amax / 4)
    for qt, top in (("int8", 127), ("fp8", 448.0)):
        q, sc = oracle.quant_tensor(X, prev, qt)
        assert sc == oracle.tensor_scale(prev, qt)
        ref = int8_ref(X, sc) if qt == "int8" else e4m3_ref(X, sc)
        np.testing.assert_array_equal(q, ref)
        mag = np.abs(q.astype(np.float64)) if qt == "int8" else np.abs(np.vectorize(oracle.e4m3_decode)(q))
        over = np.abs(X.astype(np.float64)) / float(sc) > top
        assert over.any() and np.all(mag[over] == top)


def test_zero_tensor_and_zero_history():
    """A zero maximum gives scale 0 and all-zero codes (x / 0 is not defined), as for rows."""
    X = synth.random_matrix((4, 32), seed=25)
    for qt in ("int8", "fp8"):
        q, sc = oracle.quant_tensor(X, 0.0, qt)
        assert sc == 0 and np.all(q == 0)


def test_weight_tensor_orientation_and_scale():
    """W [K, N] -> codes [N, K] with one scale max|W| / Q.  Catches: codes not transposed, a
    per-column scale where one tensor scale is meant."""
    W = synth.random_matrix((64, 24), seed=26, scale=0.02)
    W[5, 7] = 0.5                                   # one large weight sets the tensor scale
    for qt in ("int8", "fp8"):
        q, sc = oracle.quant_weight_tensor(W, qt)
        assert q.shape == (24, 64)
        assert sc == oracle.tensor_scale(np.float32(0.5), qt)
        ref = int8_ref(W, sc) if qt == "int8" else e4m3_ref(W, sc)
        np.testing.assert_array_equal(q, ref.T)


def test_layer_tensor_int8_worse_than_smoothquant_on_outliers():
    """The pages' point (s2, s3): on activations with outlier channels, one INT8 scale per tensor
    loses more than per-token scales with smoothing.  Direction only, on the tiny workload."""
    X, W = synth.make_inputs("c1")
    ref = X.astype(np.float64) @ W.astype(np.float64)
    e_t = np.linalg.norm(oracle.layer_tensor(X, W, "int8")["y64"] - ref) / np.linalg.norm(ref)
    e_s = np.linalg.norm(oracle.layer(X, W, 0.5, "int8")["y64"] - ref) / np.linalg.norm(ref)
    assert e_s < e_t


def test_layer_tensor_fp8_dequant_closed_form():
    """Per-tensor FP8 through the GEMM: y64 = (exact sum of decoded products) s_x s_w.  Checked by
    brute force on a small case.  Catches: a scale left out, the wrong operand transposed."""
    X = synth.random_matrix((6, 32), seed=27, outliers=1)
    W = synth.random_matrix((32, 5), seed=28, scale=0.05)
    out = oracle.layer_tensor(X, W, "fp8")
    dx = np.vectorize(oracle.e4m3_decode)(out["qx"]).astype(np.float64)
    dw = np.vectorize(oracle.e4m3_decode)(out["qw"]).astype(np.float64)
    brute = (dx @ dw.T) * float(out["sx"]) * float(out["sw"])
    np.testing.assert_allclose(out["y64"], brute, rtol=1e-15, atol=0)


# ---------------------------------------------------------------------------------------------
# Weight-only W8A16 (Weight-Activation Quantization, s1; the W8A16-vs-W8A8 lesson, s1)
# ---------------------------------------------------------------------------------------------

def test_w8a16_matches_numpy_dequantized_matmul():
    """y = X (q sw)^T with the dequantized weights, numpy float64 matmul.  Catches: the scale on the
    wrong axis, codes transposed, bf16 X read as something else."""
    X = synth.f32_to_bf16_bits(synth.random_matrix((9, 200), seed=31, outliers=2))
    W = synth.random_matrix((200, 13), seed=32, scale=0.02)
    q, sw = oracle.fold_quant_weight(W, None, "int8")
    y64, mag = oracle.gemm_w8a16(X, q, sw)
    Wd = q.astype(np.float64) * sw.astype(np.float64)[:, None]           # [N, K] dequantized
    ref = synth.bf16_bits_to_f32(X).astype(np.float64) @ Wd.T
    np.testing.assert_allclose(y64, ref, rtol=1e-12, atol=1e-300)
    absref = np.abs(synth.bf16_bits_to_f32(X).astype(np.float64)) @ np.abs(Wd).T
    np.testing.assert_allclose(mag, absref, rtol=1e-12, atol=1e-300)


def test_w8a16_one_hot_rows_and_integer_inputs():
    """One-hot rows of X pick single dequantized weights exactly; integer X gives sw times the
    integer GEMM exactly.  Catches: a dropped scale, an off-by-one in k."""
    K, N = 64, 5
    q = synth.random_codes((N, K), seed=33)
    sw = synth.random_scales(N, seed=34)
    X = np.zeros((3, K), np.float32)
    X[0, 0] = 1.0
    X[1, 17] = 1.0
    X[2, K - 1] = -2.0
    y64, _ = oracle.gemm_w8a16(X, q, sw)
    np.testing.assert_array_equal(y64[0], q[:, 0].astype(np.float64) * sw.astype(np.float64))
    np.testing.assert_array_equal(y64[1], q[:, 17].astype(np.float64) * sw.astype(np.float64))
    np.testing.assert_array_equal(y64[2], -2.0 * q[:, K - 1].astype(np.float64) * sw.astype(np.float64))
    Xi = np.random.Generator(np.random.PCG64(35)).integers(-127, 128, (7, K)).astype(np.float32)
    y64, _ = oracle.gemm_w8a16(Xi, q, sw)
    acc = oracle.gemm_i32(Xi.astype(np.int8), q)
    np.testing.assert_array_equal(y64, acc.astype(np.float64) * sw.astype(np.float64)[None, :])


# ---------------------------------------------------------------------------------------------
# Smoothing folded into the norm before the layer (s3 step 1 offline; the lesson's s2)
# ---------------------------------------------------------------------------------------------

def rms_ref(h64, g64, eps):
    return h64 / np.sqrt(np.mean(h64 * h64, axis=1, keepdims=True) + eps) * g64[None, :]


def test_rms_norm_matches_numpy_float64():
    """Within a few fp32 roundings of the float64 formula.  Catches: mean over the wrong axis, a
    missing eps, sum instead of mean, the gain on the wrong axis."""
    h = synth.random_matrix((11, 320), seed=41, outliers=3)
    g = synth.random_scales(320, seed=42, lo=0.5, hi=2.0)
    for eps in (1e-5, 0.0):
        y = oracle.rms_norm(h, g, eps)
        ref = rms_ref(h.astype(np.float64), g.astype(np.float64), eps)
        np.testing.assert_allclose(y, ref, rtol=4e-7, atol=0)


def test_rms_norm_exact_cases():
    """Closed forms: a constant row 4 gives r = 1/4 exactly, so X~ = g; scaling a row by a power of
    two (eps = 0) leaves the output bit-identical.  Catches: rounding the wrong quantity, rms of
    something other than h."""
    g = synth.random_scales(64, seed=43, lo=0.5, hi=2.0)
    h = np.full((1, 64), 4.0, np.float32)
    np.testing.assert_array_equal(oracle.rms_norm(h, g, 0.0)[0], g)
    h = synth.random_matrix((5, 64), seed=44, outliers=1)
    y = oracle.rms_norm(h, g, 0.0)
    for k in (-3, 5):
        np.testing.assert_array_equal(oracle.rms_norm(h * np.float32(2.0 ** k), g, 0.0), y)


def test_fold_norm_gain_divides_and_identity_holds():
    """g' = g / s (one fp32 division); with it the norm output equals the smoothed norm output to
    fp32 rounding, and (norm(h) g / s) (s W) equals norm(h) g W (the SmoothQuant identity of s3).
    Catches: multiplying by s, folding into the wrong side."""
    K, N = 96, 7
    g = synth.random_scales(K, seed=45, lo=0.5, hi=2.0)
    s = synth.random_scales(K, seed=46, lo=0.1, hi=8.0)
    gf = oracle.fold_norm_gain(g, s)
    np.testing.assert_array_equal(gf, (g / s).astype(np.float32))
    h = synth.random_matrix((9, K), seed=47, outliers=2)
    W = synth.random_matrix((K, N), seed=48, scale=0.02)
    xs = oracle.rms_norm(h, gf, 1e-5).astype(np.float64)
    x = oracle.rms_norm(h, g, 1e-5).astype(np.float64)
    np.testing.assert_allclose(xs, x / s.astype(np.float64)[None, :], rtol=5e-7, atol=0)
    ws = oracle.smooth_weight(W, s).astype(np.float64)
    ref = x @ W.astype(np.float64)
    assert np.linalg.norm(xs @ ws - ref) <= 1e-5 * np.linalg.norm(ref)


def test_norm_quant_act_is_norm_then_per_row_quantize():
    """The codes and scales are the per-row quantize of the normalized row (numpy float32 division
    and round-half-even for INT8, torch's E4M3 cast for FP8)."""
    h = synth.f32_to_bf16_bits(synth.random_matrix((13, 256), seed=49, outliers=2))
    g = synth.random_scales(256, seed=50, lo=0.5, hi=2.0)
    y = oracle.rms_norm(h, g, 1e-5)
    amax = np.max(np.abs(y), axis=1)
    for qt in ("int8", "fp8"):
        q, sx = oracle.norm_quant_act(h, g, 1e-5, qt)
        Q = np.float32(127 if qt == "int8" else 448)
        np.testing.assert_array_equal(sx, (amax / Q).astype(np.float32))
        for r in range(13):
            ref = int8_ref(y[r], sx[r]) if qt == "int8" else e4m3_ref(y[r], sx[r])
            np.testing.assert_array_equal(q[r], ref)


def test_rms_norm_mean_is_order_free():
    """The mean square is the (double-double) sum of exact squares: reversing the order of the
    terms, or a row whose terms span 2^40 in magnitude, gives the float mean of math.fsum (the
    correctly rounded sum).  Catches: a plain double sum, whose order shows in the last bits."""
    import math
    rng = np.random.Generator(np.random.PCG64(51))
    h = rng.standard_normal((6, 4096)).astype(np.float32)
    h *= np.exp2(rng.integers(-20, 20, h.shape)).astype(np.float32)
    y = oracle.rms_norm(h, None, 0.0)
    yr = oracle.rms_norm(h[:, ::-1].copy(), None, 0.0)[:, ::-1]
    np.testing.assert_array_equal(y, yr)
    for r in range(6):
        ms = np.float32(math.fsum(float(v) * float(v) for v in h[r]) / 4096.0)
        rr = np.float32(1.0) / np.sqrt(ms)
        np.testing.assert_array_equal(y[r], (h[r] * rr).astype(np.float32))


@pytest.mark.parametrize("K", [16, 128, 1024, 4096, 8192])
def test_rms_norm_mean_square_tie(K):
    """Rows whose mean square is exactly halfway between two floats (rounds to even), and the same
    just past halfway through squares that a sequential double sum drops: the oracle's mean is the
    correctly rounded one (math.fsum of the exact squares over K, a power of two) in both, and the
    two rows normalize differently.  Catches: a plain double sum, a mean rounded twice."""
    import math
    h = synth.mean_square_tie_rows(K)
    y = oracle.rms_norm(h, None, 0.0)
    seq = 0.0
    for v in h[1].astype(np.float64):
        seq += v * v
    for r in range(2):
        ms = np.float32(math.fsum(float(v) * float(v) for v in h[r]) / K)
        rr = np.float32(1.0) / np.sqrt(ms)
        np.testing.assert_array_equal(y[r], (h[r] * rr).astype(np.float32))
    assert np.float32(seq / K) == np.float32(math.fsum(float(v) * float(v) for v in h[0]) / K)
    assert y[0, 0] != y[1, 0]


# ---- LayerNorm with the smoothing folded into gain and bias ---------------------------------

def ln_ref(h, g, b, eps):
    mu = h.mean(axis=1, keepdims=True)
    var = ((h - mu) ** 2).mean(axis=1, keepdims=True)
    return (h - mu) / np.sqrt(var + eps) * g[None, :] + b[None, :]


def test_layer_norm_matches_numpy_float64():
    """Within a few fp32 roundings of the float64 formula.  Catches: a missing mean subtraction,
    the variance about 0 (that is RMS norm), a missing eps, the bias before the gain."""
    h = synth.random_matrix((11, 320), seed=61, outliers=3) + np.float32(3.0)
    g = synth.random_scales(320, seed=62, lo=0.5, hi=2.0)
    b = synth.random_scales(320, seed=63, lo=-1.0, hi=1.0)
    for eps in (1e-5, 0.0):
        y = oracle.layer_norm(h, g, b, eps)
        ref = ln_ref(h.astype(np.float64), g.astype(np.float64), b.astype(np.float64), eps)
        np.testing.assert_allclose(y, ref, rtol=0, atol=2e-6 * np.abs(ref).max())


def test_layer_norm_exact_cases():
    """Closed forms: a constant row has d = 0, so X~ = b exactly; scaling a row by a power of two
    (eps = 0) leaves the output bit-identical (the mean scales exactly, the variance by the square);
    g = 1, b = 0 leaves a row with mean 0 and mean square 1 unchanged."""
    g = synth.random_scales(64, seed=64, lo=0.5, hi=2.0)
    b = synth.random_scales(64, seed=65, lo=0.25, hi=1.0)
    h = np.full((1, 64), 3.25, np.float32)
    np.testing.assert_array_equal(oracle.layer_norm(h, g, b, 1e-5)[0], b)
    h = synth.random_matrix((5, 64), seed=66, outliers=1) + np.float32(2.0)
    y = oracle.layer_norm(h, g, b, 0.0)
    for k in (-3, 5):
        np.testing.assert_array_equal(oracle.layer_norm(h * np.float32(2.0 ** k), g, b, 0.0), y)
    row = np.array([[1.0, -1.0] * 32], np.float32)
    np.testing.assert_array_equal(oracle.layer_norm(row, None, None, 0.0), row)


def test_layer_norm_fold_and_identity():
    """Gain and bias both divided by s (the division of fold_norm_gain): the folded norm equals the
    norm divided by s to fp32 rounding, and (LN(h) g/s + b/s)(s W) = (LN(h) g + b) W (s3's identity).
    Catches: folding only the gain, multiplying the bias by s."""
    K, N = 96, 7
    g = synth.random_scales(K, seed=67, lo=0.5, hi=2.0)
    b = synth.random_scales(K, seed=68, lo=-0.5, hi=0.5)
    s = synth.random_scales(K, seed=69, lo=0.1, hi=8.0)
    gf, bf = oracle.fold_norm_gain(g, s), oracle.fold_norm_gain(b, s)
    np.testing.assert_array_equal(bf, (b / s).astype(np.float32))
    h = synth.random_matrix((9, K), seed=70, outliers=2)
    W = synth.random_matrix((K, N), seed=71, scale=0.02)
    xs = oracle.layer_norm(h, gf, bf, 1e-5).astype(np.float64)
    x = oracle.layer_norm(h, g, b, 1e-5).astype(np.float64)
    np.testing.assert_allclose(xs, x / s.astype(np.float64)[None, :], rtol=0, atol=2e-6 * np.abs(xs).max())
    ws = oracle.smooth_weight(W, s).astype(np.float64)
    ref = x @ W.astype(np.float64)
    assert np.linalg.norm(xs @ ws - ref) <= 1e-5 * np.linalg.norm(ref)


def test_layer_norm_two_pass_rounding_reading():
    """The mean is the float of math.fsum(h) / K; d = h - mu is an fp32 subtraction; the variance
    is the float of math.fsum(d^2) / K (order-free), on rows whose values span 2^40, where d is not
    exact in fp32; reversing a row changes nothing.  Catches: d in double, a plain double sum, the
    one-pass variance mean(h^2) - mu^2."""
    import math
    rng = np.random.Generator(np.random.PCG64(72))
    h = rng.standard_normal((6, 2048)).astype(np.float32)
    h *= np.exp2(rng.integers(-20, 20, h.shape)).astype(np.float32)
    y = oracle.layer_norm(h, None, None, 0.0)
    np.testing.assert_array_equal(oracle.layer_norm(h[:, ::-1].copy(), None, None, 0.0)[:, ::-1], y)
    for r in range(6):
        mu = np.float32(math.fsum(float(v) for v in h[r]) / 2048.0)
        d = (h[r] - mu).astype(np.float32)
        var = np.float32(math.fsum(float(v) * float(v) for v in d) / 2048.0)
        rr = np.float32(1.0) / np.sqrt(var)
        np.testing.assert_array_equal(y[r], (d * rr).astype(np.float32))


@pytest.mark.parametrize("K", [16, 128, 1024, 8192])
def test_layer_norm_mean_and_variance_ties(K):
    """Rows whose mean, or whose variance, is exactly a float tie (rounds to even) or just past one
    through terms a sequential double sum drops: the oracle takes the correctly rounded value of
    the exact sum in both, and the two rows of each pair quantize to different scales (with a gain
    that makes the entries at the mean set the scale)."""
    import math

    def by_fsum(row):
        mu = np.float32(math.fsum(float(v) for v in row) / K)
        d = (row - mu).astype(np.float32)
        var = np.float32(math.fsum(float(v) * float(v) for v in d) / K)
        return mu, (d * (np.float32(1.0) / np.sqrt(var))).astype(np.float32)

    h = synth.mean_tie_rows(K)
    y = oracle.layer_norm(h, None, None, 0.0)
    mus = []
    for r in range(2):
        mu, ref = by_fsum(h[r])
        mus.append(mu)
        np.testing.assert_array_equal(y[r], ref)
    assert mus[0] != mus[1]
    seq = 0.0
    for v in h[1].astype(np.float64):
        seq += v
    assert np.float32(seq / K) == mus[0]          # a plain sequential double sum lands on the tie
    g = np.ones(K, np.float32)
    g[0] = 2.0 ** -20
    for qt in ("int8", "fp8"):
        _, sx = oracle.layer_norm_quant_act(h, g, None, 0.0, qt)
        assert sx[0] != sx[1]
    if K >= 32:
        hv = synth.variance_tie_rows(K)
        y = oracle.layer_norm(hv, None, None, 0.0)
        for r in range(2):
            var = np.float32(math.fsum(float(v) * float(v) for v in hv[r]) / K)     # mean is 0 exactly
            np.testing.assert_array_equal(y[r], (hv[r] * (np.float32(1.0) / np.sqrt(var))).astype(np.float32))
        assert not np.array_equal(y[0], y[1])


def test_layer_norm_quant_act_is_norm_then_per_row_quantize():
    h = synth.random_matrix((7, 256), seed=73, outliers=2)
    g = synth.random_scales(256, seed=74, lo=0.5, hi=2.0)
    b = synth.random_scales(256, seed=75, lo=-0.5, hi=0.5)
    for qt in ("int8", "fp8"):
        q, sx = oracle.layer_norm_quant_act(h, g, b, 1e-5, qt)
        q2, sx2 = oracle.quantize_rows(oracle.layer_norm(h, g, b, 1e-5), qt)
        np.testing.assert_array_equal(sx, sx2)
        np.testing.assert_array_equal(np.ascontiguousarray(q).view(np.uint8), np.ascontiguousarray(q2).view(np.uint8))
