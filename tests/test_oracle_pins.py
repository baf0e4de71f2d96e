"""Pins of the CPU oracle against things other than itself: the pages' worked examples (fixtures in
tests/golden/, each with its source), closed forms, library routines with the same semantics
(numpy float32 arithmetic, torch's bfloat16 / float8_e4m3fn casts), invariants and brute force.

Each test names the kind of mistake it is there to catch.
"""
import json
import math
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


# ---------------------------------------------------------------------------------------------
# Smoothing: the worked example (Weight-Activation Quantization, s3)
# ---------------------------------------------------------------------------------------------

def test_worked_example_smoothed_values():
    """Catches: multiply/divide swapped between X and W, s applied to the wrong axis."""
    g = golden("smoothing_worked_example.json")
    x = f32([g["activation_channel"]])              # one token, K = 3 channels
    w = f32(g["weight_channel"]).reshape(3, 1)      # K = 3, N = 1
    s = np.full(3, g["s"], np.float32)
    xs = oracle.smooth_act(x, s)
    ws = oracle.smooth_weight(w, s)
    np.testing.assert_array_equal(xs[0], f32(g["activation_smoothed"]))
    np.testing.assert_array_equal(ws[:, 0], f32(g["weight_smoothed"]))


def test_worked_example_inner_product_preserved():
    """The page's check: both inner products equal 40.6.  With s = 8 (a power of two) every fp32
    product is identical before and after smoothing, so the two fp64 sums are bit-identical."""
    g = golden("smoothing_worked_example.json")
    x = f32([g["activation_channel"]])
    w = f32(g["weight_channel"]).reshape(3, 1)
    s = np.full(3, g["s"], np.float32)
    before = float(np.dot(x[0].astype(np.float64), w[:, 0].astype(np.float64)))
    xs, ws = oracle.smooth_act(x, s), oracle.smooth_weight(w, s)
    after = float(np.dot(xs[0].astype(np.float64), ws[:, 0].astype(np.float64)))
    assert after == before
    assert abs(after - g["inner_product"]) < 1e-5


def test_worked_example_through_quantized_layer():
    """The whole quantized path on the worked example gives 40.6 within the INT8 error bound:
    |y - XW| <= sum_k (|x~_k| e_w + |w~_k| e_x + e_x e_w) with e = scale / 2."""
    g = golden("smoothing_worked_example.json")
    x = f32([g["activation_channel"]])
    w = f32(g["weight_channel"]).reshape(3, 1)
    s = np.full(3, g["s"], np.float32)
    qx, sx = oracle.quant_act(x, s)
    qw, sw = oracle.fold_quant_weight(w, s)
    acc = oracle.gemm_i32(qx, qw)
    y64, _ = oracle.dequant_i32(acc, sx, sw)
    xs, ws = oracle.smooth_act(x, s)[0], oracle.smooth_weight(w, s)[:, 0]
    ex, ew = sx[0] / 2, sw[0] / 2
    bound = float(np.sum(np.abs(xs) * ew + np.abs(ws) * ex + ex * ew))
    assert abs(y64[0, 0] - g["inner_product"]) <= bound
    assert qx[0, 2] == 127                          # the smoothed outlier still sets X's scale
    assert qw[0, :].tolist() == [127, 127, 32]      # W~ = [16, 16, 4]: 4 / (16/127) = 31.75


# ---------------------------------------------------------------------------------------------
# INT8 quantization: the outlier row (s2), ties, division
# ---------------------------------------------------------------------------------------------

def test_outlier_row_per_tensor_scale():
    """Catches: scale = amax * 127, amax / 128, a scale taken from the wrong element."""
    g = golden("outlier_row_per_tensor.json")
    q, sc = oracle.quantize_rows(f32(g["row"]), "int8")
    assert round(float(sc[0]), g["scale_printed_decimals"]) == g["scale_printed"]
    assert sc[0] == np.float32(80.0) / np.float32(127.0)
    small = [i for i in range(len(g["row"])) if i not in g["outlier_positions"]]
    assert np.all(np.abs(q[0, small]) <= g["small_values_max_abs_code"])
    assert np.all(q[0, small] == 0)                 # reading: under round-half-even they are all 0
    assert q[0, 2] == 127                           # the maximum maps to the top code
    assert q[0, 5] == 119                           # 75 / (80/127) = 119.06


def test_round_half_to_even():
    """Catches: round-half-away (gives 1, 3, -1, -3, 127), truncation."""
    row = f32([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5])   # amax 127 -> scale exactly 1
    q, sc = oracle.quantize_rows(row, "int8")
    assert sc[0] == 1.0
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 126]


def _reciprocal_differs_case():
    """Find (amax, v) where round(v / scale) differs from round(v * (1 / scale)) in float32."""
    rng = np.random.Generator(np.random.PCG64(7))
    for _ in range(200):
        amax = np.float32(rng.uniform(1, 100))
        scale = amax / np.float32(127)
        inv = np.float32(1) / scale
        n = np.arange(0, 127, dtype=np.float32)
        base = ((n + np.float32(0.5)) * scale).astype(np.float32)
        for d in range(-3, 4):
            v = np.nextafter(base, np.float32(np.inf) if d > 0 else np.float32(-np.inf)) if d else base
            for _ in range(abs(d) - 1):
                v = np.nextafter(v, np.float32(np.inf) if d > 0 else np.float32(-np.inf))
            v = v.astype(np.float32)
            a = np.rint(v / scale)
            b = np.rint(v * inv)
            bad = np.nonzero((a != b) & (np.abs(v) < amax))[0]
            if bad.size:
                return amax, v[bad[0]], a[bad[0]], b[bad[0]]
    raise AssertionError("no distinguishing case found")


def test_division_not_reciprocal():
    """Catches: v * (1/scale) in place of v / scale (the reading fixes IEEE division)."""
    amax, v, by_div, by_rcp = _reciprocal_differs_case()
    q, sc = oracle.quantize_rows(f32([amax, v]), "int8")
    assert q[0, 1] == by_div and q[0, 1] != by_rcp


def test_quantize_matches_numpy_float32():
    """numpy float32 arithmetic has the same IEEE semantics: scale = amax / 127 and
    q = rint(v / scale) (np.rint rounds half to even).  Random rows incl. outliers and zeros."""
    X = synth.random_matrix((64, 300), seed=3, outliers=4)
    X[5] = 0.0
    q, sc = oracle.quantize_rows(X, "int8")
    amax = np.max(np.abs(X), axis=1)
    ref_sc = (amax / np.float32(127)).astype(np.float32)
    np.testing.assert_array_equal(sc, ref_sc)
    with np.errstate(invalid="ignore", divide="ignore"):
        ref_q = np.clip(np.rint(X / ref_sc[:, None]), -127, 127)
    ref_q[amax == 0] = 0
    np.testing.assert_array_equal(q.astype(np.int64), ref_q.astype(np.int64))
    assert sc[5] == 0 and np.all(q[5] == 0)


def test_quantize_invariants():
    """Every nonzero row has a code of magnitude 127 and |q*scale - v| <= scale/2 (+ rounding)."""
    X = synth.random_matrix((50, 257), seed=11, outliers=3)
    q, sc = oracle.quantize_rows(X, "int8")
    assert np.all(np.max(np.abs(q.astype(np.int32)), axis=1) == 127)
    err = np.abs(q.astype(np.float64) * sc[:, None].astype(np.float64) - X.astype(np.float64))
    assert np.all(err <= sc[:, None] * 0.5 * (1 + 2.0 ** -20))
    assert np.all(np.abs(q.astype(np.int32)) <= 127)


def test_zero_scale_rows_get_zero_codes():
    """v / scale is undefined when the scale is 0.  Reading: such a row gets all-zero codes.  That
    covers an all-zero row and a row whose maximum is so small (a subnormal) that max / Q rounds to
    0 in float32 -- for Q = 127 and for Q = 448 -- while a slightly larger subnormal maximum gives a
    nonzero (subnormal) scale and ordinary codes."""
    tiny = np.float32(1e-44)                     # 1e-44 / 127 and 1e-44 / 448 round to 0
    assert np.float32(tiny / np.float32(127)) == 0 and np.float32(tiny / np.float32(448)) == 0
    big = np.float32(2e-43)                      # 2e-43 / 127 is a nonzero subnormal
    assert np.float32(big / np.float32(127)) > 0
    X = np.zeros((3, 16), np.float32)
    X[1, :3] = [tiny, -tiny, np.float32(0.5) * tiny]
    X[2, :3] = [big, -big, np.float32(0.0)]
    for qt in ("int8", "fp8_e4m3"):
        q, sc = oracle.quantize_rows(X, qt)
        assert sc[0] == 0 and sc[1] == 0 and np.all(q[:2] == 0)
    q, sc = oracle.quantize_rows(X, "int8")
    assert sc[2] == np.float32(big / np.float32(127)) and q[2, 0] == 127 and q[2, 1] == -127


# ---------------------------------------------------------------------------------------------
# Smoothing factors: closed forms (s3 "Choosing the Smoothing Factor")
# ---------------------------------------------------------------------------------------------

def _maxima(seed=5, K=400):
    rng = np.random.Generator(np.random.PCG64(seed))
    ax = rng.uniform(0.5, 400, K).astype(np.float32)
    aw = rng.uniform(1e-3, 0.2, K).astype(np.float32)
    return ax, aw


def test_smooth_factor_alpha_half_balances_ranges():
    """alpha = 0.5 splits the difficulty evenly: max|X~_j| = ax/s and max|W~_j| = s*aw both equal
    sqrt(ax*aw) (closed form, fp64) to a few ulp.  Catches: swapped ax/aw, alpha vs 1-alpha."""
    ax, aw = _maxima()
    s = oracle.smooth_factors(ax, aw, 0.5)
    target = np.sqrt(ax.astype(np.float64) * aw.astype(np.float64))
    xr = (ax / s).astype(np.float32).astype(np.float64)
    wr = (s * aw).astype(np.float32).astype(np.float64)
    ulp = np.spacing(target.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(xr - target) <= 3 * ulp)
    assert np.all(np.abs(wr - target) <= 3 * ulp)
    exact = np.sqrt(ax.astype(np.float64)) / np.sqrt(aw.astype(np.float64))
    assert np.all(np.abs(s - exact) <= 2 * np.spacing(s))


def test_smooth_factor_alpha_one_and_zero():
    """alpha = 1 moves all difficulty to W: max|X~_j| = 1 exactly; alpha = 0 leaves it on X:
    max|W~_j| = 1 within one ulp.  Catches: exponent applied to the wrong maximum."""
    ax, aw = _maxima(6)
    s1 = oracle.smooth_factors(ax, aw, 1.0)
    np.testing.assert_array_equal(ax / s1, np.ones_like(ax))
    s0 = oracle.smooth_factors(ax, aw, 0.0)
    assert np.all(np.abs((s0 * aw).astype(np.float64) - 1.0) <= 2.0 ** -23)


@pytest.mark.parametrize("alpha", [0.25, 0.75, 0.8])
def test_smooth_factor_general_alpha(alpha):
    ax, aw = _maxima(7)
    s = oracle.smooth_factors(ax, aw, alpha).astype(np.float64)
    exact = np.power(ax.astype(np.float64), alpha) / np.power(aw.astype(np.float64), 1 - alpha)
    assert np.all(np.abs(s - exact) <= 1.0 * np.spacing(exact.astype(np.float32)))


def test_smooth_factor_zero_maxima():
    assert oracle.smooth_factor(0.0, 0.3) == 1.0
    assert oracle.smooth_factor(4.0, 0.0) == 1.0
    assert oracle.smooth_factor(4.0, 0.25) == 4.0      # sqrt(4)/sqrt(0.25) exactly


def test_absmax_matches_numpy():
    """Catches: column and row reductions swapped, sign not removed."""
    X = synth.random_matrix((33, 70), seed=1, outliers=2)
    W = synth.random_matrix((70, 45), seed=2, scale=0.02)
    np.testing.assert_array_equal(oracle.absmax_cols(X), np.max(np.abs(X), axis=0))
    np.testing.assert_array_equal(oracle.absmax_rows(W), np.max(np.abs(W), axis=1))
    Xb = synth.f32_to_bf16_bits(-np.abs(X))
    np.testing.assert_array_equal(oracle.absmax_cols(Xb), np.max(np.abs(synth.bf16_bits_to_f32(Xb)), axis=0))


# ---------------------------------------------------------------------------------------------
# The identity Y = XW = X~ W~ (s3), 1e-5 relative
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2"])
def test_smoothing_identity(name):
    """||X~ W~ - X W||_F / ||X W||_F <= 1e-5, both products in fp64 from the fp32 tensors.
    Catches: smoothing X and W by different vectors, multiplying where it should divide."""
    wl = synth.workload(name)
    M = min(wl.M, 64)
    X, W = synth.make_inputs(wl, seed=0, M=M)
    ax, aw, s = oracle.smooth_scales(X, W, wl.alpha)
    Xf = X if X.dtype == np.float32 else synth.bf16_bits_to_f32(X)
    Wf = W if W.dtype == np.float32 else synth.bf16_bits_to_f32(W)
    cols = slice(0, 512)
    ref = Xf.astype(np.float64) @ Wf[:, cols].astype(np.float64)
    sm = oracle.smooth_act(X, s).astype(np.float64) @ oracle.smooth_weight(W, s)[:, cols].astype(np.float64)
    rel = np.linalg.norm(sm - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5
    assert not np.all(s == 1)


# ---------------------------------------------------------------------------------------------
# GEMM: brute force and library matmul
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 8, 64), (2, 3, 16)])
def test_gemm_bruteforce(M, N, K):
    """Triple loop in Python; catches transposed qw, dropped k terms."""
    a = synth.random_codes((M, K), 1)
    b = synth.random_codes((N, K), 2)
    acc = oracle.gemm_i32(a, b)
    for i in range(M):
        for j in range(N):
            assert acc[i, j] == sum(int(a[i, k]) * int(b[j, k]) for k in range(K))


def test_gemm_extremes_and_numpy():
    K = 4096
    a = np.full((4, K), 127, np.int8)
    a[1] = -127
    a[2, ::2] = -127
    b = np.full((3, K), -127, np.int8)
    b[1] = 127
    acc = oracle.gemm_i32(a, b)
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    np.testing.assert_array_equal(acc, ref)
    assert acc[0, 0] == -K * 127 * 127
    a = synth.random_codes((37, 300), 4)
    b = synth.random_codes((29, 300), 5)
    np.testing.assert_array_equal(oracle.gemm_i32(a, b), a.astype(np.int64) @ b.astype(np.int64).T)


def test_dequant_closed_form_and_bf16():
    acc = synth.random_codes((9, 300), 6).astype(np.int32) * 1000
    acc = acc[:, :11]
    sx, sw = synth.random_scales(9, 1), synth.random_scales(11, 2)
    y64, yb = oracle.dequant_i32(acc, sx, sw)
    ref64 = acc.astype(np.float64) * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    np.testing.assert_allclose(y64, ref64, rtol=1e-15, atol=0)
    y32 = (acc.astype(np.float32) * sx[:, None]) * sw[None, :]
    tb = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(yb, tb)


def test_bf16_rne_ties():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    assert oracle.bf16_rne(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_rne(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_rne(-2.0) == 0xC000


# ---------------------------------------------------------------------------------------------
# FP8 E4M3 (s4)
# ---------------------------------------------------------------------------------------------

def test_e4m3_format_facts():
    g = golden("e4m3_format.json")
    vals = [oracle.e4m3_decode(c) for c in range(256)]
    finite = [v for v in vals if not math.isnan(v)]
    assert max(finite) == g["max_finite"] and min(finite) == -g["max_finite"]
    assert sum(math.isnan(v) for v in vals) == 2                     # 0x7F, 0xFF
    ones = [v for v in finite if 1.0 <= v < 2.0]
    assert len(ones) == 2 ** g["mantissa_bits"]                      # 8 values per binade


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        d = oracle.e4m3_decode(c)
        if math.isnan(d):
            assert math.isnan(tv[c])
        else:
            assert d == tv[c], c


def test_e4m3_encode_roundtrip_and_torch():
    """Every finite code round-trips; midpoints round to the even mantissa; random values in
    [-448, 448] (normals, subnormals, zeros) agree with torch's float8_e4m3fn cast."""
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c
    rng = np.random.Generator(np.random.PCG64(9))
    v = np.concatenate([
        rng.uniform(-448, 448, 4000), rng.uniform(-1, 1, 2000) * 2.0 ** -6,
        np.exp2(rng.uniform(-12, 8.8, 2000)) * rng.choice([-1, 1], 2000),
    ]).astype(np.float32)
    finite = [oracle.e4m3_decode(c) for c in range(127)]
    mids = np.array([(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])], np.float32)
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 448.0, -448.0])])
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_fp8_quantize_rows():
    """scale = amax / 448; the maximum maps to +-448 (code 0x7E / 0xFE); codes decode to within
    half an E4M3 spacing of v / scale; zero rows give scale 0 and code 0."""
    X = synth.random_matrix((20, 256), seed=12, outliers=3)
    X[3] = 0
    q, sc = oracle.quantize_rows(X, "fp8")
    amax = np.max(np.abs(X), axis=1)
    np.testing.assert_array_equal(sc, (amax / np.float32(448)).astype(np.float32))
    dec = np.vectorize(oracle.e4m3_decode)(q)
    for r in range(20):
        if amax[r] == 0:
            assert sc[r] == 0 and np.all(q[r] == 0)
            continue
        t = (X[r] / sc[r]).astype(np.float32)
        ref = torch.from_numpy(np.clip(t, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(q[r], ref)
        assert np.max(np.abs(dec[r])) == 448.0


def test_fp8_gemm_exact():
    """The exact E4M3 dot product equals an fp64 matmul of decoded codes (exact in fp64 here:
    every partial sum is a multiple of 2^-18 below 2^35)."""
    a = synth.random_codes((13, 512), 21, "fp8_e4m3")
    b = synth.random_codes((7, 512), 22, "fp8_e4m3")
    sx, sw = synth.random_scales(13, 3), synth.random_scales(7, 4)
    lut = np.array([0.0 if (c & 0x7F) == 0x7F else oracle.e4m3_decode(c) for c in range(256)])
    A, B = lut[a], lut[b]
    dot = A @ B.T
    y64, mag = oracle.gemm_fp8(a, b, sx, sw)
    scale = sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    np.testing.assert_array_equal(y64, dot * scale)
    np.testing.assert_array_equal(mag, (np.abs(A) @ np.abs(B).T) * scale)


# ---------------------------------------------------------------------------------------------
# Weight path specifics: orientation of the codes and scales
# ---------------------------------------------------------------------------------------------

def test_fold_quant_weight_orientation():
    """qw is [N, K]: row n holds output channel n.  A weight with one large column n0 puts the top
    code in row n0 only; s multiplies row j of W.  Catches: per-row instead of per-column scales,
    untransposed codes."""
    K, N = 40, 6
    W = synth.random_matrix((K, N), seed=8, scale=0.02)
    s = np.ones(K, np.float32)
    s[17] = 64.0
    qw, sw = oracle.fold_quant_weight(W, s)
    assert qw.shape == (N, K)
    Ws = W.astype(np.float32) * s[:, None]
    np.testing.assert_array_equal(sw, (np.max(np.abs(Ws), axis=0) / np.float32(127)).astype(np.float32))
    with np.errstate(divide="ignore", invalid="ignore"):
        ref = np.clip(np.rint(Ws.T / sw[:, None]), -127, 127)
    np.testing.assert_array_equal(qw.astype(np.int64), ref.astype(np.int64))
    assert np.all(np.abs(qw[:, 17].astype(np.int32)) == 127)


def test_quant_act_divides_per_channel():
    X = synth.random_matrix((5, 32), seed=9)
    s = synth.random_scales(32, 10, 0.5, 4.0)
    qx, sx = oracle.quant_act(X, s)
    Xs = (X / s[None, :]).astype(np.float32)
    q2, s2 = oracle.quantize_rows(Xs)
    np.testing.assert_array_equal(qx, q2)
    np.testing.assert_array_equal(sx, s2)


def test_layer_error_smaller_with_smoothing():
    """The pages' motivation (s2, s3): with outlier channels, smoothing lowers the quantized
    layer's error against the exact X W.  Reported direction only, on the tiny workload."""
    X, W = synth.make_inputs("c1")
    ref = X.astype(np.float64) @ W.astype(np.float64)
    smooth = oracle.layer(X, W, 0.5)["y64"]
    ones = np.ones(X.shape[1], np.float32)
    qx, sx = oracle.quant_act(X, ones)
    qw, sw = oracle.fold_quant_weight(W, ones)
    plain, _ = oracle.dequant_i32(oracle.gemm_i32(qx, qw), sx, sw)
    e_s = np.linalg.norm(smooth - ref) / np.linalg.norm(ref)
    e_p = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    assert e_s < e_p
