"""The seeded generator: shapes, outlier structure and determinism (no method arithmetic here)."""
import numpy as np

import synth


def test_outlier_channels_and_determinism():
    wl = synth.workload("c1")
    X1, W1 = synth.make_inputs(wl, seed=0)
    X2, W2 = synth.make_inputs(wl, seed=0)
    np.testing.assert_array_equal(X1, X2)
    np.testing.assert_array_equal(W1, W2)
    assert X1.shape == (16, 512) and W1.shape == (512, 512) and X1.dtype == np.float32
    rng = np.random.Generator(np.random.PCG64(0))
    idx = rng.choice(wl.K, wl.n_out, replace=False)
    colmax = np.max(np.abs(X1), axis=0)
    assert wl.n_out == 5
    assert np.min(colmax[idx]) > np.max(np.delete(colmax, idx))   # outlier columns dominate
    assert abs(float(np.std(W1)) - wl.w_std) < 0.002


def test_bf16_workload_and_counts():
    wl = synth.workload("c2")
    assert (wl.M, wl.K, wl.N, wl.n_out) == (2048, 4096, 4096, 41)
    assert synth.workload("c3").n_out == 20 and synth.workload("c5").n_out == 82
    X, W = synth.make_inputs(wl, seed=1, M=8)
    assert X.dtype == np.uint16 and X.shape == (8, 4096) and W.shape == (4096, 4096)
    f = synth.bf16_bits_to_f32(X)
    assert np.all(np.isfinite(f))


def test_bf16_rounding_is_nearest_even():
    a = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.5, 0.0], np.float32)
    b = synth.f32_to_bf16_bits(a)
    assert b.tolist() == [0x3F80, 0x3F82, 0xBFC0, 0x0000]
