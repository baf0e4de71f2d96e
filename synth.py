"""Seeded synthetic inputs for the W8A8 linear layer Y = X W.

This module only draws numbers; it holds none of the method's arithmetic (no smoothing, no
quantization, no GEMM).  Both the CPU oracle and the GPU path are fed from it.

Workload model (Weight-Activation Quantization guide, section 2 "The Problem: Activation
Outliers"): activations are roughly standard normal except for a few feature dimensions whose
values are 10-100x larger; weights are well-behaved Gaussians.  Each outlier *channel* (a column of
X, i.e. one index of the contraction dimension) gets one multiplier drawn from U(lo, hi).

Draw order (numpy ``Generator(PCG64(seed))``), fixed so that a seed names one input set:
  1. ``idx = rng.choice(K, n_out, replace=False)``   outlier channels, n_out = round(frac * K)
  2. ``f = rng.uniform(lo, hi, n_out)``               one factor per outlier channel
  3. ``X = rng.standard_normal((M, K), float32)``; ``X[:, idx] *= f``
  4. ``W = rng.normal(0, w_std, (K, N))`` cast to float32
  5. bf16 workloads: X and W are rounded to bfloat16 (round to nearest even) and returned as the
     uint16 bit patterns.

The shapes stand in for Llama-style projection layers (the pages name Llama-3.1-8B and -70B); no
dataset, checkpoint or trained weight is used.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict

import numpy as np

F32 = "f32"
BF16 = "bf16"
INT8 = "int8"
FP8 = "fp8_e4m3"


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    dtype: str          # element type of X and W as stored in HBM: "f32" or "bf16"
    out_frac: float     # fraction of the K channels that are outliers
    lo: float           # outlier multiplier range U(lo, hi)
    hi: float
    w_std: float        # standard deviation of the Gaussian weights
    qtype: str          # quantized format of the GEMM operands: "int8" or "fp8_e4m3"
    alpha: float = 0.5  # SmoothQuant migration strength

    @property
    def n_out(self) -> int:
        return int(round(self.out_frac * self.K))

    def as_dict(self) -> dict:
        d = asdict(self)
        d["n_out"] = self.n_out
        return d


WORKLOADS = {
    "tiny_16x512x512_f32_int8": Workload("tiny_16x512x512_f32_int8", 16, 512, 512, F32, 0.01, 10, 100, 0.02, INT8),
    "prefill_2048x4096x4096_int8": Workload("prefill_2048x4096x4096_int8", 2048, 4096, 4096, BF16, 0.01, 10, 100, 0.02, INT8),
    "mlp_up_8192x4096x11008_int8": Workload("mlp_up_8192x4096x11008_int8", 8192, 4096, 11008, BF16, 0.005, 20, 100, 0.02, INT8),
    "decode_16x4096x14336_int8": Workload("decode_16x4096x14336_int8", 16, 4096, 14336, BF16, 0.01, 10, 100, 0.02, INT8),
    "large_8192x8192x28672_fp8": Workload("large_8192x8192x28672_fp8", 8192, 8192, 28672, BF16, 0.01, 10, 100, 0.015, FP8),
}
# Short aliases, in the order the workloads were specified (tiny, prefill, MLP-up, decode, FP8).
ALIASES = dict(zip(["c1", "c2", "c3", "c4", "c5"], WORKLOADS))


def workload(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns.

    Input preparation only: the workloads store X and W in bf16.  Inputs here are finite.
    """
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_activations(M: int, K: int, n_out: int, lo: float, hi: float, rng: np.random.Generator):
    """X ~ N(0,1) of shape [M, K] with n_out channels scaled by U(lo, hi); returns (X, idx, f)."""
    idx = rng.choice(K, n_out, replace=False) if n_out > 0 else np.zeros(0, dtype=np.int64)
    f = rng.uniform(lo, hi, n_out)
    X = rng.standard_normal((M, K), dtype=np.float32)
    if n_out:
        X[:, idx] *= f.astype(np.float32)
    return X, idx, f


def gaussian_weights(K: int, N: int, std: float, rng: np.random.Generator) -> np.ndarray:
    return rng.normal(0.0, std, (K, N)).astype(np.float32)


def make_inputs(wl: Workload | str, seed: int = 0, M: int | None = None):
    """Return (X, W) for a workload as stored in HBM.

    f32 workloads give float32 arrays; bf16 workloads give uint16 bf16 bit patterns.
    ``M`` overrides the row count (same channel statistics), e.g. for a bounded sample.
    """
    if isinstance(wl, str):
        wl = workload(wl)
    rng = np.random.Generator(np.random.PCG64(seed))
    m = wl.M if M is None else M
    X, _, _ = outlier_activations(m, wl.K, wl.n_out, wl.lo, wl.hi, rng)
    W = gaussian_weights(wl.K, wl.N, wl.w_std, rng)
    if wl.dtype == BF16:
        return f32_to_bf16_bits(X), f32_to_bf16_bits(W)
    return X, W


def random_matrix(shape, seed: int, dtype: str = F32, scale: float = 1.0, outliers: int = 0,
                  lo: float = 10.0, hi: float = 100.0):
    """Generic seeded matrix for edge-case tests: N(0, scale^2), optional outlier columns."""
    rng = np.random.Generator(np.random.PCG64(seed))
    R, C = shape
    if outliers:
        A, _, _ = outlier_activations(R, C, outliers, lo, hi, rng)
        A *= np.float32(scale)
    else:
        A = (rng.standard_normal((R, C), dtype=np.float32) * np.float32(scale)).astype(np.float32)
    return f32_to_bf16_bits(A) if dtype == BF16 else A


def random_codes(shape, seed: int, qtype: str = INT8) -> np.ndarray:
    """Uniform random quantized operands for GEMM-only tests.

    int8: integers in [-127, 127]; fp8_e4m3: any code that is not NaN (0x7F, 0xFF).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if qtype == INT8:
        return rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8)
    c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] &= 0xF0    # replace NaN codes by a finite code
    return c


def random_scales(n: int, seed: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(lo, hi, n).astype(np.float32)


def mean_square_tie_rows(K: int) -> np.ndarray:
    """Two float32 rows of length K (a power of two, >= 16) built from powers of two.

    Row 0: one 8.0 (two when log2(K) is even), then the rest of a sum of squares that puts the mean
    square exactly halfway between two adjacent floats.  Row 1: the same plus six squares of 2^-24
    placed after the 8.0 in its first 8 elements, each below half an ulp of the running sum there,
    so that a sequential double sum drops them while the exact mean lies just past the halfway
    point.  The odd power of two keeps the square root of the mean inexact, so a one-ulp change in
    the mean shows in the normalized row."""
    assert K >= 16 and K & (K - 1) == 0
    two = (K.bit_length() - 1) % 2 == 0
    rows = np.zeros((2, K), np.float32)
    rows[:, 0] = 8.0
    if two:
        rows[:, 2] = 8.0
        rows[:, 8:10] = 2.0 ** -9           # 2 * 2^-18 = half an ulp of 128 / K, times K
    else:
        rows[:, 8] = 2.0 ** -9              # 2^-18 = half an ulp of 64 / K, times K
    small = [1, 3, 4, 5, 6, 7]
    rows[1, small] = 2.0 ** -24
    return rows


def mean_tie_rows(K: int) -> np.ndarray:
    """Two float32 rows of length K (a power of two, >= 16) whose sum is 128 + 2^-17, so their mean
    (128 + 2^-17) / K lies exactly halfway between two adjacent floats; row 1 adds six terms 2^-48
    after the 128 in its first 8 elements.  Each is below half an ulp of the running sum there, so a
    sequential double sum drops them, but together they exceed half an ulp of 128 in double, so the
    exact sum, rounded to double, and its mean lie just past the halfway point."""
    assert K >= 16 and K & (K - 1) == 0
    rows = np.zeros((2, K), np.float32)
    rows[:, 0] = 128.0
    rows[:, 1] = 2.0 ** -17
    rows[1, 2:8] = 2.0 ** -48
    return rows


def variance_tie_rows(K: int) -> np.ndarray:
    """Two float32 rows of length K (a power of two, >= 32) with mean exactly 0 (each value and its
    negation) whose mean square is that of mean_square_tie_rows(K // 2): a float tie in row 0 and
    just past it, through squares a sequential double sum drops, in row 1."""
    t = mean_square_tie_rows(K // 2)
    return np.concatenate([t, -t], axis=1)
