"""Python face of the plain CPU oracle (``w8a8_oracle.c``) for the W8A8 linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check and by the
benchmark's CPU-baseline leg.  The GPU library never imports, links or calls it, and it shares no
code with the GPU library; the two meet only on the seeded inputs from ``synth``.

Functions take numpy arrays as stored in memory (float32, or bf16 as uint16 bit patterns) and
return numpy arrays.  Each wrapper names the page section its C function follows; the C file's
header lists the readings taken where the pages leave a step open.

Parity of every function here is pinned by ``tests/test_oracle_*.py`` against the pages' worked
examples, closed forms, library routines (numpy / torch casts) and brute force.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB_PATH, build

F32, BF16 = 0, 1
INT8, FP8_E4M3 = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("W8A8_ORACLE_LIB", LIB_PATH)     # another build of the same source (sanitized)
    if path == LIB_PATH and not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    D, F = ctypes.c_double, ctypes.c_float
    sig = {
        "oracle_rounding_is_nearest": (I, []),
        "oracle_num_threads": (I, []),
        "oracle_absmax_cols": (None, [P, I, I64, I64, P]),
        "oracle_absmax_rows": (None, [P, I, I64, I64, P]),
        "oracle_smooth_factor": (F, [F, F, D]),
        "oracle_smooth_factors": (None, [P, P, I64, D, P]),
        "oracle_smooth_act": (None, [P, I, I64, I64, P, P]),
        "oracle_smooth_weight": (None, [P, I, I64, I64, P, P]),
        "oracle_e4m3_decode": (D, [ctypes.c_uint8]),
        "oracle_e4m3_encode": (ctypes.c_uint8, [F]),
        "oracle_quantize_rows": (None, [P, I64, I64, I, P, P]),
        "oracle_quant_act": (I, [P, I, I64, I64, P, I, P, P]),
        "oracle_fold_quant_weight": (I, [P, I, I64, I64, P, I, P, P]),
        "oracle_gemm_i32": (I, [P, P, I64, I64, I64, P]),
        "oracle_bf16_rne": (ctypes.c_uint16, [F]),
        "oracle_dequant_i32": (None, [P, P, P, I64, I64, P, P]),
        "oracle_gemm_fp8": (I, [P, P, I64, I64, I64, P, P, P, P]),
        "oracle_absmax_tensor": (F, [P, I, I64]),
        "oracle_tensor_scale": (F, [F, I]),
        "oracle_quantize_tensor": (None, [P, I, I64, F, I, P]),
        "oracle_quant_weight_tensor": (I, [P, I, I64, I64, I, P, P]),
        "oracle_gemm_w8a16": (I, [P, I, P, P, I64, I64, I64, P, P]),
        "oracle_fold_norm_gain": (None, [P, P, I64, P]),
        "oracle_rms_norm": (None, [P, I, I64, I64, P, F, P]),
        "oracle_norm_quant_act": (I, [P, I, I64, I64, P, F, I, P, P]),
        "oracle_layer_norm": (None, [P, I, I64, I64, P, P, F, P]),
        "oracle_layer_norm_quant_act": (I, [P, I, I64, I64, P, P, F, I, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if not lib.oracle_rounding_is_nearest():
        raise RuntimeError("oracle requires round-to-nearest-even")
    _lib = lib
    return lib


def num_threads() -> int:
    """Threads used by the oracle's parallel loops (the GEMMs); the rest runs on one thread."""
    return int(_load().oracle_num_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _input(a):
    """(contiguous array, dtype code) for an input stored as float32 or bf16 bits (uint16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def qtype_code(q) -> int:
    if q in (INT8, "int8"):
        return INT8
    if q in (FP8_E4M3, "fp8", "fp8_e4m3", "e4m3"):
        return FP8_E4M3
    raise ValueError(q)


# --- calibration maxima and smoothing factors (Weight-Activation Quantization, s3) ----------

def absmax_cols(x):
    """ax[j] = max_i |X[i, j]| for X [M, K]."""
    lib = _load()
    x, dt = _input(x)
    M, K = x.shape
    ax = np.empty(K, np.float32)
    lib.oracle_absmax_cols(_ptr(x), dt, M, K, _ptr(ax))
    return ax


def absmax_rows(w):
    """aw[j] = max_n |W[j, n]| for W [K, N]."""
    lib = _load()
    w, dt = _input(w)
    K, N = w.shape
    aw = np.empty(K, np.float32)
    lib.oracle_absmax_rows(_ptr(w), dt, K, N, _ptr(aw))
    return aw


def smooth_factors(ax, aw, alpha=0.5):
    """s_j = ax_j^alpha / aw_j^(1 - alpha); s_j = 1 where either maximum is zero."""
    lib = _load()
    ax, aw = _f32(ax), _f32(aw)
    s = np.empty(ax.shape[0], np.float32)
    lib.oracle_smooth_factors(_ptr(ax), _ptr(aw), ax.shape[0], float(alpha), _ptr(s))
    return s


def smooth_scales(x, w, alpha=0.5):
    """(ax, aw, s) from calibration activations X [M, K] and weights W [K, N]."""
    ax, aw = absmax_cols(x), absmax_rows(w)
    return ax, aw, smooth_factors(ax, aw, alpha)


def smooth_factor(ax, aw, alpha=0.5):
    return float(_load().oracle_smooth_factor(float(ax), float(aw), float(alpha)))


def smooth_act(x, s=None):
    """X~ = X diag(1/s) in float32 (division per channel)."""
    lib = _load()
    x, dt = _input(x)
    M, K = x.shape
    out = np.empty((M, K), np.float32)
    lib.oracle_smooth_act(_ptr(x), dt, M, K, _ptr(_f32(s)), _ptr(out))
    return out


def smooth_weight(w, s=None):
    """W~[j, n] = s_j * W[j, n] in float32."""
    lib = _load()
    w, dt = _input(w)
    K, N = w.shape
    out = np.empty((K, N), np.float32)
    lib.oracle_smooth_weight(_ptr(w), dt, K, N, _ptr(_f32(s)), _ptr(out))
    return out


# --- quantization (s2 INT8, s4 FP8) ----------------------------------------------------------

def _codes(buf, q):
    return buf.view(np.int8) if q == INT8 else buf


def quantize_rows(v, qtype="int8"):
    """Per-row symmetric quantization of a float32 matrix; returns (codes, scales)."""
    lib = _load()
    q = qtype_code(qtype)
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.ndim == 1:
        v = v[None, :]
    R, C = v.shape
    codes = np.empty((R, C), np.uint8)
    sc = np.empty(R, np.float32)
    lib.oracle_quantize_rows(_ptr(v), R, C, q, _ptr(codes), _ptr(sc))
    return _codes(codes, q), sc


def quant_act(x, s=None, qtype="int8"):
    """X [M, K] -> (codes [M, K], per-token scales [M]) after dividing by s."""
    lib = _load()
    q = qtype_code(qtype)
    x, dt = _input(x)
    M, K = x.shape
    codes = np.empty((M, K), np.uint8)
    sx = np.empty(M, np.float32)
    if lib.oracle_quant_act(_ptr(x), dt, M, K, _ptr(_f32(s)), q, _ptr(codes), _ptr(sx)) != 0:
        raise MemoryError("oracle_quant_act")
    return _codes(codes, q), sx


def fold_quant_weight(w, s=None, qtype="int8"):
    """W [K, N] -> (codes [N, K], per-output-channel scales [N]) after multiplying by s."""
    lib = _load()
    q = qtype_code(qtype)
    w, dt = _input(w)
    K, N = w.shape
    codes = np.empty((N, K), np.uint8)
    sw = np.empty(N, np.float32)
    if lib.oracle_fold_quant_weight(_ptr(w), dt, K, N, _ptr(_f32(s)), q, _ptr(codes), _ptr(sw)) != 0:
        raise MemoryError("oracle_fold_quant_weight")
    return _codes(codes, q), sw


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code) & 0xFF))


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def bf16_rne(v: float) -> int:
    return int(_load().oracle_bf16_rne(float(v)))


# --- GEMM and dequantize (s3 step 2; s4) ----------------------------------------------------

def gemm_i32(qx, qw):
    """acc [M, N] = qx [M, K] @ qw [N, K]^T, exact."""
    lib = _load()
    qx = np.ascontiguousarray(qx, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    M, K = qx.shape
    N, K2 = qw.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    if lib.oracle_gemm_i32(_ptr(qx), _ptr(qw), M, N, K, _ptr(acc)) != 0:
        raise OverflowError("int32 accumulator overflow")
    return acc


def dequant_i32(acc, sx, sw):
    """(y64 float64 [M, N], y_bf16 uint16 [M, N]) from int32 accumulators and scales."""
    lib = _load()
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    M, N = acc.shape
    y64 = np.empty((M, N), np.float64)
    yb = np.empty((M, N), np.uint16)
    lib.oracle_dequant_i32(_ptr(acc), _ptr(_f32(sx)), _ptr(_f32(sw)), M, N, _ptr(y64), _ptr(yb))
    return y64, yb


def gemm_fp8(qx, qw, sx, sw):
    """Exact E4M3 dot products, scaled: returns (y64, mag64), both float64 [M, N]."""
    lib = _load()
    qx = np.ascontiguousarray(qx, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    M, K = qx.shape
    N, K2 = qw.shape
    assert K == K2
    y64 = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    if lib.oracle_gemm_fp8(_ptr(qx), _ptr(qw), M, N, K, _ptr(_f32(sx)), _ptr(_f32(sw)),
                           _ptr(y64), _ptr(mag)) != 0:
        raise ValueError("NaN code in FP8 operands or K too large")
    return y64, mag


def layer(x, w, alpha=0.5, qtype="int8"):
    """The whole path on the CPU: calibration on X itself, fold, quantize, GEMM, dequantize.

    Returns a dict with every intermediate (ax, aw, s, qw, sw, qx, sx, acc or y64 ...).
    """
    q = qtype_code(qtype)
    ax, aw, s = smooth_scales(x, w, alpha)
    qw, sw = fold_quant_weight(w, s, q)
    qx, sx = quant_act(x, s, q)
    out = dict(ax=ax, aw=aw, s=s, qw=qw, sw=sw, qx=qx, sx=sx)
    if q == INT8:
        acc = gemm_i32(qx, qw)
        y64, yb = dequant_i32(acc, sx, sw)
        out.update(acc=acc, y64=y64, y_bf16=yb)
    else:
        y64, mag = gemm_fp8(qx, qw, sx, sw)
        out.update(y64=y64, mag64=mag)
    return out


# --- per-tensor scaling (Weight-Activation Quantization, s4 "Per-Tensor Scaling for FP8"; s2) --

def absmax_tensor(a) -> np.float32:
    """max |a| over the whole tensor."""
    a, dt = _input(a)
    return np.float32(_load().oracle_absmax_tensor(_ptr(a), dt, a.size))


def tensor_scale(amax, qtype="fp8") -> np.float32:
    """s = amax / Q (127 for INT8, 448 for E4M3), one fp32 division."""
    return np.float32(_load().oracle_tensor_scale(float(np.float32(amax)), qtype_code(qtype)))


def quant_tensor(a, amax, qtype="fp8"):
    """Codes of a / s with the one scale s = amax / Q, saturating at +-Q (amax may be an earlier
    tensor's maximum: delayed scaling).  Returns (codes shaped like a, s)."""
    lib = _load()
    q = qtype_code(qtype)
    a, dt = _input(a)
    sc = tensor_scale(amax, q)
    codes = np.empty(a.shape, np.uint8)
    lib.oracle_quantize_tensor(_ptr(a), dt, a.size, float(sc), q, _ptr(codes))
    return _codes(codes, q), sc


def quant_weight_tensor(w, qtype="fp8"):
    """W [K, N] -> (codes [N, K], the one scale max|W| / Q)."""
    lib = _load()
    q = qtype_code(qtype)
    w, dt = _input(w)
    K, N = w.shape
    codes = np.empty((N, K), np.uint8)
    sc = np.empty(1, np.float32)
    if lib.oracle_quant_weight_tensor(_ptr(w), dt, K, N, q, _ptr(codes), _ptr(sc)) != 0:
        raise MemoryError("oracle_quant_weight_tensor")
    return _codes(codes, q), sc[0]


def layer_tensor(x, w, qtype="fp8", amax_x=None):
    """The per-tensor path of s4 on the CPU: one scale for W, one for X, no smoothing.

    amax_x: the maximum X's scale is taken from; None takes this X's own maximum (current
    scaling), a number an earlier step's (delayed scaling, values beyond it saturate).
    """
    q = qtype_code(qtype)
    qw, sw = quant_weight_tensor(w, q)
    amax_now = absmax_tensor(x)
    qx, sx = quant_tensor(x, amax_now if amax_x is None else amax_x, q)
    M, N = x.shape[0], w.shape[1]
    sxv, swv = np.full(M, sx, np.float32), np.full(N, sw, np.float32)
    out = dict(qw=qw, sw=sw, qx=qx, sx=sx, amax_x=amax_now)
    if q == INT8:
        acc = gemm_i32(qx, qw)
        y64, yb = dequant_i32(acc, sxv, swv)
        out.update(acc=acc, y64=y64, y_bf16=yb)
    else:
        y64, mag = gemm_fp8(qx, qw, sxv, swv)
        out.update(y64=y64, mag64=mag)
    return out


# --- weight-only W8A16 GEMM (Weight-Activation Quantization, s1; the W8A16-vs-W8A8 lesson) ----

def gemm_w8a16(x, q, sw):
    """16-bit X [M, K] times dequantized INT8 weights (q [N, K], per-channel sw [N]):
    returns (y64, mag64), both float64 [M, N]; y64 = sw[n] * sum_k x[m, k] q[n, k]."""
    lib = _load()
    x, dt = _input(x)
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = x.shape
    N, K2 = q.shape
    assert K == K2
    y64 = np.empty((M, N), np.float64)
    mag = np.empty((M, N), np.float64)
    if lib.oracle_gemm_w8a16(_ptr(x), dt, _ptr(q), _ptr(_f32(sw)), M, N, K, _ptr(y64), _ptr(mag)) != 0:
        raise MemoryError("oracle_gemm_w8a16")
    return y64, mag


# --- smoothing folded into the norm before the layer (s3 step 1, offline; the lesson's s2) ----

def fold_norm_gain(g, s):
    """g'[j] = g[j] / s[j] (g None: 1), float32 [K]."""
    K = len(s) if s is not None else len(g)
    out = np.empty(K, np.float32)
    _load().oracle_fold_norm_gain(_ptr(_f32(g)), _ptr(_f32(s)), K, _ptr(out))
    return out


def rms_norm(h, g=None, eps=1e-5):
    """(h[j] * r) * g[j] per row, r = 1 / sqrt(mean(h^2) + eps): float32 [M, K]."""
    h, dt = _input(h)
    M, K = h.shape
    out = np.empty((M, K), np.float32)
    _load().oracle_rms_norm(_ptr(h), dt, M, K, _ptr(_f32(g)), float(np.float32(eps)), _ptr(out))
    return out


def norm_quant_act(h, g=None, eps=1e-5, qtype="int8"):
    """RMS norm with gain g (1/s folded in), then per-token quantize: (codes [M, K], scales [M])."""
    lib = _load()
    q = qtype_code(qtype)
    h, dt = _input(h)
    M, K = h.shape
    codes = np.empty((M, K), np.uint8)
    sx = np.empty(M, np.float32)
    if lib.oracle_norm_quant_act(_ptr(h), dt, M, K, _ptr(_f32(g)), float(np.float32(eps)), q, _ptr(codes),
                                 _ptr(sx)) != 0:
        raise MemoryError("oracle_norm_quant_act")
    return _codes(codes, q), sx


def layer_norm(h, g=None, b=None, eps=1e-5):
    """((h[j] - mu) * r) * g[j] + b[j] per row, mu and the variance about it rounded to float once:
    float32 [M, K]."""
    h, dt = _input(h)
    M, K = h.shape
    out = np.empty((M, K), np.float32)
    _load().oracle_layer_norm(_ptr(h), dt, M, K, _ptr(_f32(g)), _ptr(_f32(b)), float(np.float32(eps)), _ptr(out))
    return out


def layer_norm_quant_act(h, g=None, b=None, eps=1e-5, qtype="int8"):
    """LayerNorm with gain g and bias b (1/s folded into both), then per-token quantize:
    (codes [M, K], scales [M])."""
    lib = _load()
    q = qtype_code(qtype)
    h, dt = _input(h)
    M, K = h.shape
    codes = np.empty((M, K), np.uint8)
    sx = np.empty(M, np.float32)
    if lib.oracle_layer_norm_quant_act(_ptr(h), dt, M, K, _ptr(_f32(g)), _ptr(_f32(b)), float(np.float32(eps)), q,
                                       _ptr(codes), _ptr(sx)) != 0:
        raise MemoryError("oracle_layer_norm_quant_act")
    return _codes(codes, q), sx
