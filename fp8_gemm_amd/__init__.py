"""Python binding of libw8a8, the W8A8 linear layer for MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/w8a8.h``: each function here has the name of
the C entry point it calls, takes torch tensors that live on the GPU, allocates missing outputs
with torch and passes raw device pointers plus the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no CPU or PyTorch fallback: the library is
loaded on first use and every entry point raises ImportError if it has not been built
(``python -m fp8_gemm_amd.build``).

Layouts: X [M, K] and W [K, N] row-major float32 or bfloat16; quantized weights [N, K]; codes are
torch.int8 (INT8) or torch.uint8 holding OCP E4M3 bit patterns (view them as
torch.float8_e4m3fn); scales float32; Y bfloat16 [M, N].
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

W8A8_OK, W8A8_ERR_INVALID_ARG, W8A8_ERR_UNSUPPORTED, W8A8_ERR_HIP = 0, 1, 2, 3
W8A8_F32, W8A8_BF16 = 0, 1
W8A8_INT8, W8A8_FP8_E4M3 = 0, 1

ENTRY_POINTS = ("w8a8_smooth_scales", "w8a8_fold_quant_weight", "w8a8_quant_act", "w8a8_smooth_quant",
                "w8a8_gemm_dequant",
                "w8a8_gemm_i32", "w8a8_gemm_f32", "w8a8_absmax", "w8a8_quant_act_tensor",
                "w8a8_quant_weight_tensor", "w8a8_gemm_dequant_tensor", "w8a8_gemm_w8a16", "w8a8_fold_norm_gain",
                "w8a8_norm_quant_act", "w8a8_layer_norm_quant_act", "w8a8_status_string", "w8a8_version")


class W8A8Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {w8a8_status_string(status)} (status {status})")
        self.status = status


_lib = None


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libw8a8 is not built ({LIB_PATH} missing); run `python -m fp8_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sigs = {
        "w8a8_smooth_scales": (I, [P, I, I64, I64, P, I, I64, F, P, P, I, P, P]),
        "w8a8_fold_quant_weight": (I, [P, I, I64, I64, P, I, P, P, P]),
        "w8a8_quant_act": (I, [P, I, I64, I64, P, I, P, P, P]),
        "w8a8_smooth_quant": (I, [P, I, I64, I64, P, I, I64, F, I, P, P, P, P, P, P, P, P]),
        "w8a8_gemm_dequant": (I, [P, P, P, P, I, I64, I64, I64, P, P]),
        "w8a8_gemm_i32": (I, [P, P, I64, I64, I64, P, P]),
        "w8a8_gemm_f32": (I, [P, P, I64, I64, I64, P, P]),
        "w8a8_absmax": (I, [P, I, I64, P, I, P]),
        "w8a8_quant_act_tensor": (I, [P, I, I64, I64, P, I, P, P, P, I, P]),
        "w8a8_quant_weight_tensor": (I, [P, I, I64, I64, I, P, P, P]),
        "w8a8_gemm_dequant_tensor": (I, [P, P, P, P, I, I64, I64, I64, P, P]),
        "w8a8_gemm_w8a16": (I, [P, P, P, I64, I64, I64, P, P]),
        "w8a8_fold_norm_gain": (I, [P, P, I64, P, P]),
        "w8a8_norm_quant_act": (I, [P, I, I64, I64, P, F, I, P, P, P]),
        "w8a8_layer_norm_quant_act": (I, [P, I, I64, I64, P, P, F, I, P, P, P]),
        "w8a8_status_string": (ctypes.c_char_p, [I]),
        "w8a8_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def lib_path() -> str:
    return LIB_PATH


def w8a8_status_string(status: int) -> str:
    return _load().w8a8_status_string(int(status)).decode()


def w8a8_version() -> str:
    return _load().w8a8_version().decode()


# ---- marshalling helpers ---------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(t) -> int:
    if t.dtype == torch.float32:
        return W8A8_F32
    if t.dtype == torch.bfloat16:
        return W8A8_BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _qtype(q) -> int:
    if q in (W8A8_INT8, "int8"):
        return W8A8_INT8
    if q in (W8A8_FP8_E4M3, "fp8", "fp8_e4m3", "e4m3"):
        return W8A8_FP8_E4M3
    raise ValueError(f"unknown qtype {q!r}")


def _code_dtype(q: int):
    return torch.int8 if q == W8A8_INT8 else torch.uint8


def _dev(t, what):
    if t is not None and (not t.is_cuda or not t.is_contiguous()):
        raise ValueError(f"{what} must be a contiguous GPU tensor")
    return t


def _check(fn: str, status: int):
    if status != W8A8_OK:
        raise W8A8Error(fn, status)


# ---- entry points ------------------------------------------------------------------------------

def w8a8_smooth_scales(x, w, alpha: float = 0.5, ax=None, aw=None, s=None, accumulate: bool = False,
                       stream=None):
    """Calibration maxima and SmoothQuant factors; returns (ax, aw, s), each float32 [K]."""
    _dev(x, "x"), _dev(w, "w")
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError("x is [M, K] and w is [K, N]")
    dev = x.device
    ax = torch.empty(K, dtype=torch.float32, device=dev) if ax is None else _dev(ax, "ax")
    aw = torch.empty(K, dtype=torch.float32, device=dev) if aw is None else _dev(aw, "aw")
    s = torch.empty(K, dtype=torch.float32, device=dev) if s is None else _dev(s, "s")
    _check("w8a8_smooth_scales", _load().w8a8_smooth_scales(
        _ptr(x), _dtype(x), M, K, _ptr(w), _dtype(w), N, float(alpha), _ptr(ax), _ptr(aw),
        int(bool(accumulate)), _ptr(s), _stream(stream)))
    return ax, aw, s


def w8a8_fold_quant_weight(w, s=None, qtype="int8", wq=None, w_scale=None, stream=None):
    """W [K, N] -> (codes [N, K], per-output-channel scales float32 [N])."""
    _dev(w, "w"), _dev(s, "s")
    q = _qtype(qtype)
    K, N = w.shape
    wq = torch.empty((N, K), dtype=_code_dtype(q), device=w.device) if wq is None else _dev(wq, "wq")
    w_scale = torch.empty(N, dtype=torch.float32, device=w.device) if w_scale is None else _dev(w_scale, "w_scale")
    _check("w8a8_fold_quant_weight", _load().w8a8_fold_quant_weight(
        _ptr(w), _dtype(w), K, N, _ptr(s), q, _ptr(wq), _ptr(w_scale), _stream(stream)))
    return wq, w_scale


def w8a8_quant_act(x, s=None, qtype="int8", xq=None, x_scale=None, stream=None):
    """X [M, K] -> (codes [M, K], per-token scales float32 [M])."""
    _dev(x, "x"), _dev(s, "s")
    q = _qtype(qtype)
    M, K = x.shape
    xq = torch.empty((M, K), dtype=_code_dtype(q), device=x.device) if xq is None else _dev(xq, "xq")
    x_scale = torch.empty(M, dtype=torch.float32, device=x.device) if x_scale is None else _dev(x_scale, "x_scale")
    _check("w8a8_quant_act", _load().w8a8_quant_act(
        _ptr(x), _dtype(x), M, K, _ptr(s), q, _ptr(xq), _ptr(x_scale), _stream(stream)))
    return xq, x_scale


def w8a8_smooth_quant(x, w, alpha: float = 0.5, qtype="int8", out=None, stream=None):
    """Calibration, smoothing factors, weight fold + quantize and activation quantize in one call.
    Returns a dict ax, aw, s [K], wq [N, K], w_scale [N], xq [M, K], x_scale [M] (``out``: a dict
    of such tensors to write into)."""
    _dev(x, "x"), _dev(w, "w")
    q = _qtype(qtype)
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError("x is [M, K] and w is [K, N]")
    dev = x.device
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = dict(ax=torch.empty(K, **f32), aw=torch.empty(K, **f32), s=torch.empty(K, **f32),
                   wq=torch.empty((N, K), dtype=_code_dtype(q), device=dev), w_scale=torch.empty(N, **f32),
                   xq=torch.empty((M, K), dtype=_code_dtype(q), device=dev), x_scale=torch.empty(M, **f32))
    for name in ("ax", "aw", "s", "wq", "w_scale", "xq", "x_scale"):
        _dev(out[name], name)
    _check("w8a8_smooth_quant", _load().w8a8_smooth_quant(
        _ptr(x), _dtype(x), M, K, _ptr(w), _dtype(w), N, float(alpha), q, _ptr(out["ax"]), _ptr(out["aw"]),
        _ptr(out["s"]), _ptr(out["wq"]), _ptr(out["w_scale"]), _ptr(out["xq"]), _ptr(out["x_scale"]),
        _stream(stream)))
    return out


def w8a8_gemm_dequant(xq, x_scale, wq, w_scale, qtype="int8", y=None, stream=None):
    """Quantized GEMM + dequantize: returns Y bfloat16 [M, N]."""
    for t, n in ((xq, "xq"), (x_scale, "x_scale"), (wq, "wq"), (w_scale, "w_scale")):
        _dev(t, n)
    q = _qtype(qtype)
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq is [M, K] and wq is [N, K]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if y is None else _dev(y, "y")
    _check("w8a8_gemm_dequant", _load().w8a8_gemm_dequant(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), q, M, N, K, _ptr(y), _stream(stream)))
    return y


def w8a8_gemm_i32(xq, wq, acc=None, stream=None):
    """INT8 GEMM without the epilogue: int32 [M, N] accumulators."""
    _dev(xq, "xq"), _dev(wq, "wq")
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq is [M, K] and wq is [N, K]")
    acc = torch.empty((M, N), dtype=torch.int32, device=xq.device) if acc is None else _dev(acc, "acc")
    _check("w8a8_gemm_i32", _load().w8a8_gemm_i32(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc), _stream(stream)))
    return acc


def w8a8_gemm_f32(xq, wq, acc=None, stream=None):
    """E4M3 GEMM without the epilogue: the matrix cores' fp32 [M, N] accumulators."""
    _dev(xq, "xq"), _dev(wq, "wq")
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq is [M, K] and wq is [N, K]")
    acc = torch.empty((M, N), dtype=torch.float32, device=xq.device) if acc is None else _dev(acc, "acc")
    _check("w8a8_gemm_f32", _load().w8a8_gemm_f32(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc), _stream(stream)))
    return acc


def w8a8_layer(x, w, alpha: float = 0.5, qtype="int8", fused: bool = True, stream=None):
    """The whole path for one batch that is also its own calibration set: smooth_quant (or, with
    fused=False, smooth_scales -> fold_quant_weight -> quant_act) -> gemm_dequant.  Returns a dict
    of tensors."""
    if fused:
        r = w8a8_smooth_quant(x, w, alpha, qtype, stream=stream)
    else:
        ax, aw, s = w8a8_smooth_scales(x, w, alpha, stream=stream)
        wq, w_scale = w8a8_fold_quant_weight(w, s, qtype, stream=stream)
        xq, x_scale = w8a8_quant_act(x, s, qtype, stream=stream)
        r = dict(ax=ax, aw=aw, s=s, wq=wq, w_scale=w_scale, xq=xq, x_scale=x_scale)
    r["y"] = w8a8_gemm_dequant(r["xq"], r["x_scale"], r["wq"], r["w_scale"], qtype, stream=stream)
    return r


# ---- per-tensor scaling (one scale per tensor, held in a 1-element float32 tensor) ----------------

def w8a8_absmax(a, amax=None, accumulate: bool = False, stream=None):
    """max |a| over the whole tensor, into a float32 [1] tensor (merged with it if accumulate)."""
    _dev(a, "a")
    amax = torch.empty(1, dtype=torch.float32, device=a.device) if amax is None else _dev(amax, "amax")
    _check("w8a8_absmax", _load().w8a8_absmax(_ptr(a), _dtype(a), a.numel(), _ptr(amax), int(bool(accumulate)),
                                              _stream(stream)))
    return amax


def w8a8_quant_act_tensor(x, amax_in, qtype="fp8", xq=None, x_scale=None, amax_out=None, track: bool = False,
                          accumulate: bool = False, stream=None):
    """X [M, K] -> (codes [M, K], the one scale float32 [1], amax_out or None) with the scale
    amax_in / Q.  track: also return this X's maximum (for the next step's amax_in)."""
    _dev(x, "x"), _dev(amax_in, "amax_in")
    q = _qtype(qtype)
    M, K = x.shape
    xq = torch.empty((M, K), dtype=_code_dtype(q), device=x.device) if xq is None else _dev(xq, "xq")
    x_scale = torch.empty(1, dtype=torch.float32, device=x.device) if x_scale is None else _dev(x_scale, "x_scale")
    if track and amax_out is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    _dev(amax_out, "amax_out")
    _check("w8a8_quant_act_tensor", _load().w8a8_quant_act_tensor(
        _ptr(x), _dtype(x), M, K, _ptr(amax_in), q, _ptr(xq), _ptr(x_scale), _ptr(amax_out),
        int(bool(accumulate)), _stream(stream)))
    return xq, x_scale, amax_out


def w8a8_quant_weight_tensor(w, qtype="fp8", wq=None, w_scale=None, stream=None):
    """W [K, N] -> (codes [N, K], the one scale float32 [1] = max|W| / Q)."""
    _dev(w, "w")
    q = _qtype(qtype)
    K, N = w.shape
    wq = torch.empty((N, K), dtype=_code_dtype(q), device=w.device) if wq is None else _dev(wq, "wq")
    w_scale = torch.empty(1, dtype=torch.float32, device=w.device) if w_scale is None else _dev(w_scale, "w_scale")
    _check("w8a8_quant_weight_tensor", _load().w8a8_quant_weight_tensor(
        _ptr(w), _dtype(w), K, N, q, _ptr(wq), _ptr(w_scale), _stream(stream)))
    return wq, w_scale


def w8a8_gemm_dequant_tensor(xq, x_scale, wq, w_scale, qtype="fp8", y=None, stream=None):
    """Quantized GEMM + dequantize with one scale per operand: Y bfloat16 [M, N]."""
    for t, n in ((xq, "xq"), (x_scale, "x_scale"), (wq, "wq"), (w_scale, "w_scale")):
        _dev(t, n)
    q = _qtype(qtype)
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("xq is [M, K] and wq is [N, K]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device) if y is None else _dev(y, "y")
    _check("w8a8_gemm_dequant_tensor", _load().w8a8_gemm_dequant_tensor(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), q, M, N, K, _ptr(y), _stream(stream)))
    return y


def w8a8_layer_tensor(x, w, qtype="fp8", amax_prev=None, stream=None):
    """The per-tensor path: one scale for W (its own maximum) and one for X, from this X's maximum
    (amax_prev None: current scaling, two passes over X) or an earlier step's (delayed scaling: one
    pass that also returns this X's maximum as amax for the next step)."""
    wq, w_scale = w8a8_quant_weight_tensor(w, qtype, stream=stream)
    if amax_prev is None:
        amax = w8a8_absmax(x, stream=stream)
        xq, x_scale, _ = w8a8_quant_act_tensor(x, amax, qtype, stream=stream)
    else:
        xq, x_scale, amax = w8a8_quant_act_tensor(x, amax_prev, qtype, track=True, stream=stream)
    y = w8a8_gemm_dequant_tensor(xq, x_scale, wq, w_scale, qtype, stream=stream)
    return dict(wq=wq, w_scale=w_scale, xq=xq, x_scale=x_scale, amax=amax, y=y)


# ---- weight-only W8A16 ------------------------------------------------------------------------------

def w8a8_gemm_w8a16(x, wq, w_scale, y=None, stream=None):
    """bf16 X [M, K] times INT8 weights (wq [N, K], per-channel w_scale [N]) on the bf16 matrix
    cores: Y bfloat16 [M, N] = w_scale[n] * sum_k x[m, k] wq[n, k]."""
    for t, n in ((x, "x"), (wq, "wq"), (w_scale, "w_scale")):
        _dev(t, n)
    if x.dtype != torch.bfloat16 or wq.dtype != torch.int8:
        raise TypeError("w8a8_gemm_w8a16 takes bf16 x and int8 wq")
    M, K = x.shape
    N, K2 = wq.shape
    if K2 != K:
        raise ValueError("x is [M, K] and wq is [N, K]")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device) if y is None else _dev(y, "y")
    _check("w8a8_gemm_w8a16", _load().w8a8_gemm_w8a16(_ptr(x), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(y),
                                                      _stream(stream)))
    return y


# ---- RMS norm with the smoothing folded into its gain ----------------------------------------------

def w8a8_fold_norm_gain(g, s, out=None, stream=None):
    """g' = g / s (either may be None = 1): float32 [K]."""
    _dev(g, "g"), _dev(s, "s")
    ref = g if g is not None else s
    K = ref.numel()
    out = torch.empty(K, dtype=torch.float32, device=ref.device) if out is None else _dev(out, "out")
    _check("w8a8_fold_norm_gain", _load().w8a8_fold_norm_gain(_ptr(g), _ptr(s), K, _ptr(out), _stream(stream)))
    return out


def w8a8_norm_quant_act(h, g=None, eps: float = 1e-5, qtype="int8", xq=None, x_scale=None, stream=None):
    """RMS norm of h [M, K] with gain g (1/s folded in), then per-token quantize:
    (codes [M, K], scales float32 [M])."""
    _dev(h, "h"), _dev(g, "g")
    q = _qtype(qtype)
    M, K = h.shape
    xq = torch.empty((M, K), dtype=_code_dtype(q), device=h.device) if xq is None else _dev(xq, "xq")
    x_scale = torch.empty(M, dtype=torch.float32, device=h.device) if x_scale is None else _dev(x_scale, "x_scale")
    _check("w8a8_norm_quant_act", _load().w8a8_norm_quant_act(
        _ptr(h), _dtype(h), M, K, _ptr(g), float(eps), q, _ptr(xq), _ptr(x_scale), _stream(stream)))
    return xq, x_scale


def w8a8_layer_norm_quant_act(h, g=None, b=None, eps: float = 1e-5, qtype="int8", xq=None, x_scale=None,
                              stream=None):
    """LayerNorm of h [M, K] with gain g and bias b (1/s folded into both), then per-token
    quantize: (codes [M, K], scales float32 [M])."""
    _dev(h, "h"), _dev(g, "g"), _dev(b, "b")
    q = _qtype(qtype)
    M, K = h.shape
    xq = torch.empty((M, K), dtype=_code_dtype(q), device=h.device) if xq is None else _dev(xq, "xq")
    x_scale = torch.empty(M, dtype=torch.float32, device=h.device) if x_scale is None else _dev(x_scale, "x_scale")
    _check("w8a8_layer_norm_quant_act", _load().w8a8_layer_norm_quant_act(
        _ptr(h), _dtype(h), M, K, _ptr(g), _ptr(b), float(eps), q, _ptr(xq), _ptr(x_scale), _stream(stream)))
    return xq, x_scale
