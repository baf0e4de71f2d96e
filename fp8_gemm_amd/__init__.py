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

from . import _cabi
from .build import LIB_PATH

from ._cabi import (ENTRY_POINTS, W8A8_BF16, W8A8_ERR_HIP, W8A8_ERR_INVALID_ARG,  # noqa: F401
                    W8A8_ERR_UNSUPPORTED, W8A8_F32, W8A8_FP8_E4M3, W8A8_INT8, W8A8_OK)


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
    _lib = _cabi.load(LIB_PATH)
    return _lib


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


_CODES = (torch.int8, torch.uint8, torch.float8_e4m3fn)   # one byte per code
_F32 = (torch.float32,)


def _arg(t, what, dtypes=None, shape=None):
    """A tensor argument: None, or a contiguous GPU tensor of one of dtypes whose shape is shape
    (an int checks the element count).  Checked before any pointer reaches the library, so that a
    wrong size or element type is a Python error and not an out-of-bounds device access."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous GPU tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{what} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if isinstance(shape, int):
        if t.numel() != shape:
            raise ValueError(f"{what} must have {shape} elements, got {t.numel()}")
    elif shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _mat(t, what, dtypes):
    """A 2-D tensor argument; returns (tensor, rows, cols)."""
    _arg(t, what, dtypes)
    if t.dim() != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(t.shape)}")
    return t, t.shape[0], t.shape[1]


_FLOAT_IN = (torch.float32, torch.bfloat16)


def _check(fn: str, status: int):
    if status != W8A8_OK:
        raise W8A8Error(fn, status)


def _out(t, what, dtypes, shape, device):
    """An output: allocated when None, else checked like an argument."""
    if t is None:
        return torch.empty(shape, dtype=dtypes[0], device=device)
    return _arg(t, what, dtypes, shape)


# ---- entry points ------------------------------------------------------------------------------

def w8a8_smooth_scales(x, w, alpha: float = 0.5, ax=None, aw=None, s=None, accumulate: bool = False,
                       stream=None):
    """Calibration maxima and SmoothQuant factors; returns (ax, aw, s), each float32 [K]."""
    _, M, K = _mat(x, "x", _FLOAT_IN)
    _, K2, N = _mat(w, "w", _FLOAT_IN)
    if K2 != K:
        raise ValueError("x is [M, K] and w is [K, N]")
    ax = _out(ax, "ax", _F32, K, x.device)
    aw = _out(aw, "aw", _F32, K, x.device)
    s = _out(s, "s", _F32, K, x.device)
    _check("w8a8_smooth_scales", _load().w8a8_smooth_scales(
        _ptr(x), _dtype(x), M, K, _ptr(w), _dtype(w), N, float(alpha), _ptr(ax), _ptr(aw),
        int(bool(accumulate)), _ptr(s), _stream(stream)))
    return ax, aw, s


def w8a8_fold_quant_weight(w, s=None, qtype="int8", wq=None, w_scale=None, stream=None):
    """W [K, N] -> (codes [N, K], per-output-channel scales float32 [N])."""
    _, K, N = _mat(w, "w", _FLOAT_IN)
    _arg(s, "s", _F32, K)
    q = _qtype(qtype)
    wq = _out(wq, "wq", (_code_dtype(q),) + _CODES, (N, K), w.device)
    w_scale = _out(w_scale, "w_scale", _F32, N, w.device)
    _check("w8a8_fold_quant_weight", _load().w8a8_fold_quant_weight(
        _ptr(w), _dtype(w), K, N, _ptr(s), q, _ptr(wq), _ptr(w_scale), _stream(stream)))
    return wq, w_scale


def w8a8_quant_act(x, s=None, qtype="int8", xq=None, x_scale=None, stream=None):
    """X [M, K] -> (codes [M, K], per-token scales float32 [M])."""
    _, M, K = _mat(x, "x", _FLOAT_IN)
    _arg(s, "s", _F32, K)
    q = _qtype(qtype)
    xq = _out(xq, "xq", (_code_dtype(q),) + _CODES, (M, K), x.device)
    x_scale = _out(x_scale, "x_scale", _F32, M, x.device)
    _check("w8a8_quant_act", _load().w8a8_quant_act(
        _ptr(x), _dtype(x), M, K, _ptr(s), q, _ptr(xq), _ptr(x_scale), _stream(stream)))
    return xq, x_scale


def w8a8_smooth_quant(x, w, alpha: float = 0.5, qtype="int8", out=None, stream=None):
    """Calibration, smoothing factors, weight fold + quantize and activation quantize in one call.
    Returns a dict ax, aw, s [K], wq [N, K], w_scale [N], xq [M, K], x_scale [M] (``out``: a dict
    of such tensors to write into)."""
    _, M, K = _mat(x, "x", _FLOAT_IN)
    _, K2, N = _mat(w, "w", _FLOAT_IN)
    if K2 != K:
        raise ValueError("x is [M, K] and w is [K, N]")
    q = _qtype(qtype)
    codes = (_code_dtype(q),) + _CODES
    want = dict(ax=(_F32, K), aw=(_F32, K), s=(_F32, K), wq=(codes, (N, K)), w_scale=(_F32, N),
                xq=(codes, (M, K)), x_scale=(_F32, M))
    out = {} if out is None else dict(out)
    for name, (dts, shape) in want.items():
        out[name] = _out(out.get(name), name, dts, shape, x.device)
    _check("w8a8_smooth_quant", _load().w8a8_smooth_quant(
        _ptr(x), _dtype(x), M, K, _ptr(w), _dtype(w), N, float(alpha), q, _ptr(out["ax"]), _ptr(out["aw"]),
        _ptr(out["s"]), _ptr(out["wq"]), _ptr(out["w_scale"]), _ptr(out["xq"]), _ptr(out["x_scale"]),
        _stream(stream)))
    return out


def w8a8_quant_pair(x, w, s, w_scale, qtype="int8", xq=None, x_scale=None, wq=None, stream=None):
    """Both operands' codes in one launch, given s [K] and the final weight scales w_scale [N]
    (those of w8a8_fold_quant_weight / w8a8_smooth_quant): returns (xq [M, K], x_scale [M],
    wq [N, K])."""
    _, M, K = _mat(x, "x", _FLOAT_IN)
    _, K2, N = _mat(w, "w", _FLOAT_IN)
    if K2 != K:
        raise ValueError("x is [M, K] and w is [K, N]")
    if s is None or w_scale is None:
        raise ValueError("w8a8_quant_pair needs s and w_scale")
    _arg(s, "s", _F32, K)
    _arg(w_scale, "w_scale", _F32, N)
    q = _qtype(qtype)
    codes = (_code_dtype(q),) + _CODES
    xq = _out(xq, "xq", codes, (M, K), x.device)
    x_scale = _out(x_scale, "x_scale", _F32, M, x.device)
    wq = _out(wq, "wq", codes, (N, K), x.device)
    _check("w8a8_quant_pair", _load().w8a8_quant_pair(
        _ptr(x), _dtype(x), M, K, _ptr(w), _dtype(w), N, _ptr(s), _ptr(w_scale), q, _ptr(xq), _ptr(x_scale),
        _ptr(wq), _stream(stream)))
    return xq, x_scale, wq


def _gemm_operands(xq, wq):
    _, M, K = _mat(xq, "xq", _CODES)
    _, N, K2 = _mat(wq, "wq", _CODES)
    if K2 != K:
        raise ValueError("xq is [M, K] and wq is [N, K]")
    return M, N, K


def w8a8_gemm_dequant(xq, x_scale, wq, w_scale, qtype="int8", y=None, stream=None):
    """Quantized GEMM + dequantize: returns Y bfloat16 [M, N]."""
    M, N, K = _gemm_operands(xq, wq)
    _arg(x_scale, "x_scale", _F32, M)
    _arg(w_scale, "w_scale", _F32, N)
    q = _qtype(qtype)
    y = _out(y, "y", (torch.bfloat16,), (M, N), xq.device)
    _check("w8a8_gemm_dequant", _load().w8a8_gemm_dequant(
        _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), q, M, N, K, _ptr(y), _stream(stream)))
    return y


def w8a8_gemm_i32(xq, wq, acc=None, stream=None):
    """INT8 GEMM without the epilogue: int32 [M, N] accumulators."""
    M, N, K = _gemm_operands(xq, wq)
    acc = _out(acc, "acc", (torch.int32,), (M, N), xq.device)
    _check("w8a8_gemm_i32", _load().w8a8_gemm_i32(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc), _stream(stream)))
    return acc


def w8a8_gemm_f32(xq, wq, acc=None, stream=None):
    """E4M3 GEMM without the epilogue: the matrix cores' fp32 [M, N] accumulators."""
    M, N, K = _gemm_operands(xq, wq)
    acc = _out(acc, "acc", _F32, (M, N), xq.device)
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
    _arg(a, "a", _FLOAT_IN)
    amax = _out(amax, "amax", _F32, 1, a.device)
    _check("w8a8_absmax", _load().w8a8_absmax(_ptr(a), _dtype(a), a.numel(), _ptr(amax), int(bool(accumulate)),
                                              _stream(stream)))
    return amax


def w8a8_quant_act_tensor(x, amax_in, qtype="fp8", xq=None, x_scale=None, amax_out=None, track: bool = False,
                          accumulate: bool = False, stream=None):
    """X [M, K] -> (codes [M, K], the one scale float32 [1], amax_out or None) with the scale
    amax_in / Q.  track: also return this X's maximum (for the next step's amax_in)."""
    _, M, K = _mat(x, "x", _FLOAT_IN)
    _arg(amax_in, "amax_in", _F32, 1)
    q = _qtype(qtype)
    xq = _out(xq, "xq", (_code_dtype(q),) + _CODES, (M, K), x.device)
    x_scale = _out(x_scale, "x_scale", _F32, 1, x.device)
    if track or amax_out is not None:
        amax_out = _out(amax_out, "amax_out", _F32, 1, x.device)
    _check("w8a8_quant_act_tensor", _load().w8a8_quant_act_tensor(
        _ptr(x), _dtype(x), M, K, _ptr(amax_in), q, _ptr(xq), _ptr(x_scale), _ptr(amax_out),
        int(bool(accumulate)), _stream(stream)))
    return xq, x_scale, amax_out


def w8a8_quant_weight_tensor(w, qtype="fp8", wq=None, w_scale=None, stream=None):
    """W [K, N] -> (codes [N, K], the one scale float32 [1] = max|W| / Q)."""
    _, K, N = _mat(w, "w", _FLOAT_IN)
    q = _qtype(qtype)
    wq = _out(wq, "wq", (_code_dtype(q),) + _CODES, (N, K), w.device)
    w_scale = _out(w_scale, "w_scale", _F32, 1, w.device)
    _check("w8a8_quant_weight_tensor", _load().w8a8_quant_weight_tensor(
        _ptr(w), _dtype(w), K, N, q, _ptr(wq), _ptr(w_scale), _stream(stream)))
    return wq, w_scale


def w8a8_gemm_dequant_tensor(xq, x_scale, wq, w_scale, qtype="fp8", y=None, stream=None):
    """Quantized GEMM + dequantize with one scale per operand: Y bfloat16 [M, N]."""
    M, N, K = _gemm_operands(xq, wq)
    _arg(x_scale, "x_scale", _F32, 1)
    _arg(w_scale, "w_scale", _F32, 1)
    q = _qtype(qtype)
    y = _out(y, "y", (torch.bfloat16,), (M, N), xq.device)
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
    _, M, K = _mat(x, "x", (torch.bfloat16,))
    _, N, K2 = _mat(wq, "wq", (torch.int8,))
    if K2 != K:
        raise ValueError("x is [M, K] and wq is [N, K]")
    _arg(w_scale, "w_scale", _F32, N)
    y = _out(y, "y", (torch.bfloat16,), (M, N), x.device)
    _check("w8a8_gemm_w8a16", _load().w8a8_gemm_w8a16(_ptr(x), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(y),
                                                      _stream(stream)))
    return y


# ---- RMS norm with the smoothing folded into its gain ----------------------------------------------

def w8a8_fold_norm_gain(g, s, out=None, stream=None):
    """g' = g / s (either may be None = 1): float32 [K]."""
    ref = g if g is not None else s
    if ref is None:
        raise ValueError("w8a8_fold_norm_gain needs g or s")
    K = _arg(ref, "g" if g is not None else "s", _F32).numel()
    _arg(g, "g", _F32, K)
    _arg(s, "s", _F32, K)
    out = _out(out, "out", _F32, K, ref.device)
    _check("w8a8_fold_norm_gain", _load().w8a8_fold_norm_gain(_ptr(g), _ptr(s), K, _ptr(out), _stream(stream)))
    return out


def w8a8_norm_quant_act(h, g=None, eps: float = 1e-5, qtype="int8", xq=None, x_scale=None, stream=None):
    """RMS norm of h [M, K] with gain g (1/s folded in), then per-token quantize:
    (codes [M, K], scales float32 [M])."""
    _, M, K = _mat(h, "h", _FLOAT_IN)
    _arg(g, "g", _F32, K)
    q = _qtype(qtype)
    xq = _out(xq, "xq", (_code_dtype(q),) + _CODES, (M, K), h.device)
    x_scale = _out(x_scale, "x_scale", _F32, M, h.device)
    _check("w8a8_norm_quant_act", _load().w8a8_norm_quant_act(
        _ptr(h), _dtype(h), M, K, _ptr(g), float(eps), q, _ptr(xq), _ptr(x_scale), _stream(stream)))
    return xq, x_scale


def w8a8_layer_norm_quant_act(h, g=None, b=None, eps: float = 1e-5, qtype="int8", xq=None, x_scale=None,
                              stream=None):
    """LayerNorm of h [M, K] with gain g and bias b (1/s folded into both), then per-token
    quantize: (codes [M, K], scales float32 [M])."""
    _, M, K = _mat(h, "h", _FLOAT_IN)
    _arg(g, "g", _F32, K)
    _arg(b, "b", _F32, K)
    q = _qtype(qtype)
    xq = _out(xq, "xq", (_code_dtype(q),) + _CODES, (M, K), h.device)
    x_scale = _out(x_scale, "x_scale", _F32, M, h.device)
    _check("w8a8_layer_norm_quant_act", _load().w8a8_layer_norm_quant_act(
        _ptr(h), _dtype(h), M, K, _ptr(g), _ptr(b), float(eps), q, _ptr(xq), _ptr(x_scale), _stream(stream)))
    return xq, x_scale
