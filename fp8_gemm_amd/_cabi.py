"""The C ABI of libw8a8 as ctypes signatures (no torch): loads a build of the library and declares
every entry point of include/w8a8.h on it."""
from __future__ import annotations

import ctypes

W8A8_OK, W8A8_ERR_INVALID_ARG, W8A8_ERR_UNSUPPORTED, W8A8_ERR_HIP = 0, 1, 2, 3
W8A8_F32, W8A8_BF16 = 0, 1
W8A8_INT8, W8A8_FP8_E4M3 = 0, 1

_P, _I64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float

# name: (result type, argument types), in the order of include/w8a8.h
SIGNATURES = {
    "w8a8_smooth_scales": (_I, [_P, _I, _I64, _I64, _P, _I, _I64, _F, _P, _P, _I, _P, _P]),
    "w8a8_fold_quant_weight": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P]),
    "w8a8_quant_act": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P]),
    "w8a8_smooth_quant": (_I, [_P, _I, _I64, _I64, _P, _I, _I64, _F, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "w8a8_quant_pair": (_I, [_P, _I, _I64, _I64, _P, _I, _I64, _P, _P, _I, _P, _P, _P, _P]),
    "w8a8_gemm_dequant": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P]),
    "w8a8_gemm_i32": (_I, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_gemm_f32": (_I, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_absmax": (_I, [_P, _I, _I64, _P, _I, _P]),
    "w8a8_quant_act_tensor": (_I, [_P, _I, _I64, _I64, _P, _I, _P, _P, _P, _I, _P]),
    "w8a8_quant_weight_tensor": (_I, [_P, _I, _I64, _I64, _I, _P, _P, _P]),
    "w8a8_gemm_dequant_tensor": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _P, _P]),
    "w8a8_fold_norm_gain": (_I, [_P, _P, _I64, _P, _P]),
    "w8a8_norm_quant_act": (_I, [_P, _I, _I64, _I64, _P, _F, _I, _P, _P, _P]),
    "w8a8_layer_norm_quant_act": (_I, [_P, _I, _I64, _I64, _P, _P, _F, _I, _P, _P, _P]),
    "w8a8_gemm_w8a16": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "w8a8_status_string": (ctypes.c_char_p, [_I]),
    "w8a8_version": (ctypes.c_char_p, []),
}

ENTRY_POINTS = tuple(SIGNATURES)


def load(path: str) -> ctypes.CDLL:
    """Load the library at path and declare every entry point's signature on it."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib
