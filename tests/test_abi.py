"""The C ABI on the host: the library loads, exports every entry point that include/w8a8.h
declares, and rejects bad arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_path():
    names = declared_functions()
    for fn in ("w8a8_smooth_scales", "w8a8_fold_quant_weight", "w8a8_quant_act", "w8a8_smooth_quant",
               "w8a8_gemm_dequant",
               "w8a8_gemm_i32", "w8a8_status_string", "w8a8_version"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    import fp8_gemm_amd
    out = subprocess.run(["nm", "-D", "--defined-only", fp8_gemm_amd.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (w8a8_\w+)", out))
    assert set(declared_functions()) <= exported
    assert all(n.startswith("w8a8_") for n in exported)   # nothing else leaks with default visibility
    lib = ctypes.CDLL(fp8_gemm_amd.lib_path())
    for fn in declared_functions():
        assert hasattr(lib, fn)


def test_binding_names_match_c_entry_points():
    import fp8_gemm_amd
    for fn in declared_functions():
        assert callable(getattr(fp8_gemm_amd, fn)), fn


def test_status_strings_and_version():
    import fp8_gemm_amd as f
    assert f.w8a8_status_string(0) == "ok"
    assert "invalid" in f.w8a8_status_string(1)
    assert "unsupported" in f.w8a8_status_string(2)
    assert f.w8a8_status_string(99) == "unknown status"
    assert "gfx950" in f.w8a8_version()


def test_argument_validation_without_gpu():
    """Every rejection happens on the host before any HIP call."""
    import fp8_gemm_amd as f
    L = f._load()
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x100004)           # not 16-byte aligned
    INV, UNS, OK = f.W8A8_ERR_INVALID_ARG, f.W8A8_ERR_UNSUPPORTED, f.W8A8_OK
    # quant_act
    assert L.w8a8_quant_act(None, 1, 4, 16, None, 0, None, None, None) == INV       # NULL x
    assert L.w8a8_quant_act(fake, 7, 4, 16, None, 0, fake, fake, None) == INV       # bad dtype
    assert L.w8a8_quant_act(fake, 1, 4, 16, None, 5, fake, fake, None) == INV       # bad qtype
    assert L.w8a8_quant_act(fake, 1, -1, 16, None, 0, fake, fake, None) == INV      # negative M
    assert L.w8a8_quant_act(fake, 1, 4, 0, None, 0, fake, fake, None) == INV        # K = 0
    assert L.w8a8_quant_act(fake, 1, 4, 24, None, 0, fake, fake, None) == UNS       # K % 16
    assert L.w8a8_quant_act(odd, 1, 4, 16, None, 0, fake, fake, None) == UNS        # alignment
    assert L.w8a8_quant_act(None, 1, 0, 16, None, 0, None, None, None) == OK        # M = 0: no-op
    # smooth_scales
    assert L.w8a8_smooth_scales(fake, 1, 4, 16, fake, 1, 8, 1.5, fake, fake, 0, fake, None) == INV
    assert L.w8a8_smooth_scales(fake, 1, 4, 16, fake, 1, 8, -0.1, fake, fake, 0, fake, None) == INV
    assert L.w8a8_smooth_scales(fake, 1, 4, 16, fake, 1, 8, float("nan"), fake, fake, 0, fake, None) == INV
    assert L.w8a8_smooth_scales(fake, 1, 4, 16, fake, 1, 8, 0.5, None, fake, 0, fake, None) == INV
    # smooth_quant (x, xt, M, K, w, wt, N, alpha, qtype, ax, aw, s, wq, w_scale, xq, x_scale, stream)
    assert L.w8a8_smooth_quant(fake, 1, 4, 16, fake, 1, 8, 2.0, 0, fake, fake, fake, fake, fake, fake, fake,
                               None) == INV                                             # alpha > 1
    assert L.w8a8_smooth_quant(fake, 1, 4, 16, fake, 1, 8, 0.5, 4, fake, fake, fake, fake, fake, fake, fake,
                               None) == INV                                             # bad qtype
    assert L.w8a8_smooth_quant(fake, 1, 4, 16, fake, 1, 8, 0.5, 0, fake, fake, None, fake, fake, fake, fake,
                               None) == INV                                             # NULL s
    assert L.w8a8_smooth_quant(fake, 1, 4, 16, fake, 1, 8, 0.5, 0, fake, fake, fake, None, fake, fake, fake,
                               None) == INV                                             # NULL wq
    assert L.w8a8_smooth_quant(fake, 1, 4, 16, fake, 1, 8, 0.5, 0, fake, fake, fake, fake, fake, None, fake,
                               None) == INV                                             # NULL xq
    assert L.w8a8_smooth_quant(fake, 1, 4, 40, fake, 1, 8, 0.5, 0, fake, fake, fake, fake, fake, fake, fake,
                               None) == UNS                                             # K % 16
    assert L.w8a8_smooth_quant(fake, 1, 4, 16, fake, 1, 8, 0.5, 0, fake, fake, fake, odd, fake, fake, fake,
                               None) == UNS                                             # alignment
    # fold
    assert L.w8a8_fold_quant_weight(None, 1, 16, 8, None, 0, fake, fake, None) == INV
    assert L.w8a8_fold_quant_weight(fake, 1, 16, 0, None, 0, None, None, None) == OK
    # gemm
    assert L.w8a8_gemm_dequant(fake, fake, fake, fake, 0, 4, 4, 32, None, None) == INV
    assert L.w8a8_gemm_dequant(fake, fake, fake, fake, 2, 4, 4, 32, fake, None) == INV
    assert L.w8a8_gemm_dequant(None, None, None, None, 0, 0, 5, 32, None, None) == OK
    assert L.w8a8_gemm_i32(fake, fake, 4, 4, 133152, fake, None) == UNS              # int32 overflow bound
    assert L.w8a8_gemm_i32(fake, fake, 4, 4, 40, fake, None) == UNS
    # per-tensor entry points
    other = ctypes.c_void_p(0x200000)
    assert L.w8a8_absmax(fake, 1, 16, None, 0, None) == INV                          # NULL amax
    assert L.w8a8_absmax(fake, 1, 12, fake, 0, None) == UNS                          # n % 8
    assert L.w8a8_absmax(fake, 1, -8, fake, 0, None) == INV
    assert L.w8a8_quant_act_tensor(fake, 1, 4, 16, fake, 1, fake, other, fake, 0, None) == INV  # amax_out is amax_in
    assert L.w8a8_quant_act_tensor(fake, 1, 4, 16, None, 1, fake, other, None, 0, None) == INV  # NULL amax_in
    assert L.w8a8_quant_act_tensor(fake, 1, 4, 24, fake, 1, fake, other, None, 0, None) == UNS  # K % 16
    assert L.w8a8_quant_act_tensor(fake, 1, 4, 16, fake, 3, fake, other, None, 0, None) == INV  # bad qtype
    assert L.w8a8_quant_weight_tensor(fake, 1, 16, 8, 1, fake, None, None) == INV    # NULL w_scale
    assert L.w8a8_quant_weight_tensor(odd, 1, 16, 8, 1, fake, other, None) == UNS    # alignment
    assert L.w8a8_gemm_dequant_tensor(fake, fake, fake, fake, 1, 4, 4, 32, None, None) == INV
    assert L.w8a8_gemm_dequant_tensor(None, None, None, None, 1, 4, 0, 32, None, None) == OK
    # fused norm + quantize
    L.w8a8_norm_quant_act.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert L.w8a8_norm_quant_act(fake, 1, 4, 16, None, -1.0, 0, fake, fake, None) == INV    # eps < 0
    assert L.w8a8_norm_quant_act(fake, 1, 4, 16, None, float("nan"), 0, fake, fake, None) == INV
    assert L.w8a8_norm_quant_act(fake, 1, 4, 8208, None, 1e-5, 0, fake, fake, None) == UNS  # K > 8192
    assert L.w8a8_norm_quant_act(None, 1, 0, 16, None, 1e-5, 0, None, None, None) == OK     # M = 0
    assert L.w8a8_fold_norm_gain(None, None, 0, fake, None) == INV                          # K = 0
    L.w8a8_layer_norm_quant_act.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 16, None, None, -1.0, 0, fake, fake, None) == INV   # eps < 0
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 16, None, None, 1e-5, 2, fake, fake, None) == INV   # bad qtype
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 8208, None, None, 1e-5, 0, fake, fake, None) == UNS  # K > 8192
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 16, None, odd, 1e-5, 0, fake, fake, None) == UNS    # bias alignment
    assert L.w8a8_layer_norm_quant_act(None, 1, 0, 16, None, None, 1e-5, 0, None, None, None) == OK   # M = 0


def test_product_path_does_not_touch_the_oracle():
    """The GPU library and its binding never import, link or read the CPU oracle."""
    pkg = os.path.join(ROOT, "fp8_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, fn)
    import fp8_gemm_amd
    out = subprocess.run(["ldd", fp8_gemm_amd.lib_path()], capture_output=True, text=True).stdout
    assert "oracle" not in out
