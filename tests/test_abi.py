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
    from abi_cases import check_argument_validation
    check_argument_validation(f._load())


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
