"""The CPU oracle and the library's host code under the address and undefined-behaviour sanitizers.

- The oracle is rebuilt with gcc's sanitizers and its pin tests (test_oracle_pins.py,
  test_oracle_tensor.py) run against that build in a child process (W8A8_ORACLE_LIB selects it).
- The library is rebuilt with the sanitizers on its host code (argument validation, launch
  set-up; the gfx950 code is unchanged) and the argument-validation cases of the C ABI run against
  it in a child process without torch (tests/abi_cases.py); no GPU call is made.
- A planted out-of-bounds read, built with the oracle's sanitizer flags, must be caught: the
  sanitizer set-up itself is checked, not only that nothing was reported.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def child_env(preload, **extra):
    env = dict(os.environ)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.update(extra)
    return env


def test_sanitizer_catches_a_planted_error(tmp_path):
    from oracle.build import SANITIZE
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int main(int argc, char** argv) { int* a = malloc(4 * sizeof(int));\n"
                   "  int v = a[argc + 3]; free(a); return v; }\n")
    exe = tmp_path / "planted"
    subprocess.run(["gcc", *SANITIZE, str(src), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=child_env(""))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def test_oracle_pins_under_sanitizers(tmp_path):
    from oracle.build import SANITIZE, build
    lib = build(path=str(tmp_path / "liboracle_san.so"), extra=SANITIZE)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_tensor.py")],
                       capture_output=True, text=True, cwd=ROOT,
                       env=child_env(gcc_runtime("libasan.so"), W8A8_ORACLE_LIB=lib))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert " passed" in r.stdout


def test_abi_validation_under_sanitizers(tmp_path):
    runtime = clang_asan_runtime()
    if runtime is None:
        pytest.skip("no clang address-sanitizer runtime in this ROCm install")
    from fp8_gemm_amd.build import HOST_SANITIZE, build
    lib = build(path=str(tmp_path / "libw8a8_san.so"), obj_dir=str(tmp_path / "obj"), extra=HOST_SANITIZE)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_cases.py"), lib],
                       capture_output=True, text=True, env=child_env(runtime))
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "abi cases ok" in r.stdout
