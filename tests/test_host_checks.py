"""Host-side checks of device arithmetic and of the C header (no GPU).

- The quantize kernels' five-operation division (div_by_rcp in fp8_gemm_amd/csrc/device.h, the
  same source the kernels compile, built here for the host) equals IEEE binary32 division bit for
  bit on 10^9 random pairs plus adversarial and edge pairs inside the guarded ranges.  The kernels
  pass it the correctly rounded reciprocal, as the host does with 1.0f / b, and the remaining
  operations are fused multiply-adds, which are correctly rounded on both.
  ("Weight-Activation Quantization", section 3: activation channels are divided by their
  smoothing factors; section 2: values are divided by their scales.)
- include/w8a8.h compiles as C99 (the boundary is a C ABI).
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


def test_div_by_rcp_equals_ieee_division(tmp_path):
    exe = tmp_path / "div_by_rcp_check"
    subprocess.run([HIPCC, "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off",
                    f"-I{os.path.join(ROOT, 'fp8_gemm_amd', 'csrc')}",
                    os.path.join(ROOT, "tests", "host", "div_by_rcp_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe), "1000000000", "20241203"], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    counts = dict(zip(r.stdout.split()[0::2], map(int, r.stdout.split()[1::2])))
    assert counts["mismatches"] == 0
    assert counts["random"] >= 900_000_000 and counts["adversarial"] > 1_000_000 and counts["edge"] > 1_000_000


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use_header.c"
    src.write_text('#include "w8a8.h"\n'
                   "int main(void) {\n"
                   "  w8a8_dtype d = W8A8_BF16; w8a8_qtype q = W8A8_FP8_E4M3; w8a8_status s = W8A8_OK;\n"
                   "  return (int)d + (int)q + (int)s - 2;\n}\n")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror=implicit-function-declaration", "-D__HIP_PLATFORM_AMD__",
                    f"-I{os.path.join(ROOT, 'include')}", "-I/opt/rocm/include", str(src), "-o",
                    str(tmp_path / "use_header")], check=True, capture_output=True)
    assert subprocess.run([str(tmp_path / "use_header")]).returncode == 0
