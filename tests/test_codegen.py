"""Checks of the generated gfx950 code of the GEMM (no GPU; compiles gemm.hip to assembly).

The tiled GEMM's copies into LDS are written as inline assembly that sets M0 (the LDS address of
the copy) right before each global_load_lds_dwordx4.  The compiler reserves M0 and does not
preserve it around such asm, so correctness needs that nothing else in these kernels uses M0: no
other write of it, and none of the instructions that read it implicitly (relative register
moves, messages, GWS / ordered-count / add-TID LDS operations, interpolation, LDS-direct reads).
This test compiles gemm.hip with the library's flags and checks every GEMM kernel's code.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

IMPLICIT_M0 = re.compile(r"\b(s_movrel\w*|v_movrel\w*|s_sendmsg\w*|ds_gws\w*|ds_ordered_count|\w+_addtid\w*|"
                         r"v_interp\w*|lds_direct|lds_param_load|s_set_gpr_idx\w*)\b")


def kernel_bodies(asm):
    """{kernel symbol: [instruction lines]} for every GEMM kernel in an assembly listing."""
    out, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w*gemm\w*kernel\w*):", line)
        if m:
            name = m.group(1)
            out[name] = []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            name = None
            continue
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            out[name].append(s)
    return out


def test_m0_only_in_the_lds_copy_sequence(tmp_path):
    from fp8_gemm_amd.build import ARCH, CSRC, HIPCC_FLAGS, hipcc
    out = tmp_path / "gemm.s"
    flags = [f for f in HIPCC_FLAGS if f != "-fPIC"]
    subprocess.run([hipcc(), *flags, "--offload-device-only", "-S", os.path.join(CSRC, "gemm.hip"), "-o", str(out)],
                   check=True, capture_output=True)
    bodies = kernel_bodies(out.read_text())
    tiled = [k for k in bodies if "gemm_tile_kernel" in k]
    assert tiled, "no tiled GEMM kernel found in the assembly"
    assert m0_violations(bodies) == []
    copies = sum(1 for ins in bodies.values() for s in ins if re.fullmatch(r"s_mov_b32 m0, s\d+", s))
    assert copies > 0


def m0_violations(bodies):
    """The rule of test_m0_only_in_the_lds_copy_sequence as a function returning violations."""
    bad = []
    for name, ins in bodies.items():
        for i, s in enumerate(ins):
            if IMPLICIT_M0.search(s):
                bad.append(s)
            elif re.search(r"\bm0\b", s) and not (re.fullmatch(r"s_mov_b32 m0, s\d+", s) and i + 1 < len(ins)
                                                  and ins[i + 1].startswith("global_load_lds_dwordx4")):
                bad.append(s)
            elif s.startswith("global_load_lds") and not (i > 0 and re.fullmatch(r"s_mov_b32 m0, s\d+", ins[i - 1])):
                bad.append(s)
    return bad


def test_m0_checker_catches_planted_uses():
    good = ("_Z16gemm_tile_kernelv:\n\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v1, s[2:3]\n"
            "\tv_mfma_i32_32x32x32_i8 a[0:15], v[2:5], v[6:9], a[0:15]\n.Lfunc_end0:\n")
    assert m0_violations(kernel_bodies(good)) == []
    planted = [good.replace("\tv_mfma", "\ts_movrels_b32 s0, s1\n\tv_mfma"),
               good.replace("\tv_mfma", "\ts_mov_b32 s9, m0\n\tv_mfma"),
               good.replace("s_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v1, s[2:3]",
                            "global_load_lds_dwordx4 v1, s[2:3]\n\ts_mov_b32 m0, s4"),
               good.replace("\tv_mfma", "\ts_sendmsg sendmsg(MSG_DEALLOC_VGPRS)\n\tv_mfma")]
    for p in planted:
        assert m0_violations(kernel_bodies(p)), p
