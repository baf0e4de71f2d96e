"""bench.py's host logic (no GPU): the one-GPU refusal, the algorithmic byte counts the rooflines
divide by, and the GEMM kernel name it reports for each workload (a mirror of the library's
dispatch)."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_prefill_calls():
    wl = synth.workload("prefill_2048x4096x4096_int8")
    M, K, N = wl.M, wl.K, wl.N
    b = bench.stage_bytes(wl)
    # GEMM: both code matrices read once, both scale vectors, the bf16 output written once.
    assert b["gemm_dequant"] == M * K + N * K + 4 * M + 4 * N + 2 * M * N == 41967616
    # Activation quantize: bf16 X read, codes and one scale per row written, s read.
    assert b["quant_act"] == 2 * M * K + M * K + 4 * M + 4 * K
    # Paired quantize: X and W read, both code matrices written, s and the weight scales read.
    assert b["quant_pair"] == 2 * M * K + 2 * K * N + M * K + K * N + 4 * M + 4 * K + 4 * N == 75538432
    # The forced passes of the one-call preparation: X twice, W three times.
    p = bench.stage_pass_bytes(wl)
    assert p["smooth_quant"] - b["smooth_quant"] == 2 * M * K + 2 * 2 * K * N


def test_gemm_kernel_names_follow_the_dispatch():
    name = lambda w: bench.gemm_kernel_name(synth.workload(w).M, synth.workload(w).N, synth.workload(w).K,
                                           synth.workload(w).qtype)
    assert name("decode_16x4096x14336_int8") == "gemm_decode_lds_kernel"
    assert name("prefill_2048x4096x4096_int8") == "gemm_tile_kernel"
    assert name("large_8192x8192x28672_fp8") == "gemm_tile_kernel"
    assert bench.gemm_kernel_name(16, 4096, 8192, "fp8_e4m3") == "gemm_decode_kernel"
    assert bench.gemm_kernel_name(30, 4096, 4096, "int8") == "gemm_small_m_kernel"
