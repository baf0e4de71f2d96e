"""Argument validation of the C ABI, callable without a GPU and without torch.

Every rejection of include/w8a8.h happens on the host before any HIP call, so these cases run
anywhere the library loads: in test_abi.py against the built library, and as a script against a
build whose host code carries the address and undefined-behaviour sanitizers
(``python tests/abi_cases.py <library>``, run by test_sanitizers.py).
"""
import ctypes
import importlib.util
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location(
    "w8a8_cabi", os.path.join(os.path.dirname(HERE), "fp8_gemm_amd", "_cabi.py"))
_cabi = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_cabi)
W8A8_OK, W8A8_ERR_INVALID_ARG, W8A8_ERR_UNSUPPORTED = _cabi.W8A8_OK, _cabi.W8A8_ERR_INVALID_ARG, _cabi.W8A8_ERR_UNSUPPORTED


def check_argument_validation(L):
    """L: the library with its signatures declared (fp8_gemm_amd._cabi.load)."""
    fake = ctypes.c_void_p(0x100000)          # never dereferenced: validation fails first
    odd = ctypes.c_void_p(0x100004)           # not 16-byte aligned
    INV, UNS, OK = W8A8_ERR_INVALID_ARG, W8A8_ERR_UNSUPPORTED, W8A8_OK
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
    # quant_pair (x, xt, M, K, w, wt, N, s, w_scale, qtype, xq, x_scale, wq, stream)
    assert L.w8a8_quant_pair(fake, 1, 4, 16, fake, 1, 8, None, fake, 0, fake, fake, fake, None) == INV     # NULL s
    assert L.w8a8_quant_pair(fake, 1, 4, 16, fake, 1, 8, fake, None, 0, fake, fake, fake, None) == INV     # NULL w_scale
    assert L.w8a8_quant_pair(fake, 1, 4, 16, fake, 9, 8, fake, fake, 0, fake, fake, fake, None) == INV     # bad dtype
    assert L.w8a8_quant_pair(fake, 1, 4, 16, fake, 1, 8, fake, fake, 3, fake, fake, fake, None) == INV     # bad qtype
    assert L.w8a8_quant_pair(fake, 1, 4, 24, fake, 1, 8, fake, fake, 0, fake, fake, fake, None) == UNS     # K % 16
    assert L.w8a8_quant_pair(fake, 1, 4, 16, fake, 1, 8, fake, fake, 0, fake, fake, odd, None) == UNS      # alignment
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
    assert L.w8a8_norm_quant_act(fake, 1, 4, 16, None, -1.0, 0, fake, fake, None) == INV    # eps < 0
    assert L.w8a8_norm_quant_act(fake, 1, 4, 16, None, float("nan"), 0, fake, fake, None) == INV
    assert L.w8a8_norm_quant_act(fake, 1, 4, 8208, None, 1e-5, 0, fake, fake, None) == UNS  # K > 8192
    assert L.w8a8_norm_quant_act(None, 1, 0, 16, None, 1e-5, 0, None, None, None) == OK     # M = 0
    assert L.w8a8_fold_norm_gain(None, None, 0, fake, None) == INV                          # K = 0
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 16, None, None, -1.0, 0, fake, fake, None) == INV   # eps < 0
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 16, None, None, 1e-5, 2, fake, fake, None) == INV   # bad qtype
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 8208, None, None, 1e-5, 0, fake, fake, None) == UNS  # K > 8192
    assert L.w8a8_layer_norm_quant_act(fake, 1, 4, 16, None, odd, 1e-5, 0, fake, fake, None) == UNS    # bias alignment
    assert L.w8a8_layer_norm_quant_act(None, 1, 0, 16, None, None, 1e-5, 0, None, None, None) == OK   # M = 0
    # status strings of every code and of an unknown one
    for st in (0, 1, 2, 3, 99):
        assert L.w8a8_status_string(st)
    assert L.w8a8_version().startswith(b"libw8a8")


if __name__ == "__main__":
    check_argument_validation(_cabi.load(sys.argv[1]))
    print("abi cases ok")
