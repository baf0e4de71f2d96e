"""Host <-> device transfers for the GPU tests (numpy arrays as stored <-> torch GPU tensors)."""
import sys

import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """float32 -> float32, uint16 (bf16 bits) -> bfloat16, int8/uint8 codes as is."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def announce(msg: str):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def assert_rel_tol(y_bits: np.ndarray, ref64: np.ndarray, rtol: float = 1e-2, extra=None):
    """Elementwise |y - ref| <= rtol * |ref| (+ extra); zeros of ref must be exact zeros."""
    y = bf16_to_f64(y_bits)
    bound = rtol * np.abs(ref64)
    if extra is not None:
        bound = bound + extra
    err = np.abs(y - ref64)
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} outputs out of tolerance; first at {tuple(i)}: "
                             f"y={y[tuple(i)]!r} ref={ref64[tuple(i)]!r} bound={bound[tuple(i)]!r}")


# Accumulation error of the E4M3 matrix-core GEMM (v_mfma_f32_16x16x128_f8f6f4), from the
# arithmetic pinned by test_gpu_edges.py::test_fp8_accumulator_arithmetic: products of 8
# consecutive K positions are summed in a fixed-point window about 13 bits below the block's
# largest product (smaller parts truncated toward zero), and block sums are accumulated in fp32
# with round-to-nearest-even.  Per block the error is below 7 * 2^-12 * max|p| <= 7 * 2^-12 *
# sum|p|; the fp32 accumulation of K/8 block sums adds at most (K/8) * 2^-24 * sum|p|.
def fp8_accumulation_bound(K: int, mag64):
    """Worst-case |acc - exact| (scaled like mag64 = sum_k |products| * sx * sw)."""
    return (7.0 * 2.0 ** -12 + (K / 8.0 + 1.0) * 2.0 ** -24) * mag64 * 1.01
