"""fp64 GEMM references and the comparison metric (oracle; test infrastructure only).

out[m, n] = sum_k A[m, k] * W[n, k] (+ bias[n]), i.e. out = A @ W^T with W
stored [N, K] as a linear layer's weight.  The quantized references multiply
the dequantized operands exactly as decoded from the oracle's own codes, so
the only approximation is float64 summation (relative error ~K * 2**-53).

The block-scaled product is what the low-precision GEMM of the aitrends.kr
MXFP8/NVFP4 article computes ("Section details": quantized weights and
dynamically quantized activations feeding the FP8/FP4 GEMM); the bf16 form
is the unquantized path kept for layers with min(M, K, N) < 1024 (same
article, second "Evidence" block).
"""

from __future__ import annotations

import numpy as np

from .formats import decode_bf16
from .quant import Scheme, dequant_mx, dequant_nvfp4


def _matmul_t(a: np.ndarray, w: np.ndarray, bias, row_chunk: int = 2048) -> np.ndarray:
    M = a.shape[0]
    out = np.empty((M, w.shape[0]), dtype=np.float64)
    wt = np.ascontiguousarray(w.T)
    for r0 in range(0, M, row_chunk):
        out[r0:r0 + row_chunk] = a[r0:r0 + row_chunk] @ wt
    if bias is not None:
        out += decode_bf16(np.asarray(bias, dtype=np.uint16))[None, :]
    return out


def gemm_mx_ref(a_codes, a_scales, w_codes, w_scales, scheme: Scheme, bias=None) -> np.ndarray:
    """fp64 reference of the MXFP8 / MXFP4 block-scaled GEMM."""
    return _matmul_t(dequant_mx(a_codes, a_scales, scheme), dequant_mx(w_codes, w_scales, scheme), bias)


def gemm_nvfp4_ref(a_codes, a_scales, a_ts, w_codes, w_scales, w_ts, bias=None) -> np.ndarray:
    """fp64 reference of the NVFP4 GEMM: both per-tensor scales are folded into the operands."""
    return _matmul_t(dequant_nvfp4(a_codes, a_scales, a_ts), dequant_nvfp4(w_codes, w_scales, w_ts), bias)


def gemm_bf16_ref(a_bits, w_bits, bias=None) -> np.ndarray:
    """fp64 reference of the bf16 GEMM (inputs as bf16 bit patterns)."""
    return _matmul_t(decode_bf16(a_bits), decode_bf16(w_bits), bias)


def normwise_error(y: np.ndarray, r: np.ndarray) -> float:
    """max_i |y_i - r_i| / max_i |r_i|; infinite if y holds NaN or Inf.

    Elementwise relative error is unbounded where r cancels to ~0, so the
    gate is normwise: the bf16 output rounding alone contributes up to
    2**-9 = 1.953e-3 of max|r|.
    """
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    denom = float(np.abs(r).max()) if r.size else 0.0
    num = float(np.abs(y - r).max()) if r.size else 0.0
    if denom == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / denom
