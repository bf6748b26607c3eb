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

from .formats import decode_bf16, floor_log2
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


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2 / pi) (x + 0.044715 x^3))), in fp64.

    The activation between a DiT MLP's up- and down-projections (wavespeed.ai
    "WaveSpeedAI X DataCrunch: FLUX real-time image inference on B200", model
    overview: the MLP of each transformer block); the tanh form is a reading,
    the one FLUX's MLP uses.  Applied to the fp64 GEMM reference when checking
    the GEMM epilogue that quantizes act(y) for the next layer.
    """
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x * x * x)))


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


def bf16_round(r: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits: the step is 2**(floor(log2|r|) - 7) for
    normal magnitudes and 2**-133 below 2**-126.  Overflow is not expected
    from these GEMMs and raises.
    """
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    e = np.where(a == 0, -126, np.maximum(floor_log2(np.where(a == 0, 1.0, a)), -126))
    step_exp = e - 7
    q = np.rint(np.ldexp(a, -step_exp))
    out = np.copysign(np.ldexp(q, step_exp), r)
    if np.any(np.abs(out) > 3.3895313892515355e38):
        raise OverflowError("value beyond the bf16 range")
    return out


def bf16_half_ulp(y: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at bf16 values y: 2**(floor(log2|y|) - 8), or 2**-134 below 2**-126."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.where(a == 0, -126, np.maximum(floor_log2(np.where(a == 0, 1.0, a)), -126))
    return np.ldexp(1.0, e - 8)


def gemm_error(y: np.ndarray, r: np.ndarray) -> float:
    """Normwise error of a bf16 GEMM result beyond its own output rounding.

    max_i max(|y_i - r_i| - halfulp_bf16(y_i), 0) / max_i |r_i|.  A result y_i
    obtained by rounding an accumulator a_i to bf16 satisfies
    |y_i - a_i| <= halfulp(y_i), so this bounds the accumulator's error
    |a_i - r_i|.  The output rounding itself may reach 2**-8 of max|r|
    (8 significant bits), which is why it is separated from the 2e-3 gate.
    Infinite if y holds NaN or Inf.
    """
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    if r.size == 0:
        return 0.0
    denom = float(np.abs(r).max())
    excess = np.maximum(np.abs(y - r) - bf16_half_ulp(y), 0.0)
    num = float(excess.max())
    if denom == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / denom


def gemm_error_rows(y: np.ndarray, r: np.ndarray) -> float:
    """gemm_error applied to each row against that row's own max|r|, maximised over the rows.

    The normwise gate divides by the largest |r| of the whole matrix, so an
    error confined to rows of small magnitude (rows scaled by exp(N(0, 0.5)),
    or outside the outlier channels) can hide under it; here each row answers
    for itself.  A row whose reference is all zeros passes only if its outputs
    are within their own rounding of zero.  Infinite if y holds NaN or Inf.
    """
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    if r.size == 0:
        return 0.0
    r2 = r.reshape(r.shape[0], -1)
    excess = np.maximum(np.abs(y - r) - bf16_half_ulp(y), 0.0).reshape(r2.shape)
    num = excess.max(axis=1)
    den = np.abs(r2).max(axis=1)
    if np.any((den == 0.0) & (num > 0.0)):
        return float("inf")
    ok = den > 0.0
    return float((num[ok] / den[ok]).max()) if np.any(ok) else 0.0


def rounding_mismatch_rate(y: np.ndarray, r: np.ndarray, rel: float = 1.0 / 16) -> float:
    """Fraction of the outputs with |r_i| >= rel * max|r| whose bf16 value differs from bf16_round(r_i).

    A correctly rounding fp32-accumulating kernel differs only where r_i lies
    within its accumulation error of a rounding midpoint; a truncating or
    double-rounding epilogue differs on a large fraction.
    """
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    sel = np.abs(r) >= rel * np.abs(r).max()
    if not np.any(sel):
        return 0.0
    return float(np.mean(y[sel] != bf16_round(r[sel])))
