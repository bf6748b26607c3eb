"""Block-scaled FP8 attention reference (oracle; test infrastructure only).

What it computes, and where the pages define it.  The devin.kr article on
FLUX image generation accelerated on Blackwell ("Compute efficiency and
acceleration") lowers the cost of attention by running it in 8-bit floating
point with a per-token correction of the quantization error, for a 1.16-1.18x
speed-up.  The pages give no steps, so the following readings (the plainest
block-scaled FP8 attention consistent with the rest of the pages' microscaling
recipe) define the method, for one head with queries Q [Sq, D], keys K [Skv, D]
and values V [Skv, Dv]:

  1. Q and K are MXFP8-quantized along the head dimension D (E4M3 codes, one
     E8M0 scale per 32 channels of each token): the per-token scales correct
     each token's range (aitrends.kr MXFP8/NVFP4 article, Glossary
     "Microscaling Formats" and "MXFP8", for the format);
  2. V is MXFP8-quantized along the token axis (one E8M0 scale per 32
     consecutive tokens of each channel), the contraction axis of P V;
  3. scores s = Q^ K^T / sqrt(D) from the dequantized operands, exactly;
  4. the plain softmax numerator p = exp(s - m) with m the exact maximum of
     the query's scores over all keys, so 0 < p <= 1 and the largest p is 1;
  5. p is E4M3-quantized with the fixed scale 2**8 (p * 256 <= 256 < 448, so
     never saturated), and P^ V^ is accumulated;
  6. the row sum l is that of the unquantized p; the output is (P^ V^) / l.

No key tiling enters the definition: every P code depends only on its own
score and the row's maximum.  Everything is float64; the only approximations
are the format encodings the method itself applies (steps 1, 2, 5) and
float64 summation.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import E4M3, decode_e4m3, encode
from .quant import MXFP8, dequant_mx, quantize_mx

P_SCALE_EXP = 8  # P in (0, 1] is encoded as E4M3(p * 2**8)


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Textbook softmax attention softmax(q k^T / sqrt(D)) v in float64, one head ([S, D] arrays)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    s = q @ k.T / math.sqrt(q.shape[1])
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def quantize_qkv(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray):
    """Steps 1-2: MXFP8 quantization of one head's bf16 Q, K (along D) and V (along tokens).

    Returns dict with the codes and scales in the library's layouts (Q, K: [S, D] codes and
    [S, D/32] scales; V as V^T: [D, Skv] codes and [D, Skv/32] scales) and the dequantized
    float64 operands q, k, v ([S, D] each)."""
    qc, qs = quantize_mx(q_bits, MXFP8)
    kc, ks = quantize_mx(k_bits, MXFP8)
    vtc, vts = quantize_mx(np.ascontiguousarray(np.asarray(v_bits).T), MXFP8)
    return {
        "q_codes": qc, "q_scales": qs, "k_codes": kc, "k_scales": ks, "vt_codes": vtc, "vt_scales": vts,
        "q": dequant_mx(qc, qs, MXFP8), "k": dequant_mx(kc, ks, MXFP8), "v": dequant_mx(vtc, vts, MXFP8).T,
    }


def quantize_p(p: np.ndarray) -> np.ndarray:
    """Step 5: p in [0, 1] -> dec_E4M3(RNE(p * 2**8)) / 2**8."""
    return decode_e4m3(encode(E4M3, np.ldexp(p, P_SCALE_EXP))) * 2.0 ** -P_SCALE_EXP


def softmax_numerators(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Steps 3-4: p = exp(s - max over all keys of s), s = q k^T / sqrt(D); [Sq, Skv] float64."""
    s = (q @ k.T) / math.sqrt(q.shape[1])
    return np.exp(s - s.max(axis=1, keepdims=True))


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, quantize_probs: bool = True) -> np.ndarray:
    """Steps 3-6 on the dequantized float64 operands of one head; with quantize_probs=False, step 5 is
    left out (plain softmax attention of the dequantized operands)."""
    p = softmax_numerators(q, k)
    ph = quantize_p(p) if quantize_probs else p
    return (ph @ v) / p.sum(axis=1, keepdims=True)


def attention_fp8_ref(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, rows=None) -> np.ndarray:
    """The block-scaled FP8 attention of one head from bf16 bit patterns [S, D]; float64 [Sq, D].

    `rows` (optional) restricts the output to those query rows (each row is independent)."""
    t = quantize_qkv(q_bits, k_bits, v_bits)
    q = t["q"] if rows is None else t["q"][np.asarray(rows)]
    return attend(q, t["k"], t["v"], True)


# E4M3 values >= 0 in increasing order (for the neighbours of a midpoint)
_E4M3_GRID = np.unique(decode_e4m3(np.arange(0x7F)))
_E4M3_MIDS = (_E4M3_GRID[1:] + _E4M3_GRID[:-1]) / 2


def _ambiguous(q: np.ndarray, k: np.ndarray, score_eta: float, exp_eta: float):
    """For every (query, key): p, whether p * 2^8 lies within the floating-point error bound of an E4M3
    midpoint, and the two E4M3 neighbours (lo, hi) of that nearest midpoint."""
    c = 1.0 / math.sqrt(q.shape[1])
    A = np.abs(q) @ np.abs(k).T
    # relative bound on p, per row: the score's error and that of the row maximum (each up to
    # c * score_eta * max_j A), plus the exponential and the scaling
    tol = c * score_eta * 2.0 * A.max(axis=1) + exp_eta
    p = softmax_numerators(q, k)
    x = np.ldexp(p, P_SCALE_EXP)
    i = np.clip(np.searchsorted(_E4M3_MIDS, x), 1, len(_E4M3_MIDS) - 1)
    mid = np.where(np.abs(_E4M3_MIDS[i - 1] - x) < np.abs(_E4M3_MIDS[i] - x), _E4M3_MIDS[i - 1], _E4M3_MIDS[i])
    idx = np.searchsorted(_E4M3_GRID, mid)
    near = np.abs(x - mid) <= x * tol[:, None]
    return p, near, _E4M3_GRID[idx - 1], _E4M3_GRID[idx]


def p_code_slack(q: np.ndarray, k: np.ndarray, v: np.ndarray, score_eta: float, exp_eta: float = 2.0 ** -20,
                 forced=None):
    """Bound of what a valid other rounding of near-midpoint P codes can change in the output.

    Step 5 rounds p * 2^8 to E4M3, a decision taken from floating-point scores.
    A kernel that forms each score in a float accumulator of unit roundoff u
    over D products errs by at most gamma_D sum_d |q_d k_d| with gamma_D about
    D u (the recursive-summation bound), in the score itself and in the row's
    maximum.  `score_eta` is that relative bound (D * 2^-24 for fp32 and
    D = 128); `exp_eta` covers the exponential and the scaling.  For each key
    whose p * 2^8 lies within the resulting relative distance of an E4M3
    midpoint, either neighbour is a correct code; the returned slack [Sq, Dv]
    sums, per output, one E4M3 step (divided by 2^8) times |v_j| divided by
    the row sum, over those keys.

    `forced` (optional, for checking the bound): a set of (row, key) pairs
    whose code is taken as the other neighbour of the nearest midpoint; the
    function then also returns the output computed with those codes.
    Returns (slack, out_forced or None)."""
    p, near, lo, hi = _ambiguous(q, k, score_eta, exp_eta)
    l = p.sum(axis=1)
    slack = ((near * (hi - lo) * 2.0 ** -P_SCALE_EXP) @ np.abs(v)) / l[:, None]
    if not forced:
        return slack, None
    ph = quantize_p(p)
    for (r, j) in forced:
        cur = ph[r, j] * 2.0 ** P_SCALE_EXP
        ph[r, j] = (hi[r, j] if cur == lo[r, j] else lo[r, j]) * 2.0 ** -P_SCALE_EXP
    return slack, (ph @ v) / l[:, None]


def near_midpoint_keys(q: np.ndarray, k: np.ndarray, score_eta: float, exp_eta: float = 2.0 ** -20):
    """The (row, key) pairs whose P code p_code_slack treats as ambiguous."""
    _, near, _, _ = _ambiguous(q, k, score_eta, exp_eta)
    return [(int(r), int(j)) for r, j in zip(*np.nonzero(near))]
