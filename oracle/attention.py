"""Block-scaled FP8 attention reference (oracle; test infrastructure only).

What it computes, and where the pages define it.  The devin.kr article on
FLUX image generation accelerated on Blackwell ("Compute efficiency and
acceleration") lowers the cost of attention by running it in 8-bit floating
point with a per-token correction of the quantization error, for a 1.16-1.18x
speed-up.  The pages give no steps, so the following readings (the plainest
block-scaled FP8 attention consistent with the rest of the pages' microscaling
recipe) define the method, for one head with queries Q [Sq, D], keys K [Skv, D]
and values V [Skv, D]:

  1. Q and K are MXFP8-quantized along the head dimension D (E4M3 codes, one
     E8M0 scale per 32 channels of each token): the per-token scales correct
     each token's range (aitrends.kr MXFP8/NVFP4 article, Glossary
     "Microscaling Formats" and "MXFP8", for the format);
  2. V is MXFP8-quantized along the token axis (one E8M0 scale per 32
     consecutive tokens of each channel), the contraction axis of P V;
  3. scores s = Q^ K^T / sqrt(D) from the dequantized operands, exactly;
  4. softmax online over key tiles of `kv_tile` keys in key order (the order a
     single-pass kernel visits them): running max m, p = exp(s - m) <= 1,
     accumulator and row sum rescaled by exp(m_old - m_new);
  5. p is E4M3-quantized with the fixed scale 2**8 (p * 256 <= 256 < 448, so
     never saturated), and P^ V^ is accumulated;
  6. the row sum l accumulates the unquantized p; the output is acc / l.

Everything is float64; the only approximations are the format encodings the
method itself applies (steps 1, 2, 5) and float64 summation.
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


def online_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, kv_tile: int = 64,
                     quantize_probs: bool = True) -> np.ndarray:
    """Steps 3-6 on float64 operands (one head): the online softmax over key tiles in order."""
    Sq, D = q.shape
    Skv = k.shape[0]
    c = 1.0 / math.sqrt(D)
    m = np.full(Sq, -np.inf)
    l = np.zeros(Sq)
    acc = np.zeros((Sq, v.shape[1]))
    for t0 in range(0, Skv, kv_tile):
        s = (q @ k[t0:t0 + kv_tile].T) * c
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.exp(m - m_new)  # 0 at the first tile (m = -inf)
        p = np.exp(s - m_new[:, None])
        ph = quantize_p(p) if quantize_probs else p
        acc = acc * alpha[:, None] + ph @ v[t0:t0 + kv_tile]
        l = l * alpha + p.sum(axis=1)
        m = m_new
    return acc / l[:, None]


def attention_fp8_ref(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, kv_tile: int = 64,
                      rows=None) -> np.ndarray:
    """The block-scaled FP8 attention of one head from bf16 bit patterns [S, D]; float64 [Sq, D].

    `rows` (optional) restricts the output to those query rows (each row is independent)."""
    t = quantize_qkv(q_bits, k_bits, v_bits)
    q = t["q"] if rows is None else t["q"][np.asarray(rows)]
    return online_attention(q, t["k"], t["v"], kv_tile, True)


# E4M3 values >= 0 in increasing order (for the neighbours of a midpoint)
_E4M3_GRID = np.unique(decode_e4m3(np.arange(0x7F)))


def p_code_slack(q: np.ndarray, k: np.ndarray, v: np.ndarray, score_eta: float, exp_eta: float = 2.0 ** -20,
                 kv_tile: int = 64, forced=None):
    """Bound of what a valid other rounding of near-midpoint P codes can change in the output.

    Step 5 rounds p * 2^8 to E4M3, a decision taken from floating-point scores.
    A kernel that forms each score in a float accumulator of unit roundoff u
    over D products errs by at most gamma_D sum_d |q_d k_d| with gamma_D about
    D u (the recursive-summation bound), in the score itself and in the row's
    running maximum.  `score_eta` is that relative bound (D * 2^-24 for fp32
    and D = 128); `exp_eta` covers the exponential and the scaling.  For each
    key whose p * 2^8 lies within the resulting relative distance of an E4M3
    midpoint, either neighbour is a correct code; the returned slack [Sq, D]
    sums, per output, one E4M3 step (divided by 2^8) times |v_j| rescaled to
    the final maximum and divided by the final row sum, over those keys.

    `forced` (optional, for checking the bound): a set of (row, key) pairs
    whose code is taken as the other neighbour of the nearest midpoint; the
    function then also returns the output computed with those codes.
    Returns (slack, out_forced or None)."""
    Sq, D = q.shape
    Skv = k.shape[0]
    c = 1.0 / math.sqrt(D)
    A = np.abs(q) @ np.abs(k).T
    tol = c * score_eta * 2.0 * A.max(axis=1) + exp_eta  # relative bound on p, per row
    mids = (_E4M3_GRID[1:] + _E4M3_GRID[:-1]) / 2
    m = np.full(Sq, -np.inf)
    l = np.zeros(Sq)
    contrib = np.zeros((Sq, v.shape[1]))
    acc = np.zeros((Sq, v.shape[1]))
    for t0 in range(0, Skv, kv_tile):
        s = (q @ k[t0:t0 + kv_tile].T) * c
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.exp(m - m_new)
        p = np.exp(s - m_new[:, None])
        x = np.ldexp(p, P_SCALE_EXP)
        i = np.clip(np.searchsorted(mids, x), 1, len(mids) - 1)
        near_mid = np.where(np.abs(mids[i - 1] - x) < np.abs(mids[i] - x), mids[i - 1], mids[i])
        idx = np.searchsorted(_E4M3_GRID, near_mid)
        step = _E4M3_GRID[idx] - _E4M3_GRID[idx - 1]
        near = np.abs(x - near_mid) <= x * tol[:, None]
        contrib = contrib * alpha[:, None] + (near * step * 2.0 ** -P_SCALE_EXP) @ np.abs(v[t0:t0 + kv_tile])
        ph = quantize_p(p)
        if forced:
            for (r, j) in forced:
                if t0 <= j < t0 + kv_tile:
                    jj = j - t0
                    lo, hi = _E4M3_GRID[idx[r, jj] - 1], _E4M3_GRID[idx[r, jj]]
                    cur = ph[r, jj] * 2.0 ** P_SCALE_EXP
                    ph[r, jj] = (hi if cur == lo else lo) * 2.0 ** -P_SCALE_EXP
        acc = acc * alpha[:, None] + ph @ v[t0:t0 + kv_tile]
        l = l * alpha + p.sum(axis=1)
        m = m_new
    slack = contrib / l[:, None]
    return slack, (acc / l[:, None] if forced else None)


def near_midpoint_keys(q: np.ndarray, k: np.ndarray, score_eta: float, exp_eta: float = 2.0 ** -20,
                       kv_tile: int = 64):
    """The (row, key) pairs whose P code p_code_slack treats as ambiguous."""
    Sq, D = q.shape
    c = 1.0 / math.sqrt(D)
    A = np.abs(q) @ np.abs(k).T
    tol = c * score_eta * 2.0 * A.max(axis=1) + exp_eta
    mids = (_E4M3_GRID[1:] + _E4M3_GRID[:-1]) / 2
    out = []
    m = np.full(Sq, -np.inf)
    for t0 in range(0, k.shape[0], kv_tile):
        s = (q @ k[t0:t0 + kv_tile].T) * c
        m = np.maximum(m, s.max(axis=1))
        x = np.ldexp(np.exp(s - m[:, None]), P_SCALE_EXP)
        i = np.clip(np.searchsorted(mids, x), 1, len(mids) - 1)
        d = np.minimum(np.abs(mids[i - 1] - x), np.abs(mids[i] - x))
        for r, j in zip(*np.nonzero(d <= x * tol[:, None])):
            out.append((int(r), int(t0 + j)))
    return out
