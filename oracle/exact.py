"""Scalar reference in exact rational arithmetic (oracle; test infrastructure only).

Everything here is a literal reading of the definitions with
``fractions.Fraction`` and pure-Python loops, used on small or exhaustive
inputs to pin the vectorized numpy oracle.  It deliberately shares no
arithmetic with ``formats.encode``: the element encoder here is an argmin over
the whole code table, not a rounding formula.

Definitions: OCP Microscaling Formats (MX) v1.0 (E4M3, E2M1, E8M0 and the
shared-exponent rule), named by the aitrends.kr MXFP8/NVFP4 article,
Glossary "MXFP8"; NVFP4 as E2M1 with an E4M3 scale per 16 elements and an
fp32 per-tensor scale (same article, Glossary "NVFP4" and the dynamic
per-tensor-scale setting under "Section details").
"""

from __future__ import annotations

from fractions import Fraction
from functools import lru_cache
from typing import List, Sequence, Tuple


def _minifloat_value(code: int, ebits: int, mbits: int, bias: int) -> Fraction:
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        mag = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
    return -mag if s else mag


@lru_cache(maxsize=None)
def e4m3_table() -> Tuple[Tuple[int, Fraction], ...]:
    """All non-negative finite E4M3 codes with their exact values (0x00 .. 0x7E)."""
    return tuple((c, _minifloat_value(c, 4, 3, 7)) for c in range(0x7F))


@lru_cache(maxsize=None)
def e2m1_table() -> Tuple[Tuple[int, Fraction], ...]:
    """All non-negative E2M1 codes with their exact values (0x0 .. 0x7)."""
    return tuple((c, _minifloat_value(c, 2, 1, 1)) for c in range(8))


@lru_cache(maxsize=None)
def e2m3_table() -> Tuple[Tuple[int, Fraction], ...]:
    """All non-negative E2M3 codes with their exact values (0x00 .. 0x1F)."""
    return tuple((c, _minifloat_value(c, 2, 3, 1)) for c in range(32))


@lru_cache(maxsize=None)
def e3m2_table() -> Tuple[Tuple[int, Fraction], ...]:
    """All non-negative E3M2 codes with their exact values (0x00 .. 0x1F)."""
    return tuple((c, _minifloat_value(c, 3, 2, 3)) for c in range(32))


def bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite bf16")
    if e == 0:
        mag = Fraction(m, 128) * Fraction(2) ** -126
    else:
        mag = (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -mag if s else mag


def encode_argmin(table: Sequence[Tuple[int, Fraction]], v: Fraction, negative: bool, sign_bit: int) -> int:
    """Nearest code by brute force over the table; ties go to the even code; saturates at the max."""
    a = abs(v)
    best_code, best_dist = None, None
    for code, val in table:
        d = abs(a - val)
        if best_dist is None or d < best_dist or (d == best_dist and code % 2 == 0):
            best_code, best_dist = code, d
    return best_code | (sign_bit if negative else 0)


def e4m3_encode(v: Fraction, negative: bool) -> int:
    return encode_argmin(e4m3_table(), v, negative, 0x80)


def e2m1_encode(v: Fraction, negative: bool) -> int:
    return encode_argmin(e2m1_table(), v, negative, 0x8)


def e2m3_encode(v: Fraction, negative: bool) -> int:
    return encode_argmin(e2m3_table(), v, negative, 0x20)


def e3m2_encode(v: Fraction, negative: bool) -> int:
    return encode_argmin(e3m2_table(), v, negative, 0x20)


def _floor_log2(a: Fraction) -> int:
    """floor(log2 a) for a > 0, by exact comparison."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _ceil_log2(q: Fraction) -> int:
    """ceil(log2 q) for a positive rational q, exactly."""
    f = _floor_log2(q)
    return f if q == Fraction(2) ** f else f + 1


def mx_block(bits: Sequence[int], elem: str, rule: str = "floor") -> Tuple[int, List[int]]:
    """Quantize one block of finite bf16 bit patterns to (E8M0 scale byte, element codes).

    Shared exponent, clamped to [-127, 127], an all-zero block using e = -127:
      "floor" (OCP MX v1.0): e = floor(log2 amax) - emax_elem;
      "rceil": e = ceil(log2(amax / max_elem)), the smallest power of two that
               brings the block maximum within the element format's range.
    Elements are x / 2**e encoded round-to-nearest-even with saturation.
    """
    emax, max_elem, enc = {
        "e4m3": (8, Fraction(448), e4m3_encode),
        "e2m1": (2, Fraction(6), e2m1_encode),
        "e2m3": (2, Fraction(15, 2), e2m3_encode),
        "e3m2": (4, Fraction(28), e3m2_encode),
    }[elem]
    vals = [bf16_value(b) for b in bits]
    negs = [bool((b >> 15) & 1) for b in bits]
    amax = max(abs(v) for v in vals)
    if amax == 0:
        e = -127
    elif rule == "floor":
        e = max(-127, min(127, _floor_log2(amax) - emax))
    elif rule == "rceil":
        e = max(-127, min(127, _ceil_log2(amax / max_elem)))
    else:
        raise ValueError(f"unknown scale rule {rule!r}")
    scale = Fraction(2) ** e
    return e + 127, [enc(v / scale, n) for v, n in zip(vals, negs)]


def fp32_round(q: Fraction) -> Fraction:
    """Round a positive rational to the nearest binary32 value (ties to even), exactly."""
    if q == 0:
        return Fraction(0)
    e = max(_floor_log2(q), -126)
    ulp = Fraction(2) ** (e - 23)
    n = q / ulp
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo * ulp


def nvfp4_tensor_scale(bits: Sequence[int]) -> Fraction:
    """Per-tensor scale ts = RN_fp32(G / (448 * 6)); G = 0 gives 1."""
    g = max(abs(bf16_value(b)) for b in bits)
    if g == 0:
        return Fraction(1)
    return fp32_round(g / (448 * 6))


def nvfp4_block(bits: Sequence[int], ts: Fraction) -> Tuple[int, List[int]]:
    """Quantize one 16-element block given the per-tensor scale ts.

    Block scale sc = E4M3 encode of B / (6 * ts) (one rounding of the exact
    quotient, saturating at 448); a nonzero block whose scale rounds to zero
    takes the smallest subnormal code 0x01; an all-zero block takes 0x00 and
    signed-zero elements.  Elements are x / (dec(sc) * ts) encoded to E2M1.
    """
    vals = [bf16_value(b) for b in bits]
    negs = [bool((b >> 15) & 1) for b in bits]
    bmax = max(abs(v) for v in vals)
    if bmax == 0:
        return 0, [0x8 if n else 0x0 for n in negs]
    sc = e4m3_encode(bmax / (6 * ts), False)
    if sc == 0:
        sc = 1
    denom = _minifloat_value(sc, 4, 3, 7) * ts
    return sc, [e2m1_encode(v / denom, n) for v, n in zip(vals, negs)]
