"""Closed-form element and scale formats (oracle; test infrastructure only).

The pages name the formats but print no bit layouts (aitrends.kr MXFP8/NVFP4
article, Glossary: "Microscaling Formats", "MXFP8", "NVFP4").  MXFP8 is the
OCP-standard microscaling format, so the layouts below are those of the OCP
Microscaling Formats (MX) v1.0 specification:

* bf16  : 1 sign, 8 exponent (bias 127), 7 mantissa bits; IEEE semantics.
* E4M3  : 1 sign, 4 exponent (bias 7), 3 mantissa bits.  Exponent field 0
          is subnormal (m * 2**-9).  No infinities; S.1111.111 is NaN, so
          the largest finite magnitude is 1.75 * 2**8 = 448 (code 0x7E).
* E2M1  : 1 sign, 2 exponent (bias 1), 1 mantissa bit.  Magnitudes
          {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no NaN or infinity.
* E8M0  : 8-bit unsigned exponent, bias 127, value 2**(c-127); 0xFF is NaN.

All arithmetic is float64 on values that are exact in float64.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class ElemFormat:
    """A sign-magnitude minifloat element format without infinities."""

    name: str
    ebits: int
    mbits: int
    bias: int
    max_value: float  # largest finite magnitude
    max_code: int  # magnitude code of max_value
    emax: int  # unbiased exponent of the largest normal number

    @property
    def emin(self) -> int:
        """Unbiased exponent of the smallest normal number (also the subnormal exponent)."""
        return 1 - self.bias

    @property
    def sign_bit(self) -> int:
        return 1 << (self.ebits + self.mbits)


E4M3 = ElemFormat("e4m3", ebits=4, mbits=3, bias=7, max_value=448.0, max_code=0x7E, emax=8)
E2M1 = ElemFormat("e2m1", ebits=2, mbits=1, bias=1, max_value=6.0, max_code=0x7, emax=2)
# the two 6-bit element formats of the OCP MX v1.0 specification (MXFP6)
E2M3 = ElemFormat("e2m3", ebits=2, mbits=3, bias=1, max_value=7.5, max_code=0x1F, emax=2)
E3M2 = ElemFormat("e3m2", ebits=3, mbits=2, bias=3, max_value=28.0, max_code=0x1F, emax=4)


def _decode_minifloat(fmt: ElemFormat, codes: np.ndarray) -> np.ndarray:
    """value = (-1)^s * 2^(E-bias) * (1 + m/2^mbits), or 2^(1-bias) * m/2^mbits if E == 0."""
    c = np.asarray(codes).astype(np.int64)
    s = (c >> (fmt.ebits + fmt.mbits)) & 1
    e = (c >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    m = c & ((1 << fmt.mbits) - 1)
    frac = m.astype(np.float64) / (1 << fmt.mbits)
    normal = np.ldexp(1.0 + frac, (e - fmt.bias).astype(np.int64))
    subnormal = np.ldexp(frac, np.full_like(e, fmt.emin))
    mag = np.where(e == 0, subnormal, normal)
    return np.where(s == 1, -mag, mag)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 (OCP "FN" variant) codes; S.1111.111 decodes to NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    v = _decode_minifloat(E4M3, c)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """Decode 4-bit E2M1 codes (low nibble of each value)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return _decode_minifloat(E2M1, c)


def decode_e2m3(codes: np.ndarray) -> np.ndarray:
    """Decode 6-bit E2M3 codes (no NaN or Inf)."""
    return _decode_minifloat(E2M3, np.asarray(codes).astype(np.int64) & 0x3F)


def decode_e3m2(codes: np.ndarray) -> np.ndarray:
    """Decode 6-bit E3M2 codes (no NaN or Inf)."""
    return _decode_minifloat(E3M2, np.asarray(codes).astype(np.int64) & 0x3F)


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """Decode E8M0 scale bytes: 2**(c-127); 0xFF is NaN."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 0xFF, np.nan, v)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64 from the sign/exponent/mantissa fields."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = b >> 15
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    frac = m.astype(np.float64) / 128.0
    normal = np.ldexp(1.0 + frac, (e - 127).astype(np.int64))
    subnormal = np.ldexp(frac, np.full_like(e, -126))
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where(e == 0xFF, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def encode(fmt: ElemFormat, v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even, saturating encode of exact reals ``v`` (float64) into ``fmt``.

    Steps (OCP MX v1.0 element conversion with saturation):
      1. the sign of the code is the sign bit of v (kept for zero);
      2. a = |v|; a >= max_value encodes to max_value;
      3. otherwise a lies between two neighbouring grid points (subnormals
         included); the nearer one is chosen, and on a tie the one whose
         mantissa LSB (= code LSB) is zero.

    The grid spacing around a is 2**(E - mbits) with E = max(floor(log2 a), emin),
    so rounding a / 2**(E - mbits) to the nearest even integer q gives the
    code (E - emin) * 2**mbits + q; a carry of q into the next binade lands
    on the correct code because the code is monotone in the value.
    Inputs must be finite.  Returns int64 codes.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode() needs finite inputs")
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    _, ex = np.frexp(a)  # a = f * 2**ex, f in [0.5, 1)
    E = np.where(a == 0, fmt.emin, np.maximum(ex.astype(np.int64) - 1, fmt.emin))
    q = np.rint(np.ldexp(a, -(E - fmt.mbits)))  # exact scaling, then RNE
    code = (E - fmt.emin) * (1 << fmt.mbits) + q.astype(np.int64)
    code = np.where(a >= fmt.max_value, fmt.max_code, code)
    return code | (sign * fmt.sign_bit)


def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive finite float64 a, exactly (from the exponent)."""
    _, ex = np.frexp(np.asarray(a, dtype=np.float64))
    return ex.astype(np.int64) - 1
