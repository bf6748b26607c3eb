"""MXFP8 / MXFP4 / NVFP4 quantizers and dequantizers (oracle; test infrastructure only).

Inputs are bf16 bit patterns (uint16 arrays, row-major [rows, K], blocks run
along K).  Outputs use the layouts of the library:

* MX codes: uint8 [rows, K] (E4M3) or uint8 [rows, K/2] (E2M1, element 2j in
  the low nibble of byte j, element 2j+1 in the high nibble) or uint8
  [rows, K] (E2M3 / E3M2: each 32-element block occupies a 32-byte slot, the
  24 little-endian bytes of its 192-bit integer, element j at bits 6j ..
  6j+5, then 8 zero bytes);
* MX scales: uint8 [rows, K/32] E8M0, row-major;
* NVFP4: uint8 [rows, K/2] packed E2M1, uint8 [rows, K/16] E4M3 block scales
  and one float32 per-tensor scale.

Method (aitrends.kr MXFP8/NVFP4 article, Glossary "Microscaling Formats":
a short block shares one scale; "MXFP8": the OCP standard; "NVFP4": 4-bit
E2M1 with finer scaling; "Section details", TorchAO configuration: dynamic
activation quantization with a dynamic per-tensor scale).  Step numbers below
follow the OCP MX v1.0 quantization procedure.
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np

from .formats import (E2M1, E2M3, E3M2, E4M3, ElemFormat, decode_bf16, decode_e2m1, decode_e2m3, decode_e3m2,
                      decode_e4m3, decode_e8m0, encode, floor_log2)


@dataclass(frozen=True)
class Scheme:
    name: str
    elem: ElemFormat
    block: int
    packed: bool  # two 4-bit codes per byte
    fp6: bool = False  # 6-bit codes, one 32-byte slot per 32-element block


MXFP8 = Scheme("mxfp8", E4M3, 32, False)
MXFP4 = Scheme("mxfp4", E2M1, 32, True)
NVFP4 = Scheme("nvfp4", E2M1, 16, True)
# MXFP6 (OCP MX v1.0), the 6-bit formats of the same family as MXFP8 and MXFP4
MXFP6_E2M3 = Scheme("mxfp6_e2m3", E2M3, 32, False, True)
MXFP6_E3M2 = Scheme("mxfp6_e3m2", E3M2, 32, False, True)


def should_quantize(M: int, K: int, N: int) -> bool:
    """Selective quantization: layers with min(M, K, N) < 1024 stay in bf16.

    aitrends.kr MXFP8/NVFP4 article, "Section details", second "Evidence"
    block: layers whose shapes are too small for the gain to beat the
    overhead, min(M, K, N) < 1024, are excluded from quantization.
    """
    return min(M, K, N) >= 1024


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """[rows, K] 4-bit codes -> [rows, K/2] bytes; element 2j in the low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[rows, K/2] bytes -> [rows, K] 4-bit codes."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """[rows, K] 6-bit codes -> [rows, K] bytes: each 32-element block becomes a 32-byte slot holding the
    24 little-endian bytes of sum_j code_j * 2**(6 j), then 8 zero bytes."""
    c = np.asarray(codes).astype(np.uint64) & np.uint64(0x3F)
    rows, K = c.shape
    c = c.reshape(rows, K // 32, 32)
    words = np.zeros((rows, K // 32, 3), dtype=np.uint64)
    for j in range(32):
        bit = 6 * j
        w, off = bit // 64, bit % 64
        words[..., w] |= (c[..., j] << np.uint64(off)) & np.uint64(0xFFFFFFFFFFFFFFFF)
        if off > 58:  # the code straddles two 64-bit words
            words[..., w + 1] |= c[..., j] >> np.uint64(64 - off)
    slots = np.zeros((rows, K // 32, 4), dtype="<u8")
    slots[..., :3] = words
    return slots.view(np.uint8).reshape(rows, K)


def unpack_fp6(packed: np.ndarray) -> np.ndarray:
    """[rows, K] bytes (32-byte slots) -> [rows, K] 6-bit codes; the slots' last 8 bytes are ignored."""
    p = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    rows = p.shape[0]
    nb = p.shape[1] // 32
    words = p.reshape(rows, nb, 32).view("<u8").astype(np.uint64)[..., :3]  # [rows, nb, 3]
    out = np.empty((rows, nb, 32), dtype=np.uint8)
    for j in range(32):
        bit = 6 * j
        w, off = bit // 64, bit % 64
        v = words[..., w] >> np.uint64(off)
        if off > 58:
            v |= words[..., w + 1] << np.uint64(64 - off)
        out[..., j] = (v & np.uint64(0x3F)).astype(np.uint8)
    return out.reshape(rows, nb * 32)


def _check_bits(bits: np.ndarray, block: int) -> np.ndarray:
    b = np.asarray(bits)
    if b.dtype != np.uint16 or b.ndim != 2:
        raise TypeError("expected a 2-D uint16 array of bf16 bit patterns")
    if b.shape[1] % block:
        raise ValueError(f"K={b.shape[1]} is not a multiple of the block size {block}")
    return b


SCALE_RULES = ("floor", "rceil")


def quantize_mx(bits: np.ndarray, scheme: Scheme, rule: str = "floor"):
    """MX quantization of a bf16 matrix along K.

    For each row and each block of 32 consecutive K elements:
      1. if any element is NaN or Inf: scale byte 0xFF, codes 0;
      2. amax = max |x|;
      3. shared exponent e, clamped to [-127, 127] (e = -127 for an all-zero
         block):
         * rule "floor" (the OCP MX v1.0 rule): e = floor(log2 amax) - emax_elem.
           The block maximum can exceed the element format's largest value
           (up to 2x) and then saturates;
         * rule "rceil": e = the smallest integer with amax <= max_elem * 2**e,
           i.e. ceil(log2(amax / max_elem)), so no element saturates.  It is
           the floor exponent, plus one when amax > max_elem * 2**e_floor;
      4. scale byte = e + 127;
      5. code = RNE-saturating encode of x / 2**e (a power-of-two division,
         exact in float64);
      6. E2M1 codes are packed two per byte.
    Returns (codes uint8, scales uint8).

    The pages fix the format family only by name (aitrends.kr MXFP8/NVFP4
    article, Glossary "Microscaling Formats": one shared scale per short
    block keeps a wide range at low bit depth; "MXFP8": the OCP standard).
    "floor" is that standard's rule; "rceil" is the variant that rounds the
    shared scale up instead, offered as an option beside it.
    """
    if scheme.block != 32:
        raise ValueError("MX schemes use 32-element blocks")
    if rule not in SCALE_RULES:
        raise ValueError(f"unknown scale rule {rule!r}")
    b = _check_bits(bits, 32)
    rows, K = b.shape
    x = decode_bf16(b).reshape(rows, K // 32, 32)
    finite = np.isfinite(x).all(axis=-1)
    xf = np.where(finite[..., None], x, 0.0)
    amax = np.abs(xf).max(axis=-1)
    e = np.where(amax == 0, -127, floor_log2(np.where(amax == 0, 1.0, amax)) - scheme.elem.emax)
    if rule == "rceil":
        # both sides exact in float64: amax is a bf16 value, the product a power-of-two multiple of max_elem
        e = e + (amax > np.ldexp(scheme.elem.max_value, e)).astype(np.int64)
    e = np.clip(e, -127, 127)
    scaled = np.ldexp(xf, -e[..., None])
    codes = encode(scheme.elem, scaled)
    codes = np.where(finite[..., None], codes, 0).reshape(rows, K)
    scales = np.where(finite, e + 127, 0xFF).astype(np.uint8)
    if scheme.packed:
        return pack_fp4(codes), scales
    if scheme.fp6:
        return pack_fp6(codes), scales
    return codes.astype(np.uint8), scales


def nvfp4_tensor_scale(bits: np.ndarray) -> np.float32:
    """ts = RN_fp32(G / 2688) with G = max |x| over the tensor; G = 0 gives 1.

    2688 = 448 * 6 maps the largest block amax to the largest E4M3 scale
    times the largest E2M1 element.  Rounded exactly through Fraction.
    Any NaN/Inf in the tensor gives NaN.
    """
    x = decode_bf16(np.asarray(bits))
    if not np.all(np.isfinite(x)):
        return np.float32(np.nan)
    g = float(np.abs(x).max()) if x.size else 0.0
    if g == 0.0:
        return np.float32(1.0)
    q = Fraction(g) / 2688
    # float64(q) is within 2**-53 relative of q; converting that to float32
    # cannot double-round because q's binary expansion is either short
    # (exact) or periodic and never within 2**-53 of a float32 midpoint; the
    # exact check below rejects the impossible case loudly.
    f = np.float32(float(q))
    lo, hi = np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(np.inf))
    dist = abs(Fraction(float(f)) - q)
    if dist > abs(Fraction(float(lo)) - q) or dist > abs(Fraction(float(hi)) - q):
        raise AssertionError("float32 rounding of G/2688 is not nearest")
    return f


def quantize_nvfp4(bits: np.ndarray, ts=None):
    """NVFP4-style quantization: E2M1 codes, E4M3 scale per 16 elements, fp32 per-tensor scale.

    ``ts`` may be given to quantize a subset of a tensor's rows with the
    per-tensor scale of the whole tensor (``nvfp4_tensor_scale(full)``).

      1. ts = nvfp4_tensor_scale(x)  (global amax G; ts = RN_fp32(G/2688));
      2. per 16-block with amax B: B = 0 gives sc = 0x00; otherwise
         sc = E4M3 RNE-saturating encode of B / (6 * ts), and a result of
         0x00 is raised to 0x01;
      3. code = E2M1 encode of x / (dec(sc) * ts); sc = 0x00 gives signed zeros.
    The quotients are evaluated in float64: their operands carry at most 8, 4
    and 24 significant bits, so a non-tie quotient is at least ~2**-32
    (relative) away from any rounding midpoint while float64 division errs by
    at most 2**-53; the rounding decisions are therefore those of the exact
    quotient (pinned against ``exact.nvfp4_block``).
    Non-finite input: ts = NaN, every scale 0x7F, every code 0.
    Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/16], ts float32).
    """
    b = _check_bits(bits, 16)
    rows, K = b.shape
    ts = nvfp4_tensor_scale(b) if ts is None else np.float32(ts)
    if np.isnan(ts):
        return (np.zeros((rows, K // 2), np.uint8), np.full((rows, K // 16), 0x7F, np.uint8), ts)
    x = decode_bf16(b).reshape(rows, K // 16, 16)
    bmax = np.abs(x).max(axis=-1)
    ts64 = float(ts)
    sc = encode(E4M3, bmax / (6.0 * ts64))
    sc = np.where((sc == 0) & (bmax > 0), 1, sc)
    sc = np.where(bmax == 0, 0, sc)
    denom = decode_e4m3(sc) * ts64
    safe = np.where(sc == 0, 1.0, denom)
    codes = encode(E2M1, x / safe[..., None])
    codes = np.where((sc == 0)[..., None], np.signbit(x).astype(np.int64) * 0x8, codes)
    return pack_fp4(codes.reshape(rows, K)), sc.astype(np.uint8), ts


def dequant_mx(codes: np.ndarray, scales: np.ndarray, scheme: Scheme) -> np.ndarray:
    """value = dec_elem(code) * 2**(scale - 127), float64 [rows, K] (exact)."""
    c = unpack_fp4(codes) if scheme.packed else unpack_fp6(codes) if scheme.fp6 else np.asarray(codes)
    dec = {"e2m1": decode_e2m1, "e4m3": decode_e4m3, "e2m3": decode_e2m3, "e3m2": decode_e3m2}[scheme.elem.name]
    v = dec(c)
    rows, K = v.shape
    s = decode_e8m0(scales).reshape(rows, K // 32, 1)
    return (v.reshape(rows, K // 32, 32) * s).reshape(rows, K)


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, ts) -> np.ndarray:
    """value = dec_E2M1(code) * dec_E4M3(sc) * ts, float64 [rows, K] (exact)."""
    v = decode_e2m1(unpack_fp4(codes))
    rows, K = v.shape
    s = decode_e4m3(scales).reshape(rows, K // 16, 1)
    return (v.reshape(rows, K // 16, 16) * s).reshape(rows, K) * float(ts)
