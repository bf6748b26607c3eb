"""Pins for the oracle's format decoders and element encoder.

Each check compares the oracle against something other than itself:
library decoders (torch's float8 dtypes, numpy's float32 view), the hand-
written landmark table under tests/golden (OCP MX v1.0 values), an exhaustive
brute-force nearest-code search, and the exact Fraction reference.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import E2M1, E4M3, decode_bf16, decode_e2m1, decode_e4m3, decode_e8m0, encode
from oracle import exact


def _landmarks(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "format_landmarks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                fmt, code, val = line.split()
                rows.append((fmt, int(code, 16), val))
    return rows


def test_landmarks(golden_dir):
    dec = {"e4m3": decode_e4m3, "e2m1": decode_e2m1, "e8m0": decode_e8m0}
    rows = _landmarks(golden_dir)
    assert len(rows) > 20
    for fmt, code, val in rows:
        got = float(dec[fmt](np.array([code]))[0])
        if val == "nan":
            assert math.isnan(got), (fmt, hex(code))
        else:
            want = float(val)
            assert got == want, (fmt, hex(code), got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, want), (fmt, hex(code))


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    assert int(np.isfinite(got).sum()) == 254


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_bf16_decode_matches_float32_view():
    bits = np.arange(65536, dtype=np.uint32)
    ref = (bits << 16).view(np.float32).astype(np.float64)
    got = decode_bf16(bits.astype(np.uint16))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_e2m1_decode_closed_form():
    # sign * {0, .5, 1, 1.5, 2, 3, 4, 6}
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    got = decode_e2m1(np.arange(16))
    assert list(got[:8]) == mags
    assert list(-got[8:]) == mags
    assert np.all(np.signbit(got[8:]))


def _brute_force_codes(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Nearest grid index, ties to the even index; saturating above the top of the grid."""
    d = np.abs(a[:, None] - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    idx = np.arange(grid.size)[None, :]
    even_hit = cand & (idx % 2 == 0)
    first = np.argmax(cand, axis=1)
    first_even = np.argmax(even_hit, axis=1)
    return np.where(even_hit.any(axis=1), first_even, first)


def _all_8bit_significand_values(lo_exp: int, hi_exp: int) -> np.ndarray:
    sig = np.arange(128, 256, dtype=np.float64)
    vals = [np.ldexp(sig, k - 7) for k in range(lo_exp, hi_exp + 1)]
    return np.concatenate([np.zeros(1)] + vals)


@pytest.mark.parametrize("fmt_name", ["e4m3", "e2m1"])
def test_encode_exhaustive_brute_force(fmt_name):
    """Every non-negative value with an 8-bit significand over the whole relevant range."""
    if fmt_name == "e4m3":
        fmt = E4M3
        # grid from the library decoder, not from the oracle
        grid = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        a = _all_8bit_significand_values(-14, 10)
    else:
        fmt = E2M1
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
        a = _all_8bit_significand_values(-6, 4)
    want = _brute_force_codes(a, grid)
    got = encode(fmt, a)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(a[i], got[i], want[i]) for i in bad[:5]]
    # negative inputs: same magnitude code with the sign bit
    gotn = encode(fmt, -a)
    assert np.array_equal(gotn, want | fmt.sign_bit)


def test_encode_e4m3_matches_torch_cast_in_range():
    """torch's float8_e4m3fn cast rounds to nearest-even; it agrees wherever no saturation applies."""
    a = _all_8bit_significand_values(-14, 8)
    a = np.concatenate([a, -a])
    a = a[np.abs(a) <= 448]
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = encode(E4M3, a)
    assert np.array_equal(got, ref)


def test_encode_saturates_instead_of_nan():
    big = np.array([448.0, 449.0, 464.0, 465.0, 1e30, -500.0])
    assert list(encode(E4M3, big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert list(encode(E2M1, np.array([6.0, 6.5, 7.0, 1e9, -8.0]))) == [7, 7, 7, 7, 0xF]


def test_encode_signed_zero():
    assert list(encode(E4M3, np.array([0.0, -0.0, -1e-30]))) == [0x00, 0x80, 0x80]
    assert list(encode(E2M1, np.array([0.0, -0.0, -0.1]))) == [0x0, 0x8, 0x8]


def test_encode_matches_exact_on_random_rationals():
    """Non-dyadic reals (as NVFP4 quotients are): float64 encode vs exact argmin on the Fraction."""
    rng = np.random.default_rng(1)
    for _ in range(3000):
        num = int(rng.integers(1, 1 << 8)) * 2 ** int(rng.integers(-12, 12))
        den = int(rng.integers(1, 1 << 24)) * int(rng.integers(1, 16))
        q = Fraction(num) / den * Fraction(2) ** int(rng.integers(-4, 20))
        for fmt, ex in ((E4M3, exact.e4m3_encode), (E2M1, exact.e2m1_encode)):
            got = int(encode(fmt, np.array([float(q)]))[0])
            assert got == ex(q, False), (fmt.name, q)


def test_exact_tables_agree_with_vector_decoders():
    for code, val in exact.e4m3_table():
        assert Fraction(float(decode_e4m3(np.array([code]))[0])) == val
    for code, val in exact.e2m1_table():
        assert Fraction(float(decode_e2m1(np.array([code]))[0])) == val
