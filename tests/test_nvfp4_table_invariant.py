"""Pin of the property behind the NVFP4 block pass's table path, in exact rational arithmetic (CPU).

A bf16 |x| under E4M3 block-scale code c and tensor scale ts gets the E2M1
magnitude that counts the midpoints mu_j * dec(c) * ts (mu = 1/4, 3/4, 5/4, 7/4,
5/2, 7/2, 5; ties to the even code) at or below it (aitrends.kr MXFP8/NVFP4
article, Glossary "NVFP4"; E2M1 and E4M3 encodings of the OCP Microscaling
Formats specification).  As bf16 bit patterns, each midpoint is a threshold
T_j(c): the smallest pattern that rounds above it.  The kernel relies on this:
for ts >= 2^-60, T_j(c) = T_j(r) + 128 E for the code r = 0x38 | k whose value
1 + k/8 has the significand of dec(c) = 2^E (1 + k/8), so one byte table per
significand class k decides every code of that class.  This file checks that
claim for every code 1..0x7E over a spread of float32 tensor scales, the
spacing and length bounds the kernel checks before using its tables, and
(as a control) that the relation does fail where thresholds become subnormal.
"""

from fractions import Fraction

import numpy as np

MIDPOINTS = [(Fraction(1, 4), False), (Fraction(3, 4), True), (Fraction(5, 4), False), (Fraction(7, 4), True),
             (Fraction(5, 2), False), (Fraction(7, 2), True), (Fraction(5), False)]  # (mu_j, tie goes up)
TABLE_BYTES = 640  # bytes per class table in the kernel


def e4m3_value(c: int) -> Fraction:
    e, m = c >> 3, c & 7
    if e == 0:
        return Fraction(m, 8) * Fraction(2) ** -6
    return (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def bf16_value(p: int) -> Fraction:
    e, m = p >> 7, p & 0x7F
    if e == 0:
        return Fraction(m, 128) * Fraction(2) ** -126
    return (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def threshold(x: Fraction, tie_up: bool) -> int:
    """Smallest bf16 magnitude pattern p (finite: <= 0x7F7F, else 0x7F80) whose value is above x, or
    equal to it when the tie goes up; every bf16 |y| rounds above the midpoint x exactly when its
    pattern is >= p (patterns order like values)."""
    lo, hi = 0, 0x7F80
    while lo < hi:
        mid = (lo + hi) // 2
        v = bf16_value(mid)
        if v > x or (v == x and tie_up):
            hi = mid
        else:
            lo = mid + 1
    return lo


def thresholds(c: int, ts: Fraction):
    d = e4m3_value(c)
    return [threshold(mu * d * ts, up) for mu, up in MIDPOINTS]


def significand_class(c: int):
    """(k, E) with dec(c) = 2^E (1 + k/8)."""
    d = e4m3_value(c)
    E = 0
    while d >= 2:
        d /= 2
        E += 1
    while d < 1:
        d *= 2
        E -= 1
    k = (d - 1) * 8
    assert k.denominator == 1
    return int(k), E


def _tensor_scales():
    rng = np.random.default_rng(11)
    vals = [2.0 ** -60, float(np.nextafter(np.float32(2.0 ** -60), np.float32(1))), 1.0,
            float(np.float32(2688.0 / 2688.0)), float(np.float32(float.fromhex("0x1.2p-7")))]
    # ts = RN_fp32(G / 2688) for a few bf16 tensor maxima G, and random float32 scales over 2^-60 .. 2^40
    for g in (1.0, 3.0, 448.0, 2688.0, 65280.0, 3.0e38):
        vals.append(float(np.float32(g / 2688.0)))
    for e in rng.uniform(-60.0, 40.0, 12):
        vals.append(float(np.float32(2.0 ** e)))
    return [Fraction(v) for v in vals if v >= 2.0 ** -60]


def test_thresholds_shift_with_the_scale_exponent():
    reps = {}
    for ts in _tensor_scales():
        rep_t = {k: thresholds(0x38 | k, ts) for k in range(8)}
        for k, t in rep_t.items():
            # the kernel's own checks on each class table: distinct steps >= 21 entries apart, and the
            # last threshold inside the table
            assert all(t[j + 1] - t[j] >= TABLE_BYTES // 32 + 1 for j in range(6)), (ts, k, t)
            assert t[6] - t[0] <= TABLE_BYTES - 2, (ts, k, t)
        for c in range(1, 0x7F):
            k, E = significand_class(c)
            t = thresholds(c, ts)
            assert t == [r + 128 * E for r in rep_t[k]], (ts, c, t, rep_t[k], E)
        reps[ts] = rep_t
    assert len(reps) >= 20


def test_relation_fails_for_subnormal_thresholds():
    """Control: with thresholds in bf16's subnormal range the exponent shift no longer holds for some
    code, so the check above can fail (the kernel searches the thresholds there instead)."""
    ts = Fraction(2) ** -130
    bad = 0
    for c in range(1, 0x7F):
        k, E = significand_class(c)
        if thresholds(c, ts) != [r + 128 * E for r in thresholds(0x38 | k, ts)]:
            bad += 1
    assert bad > 0


def test_class_and_representative():
    assert significand_class(0x38) == (0, 0) and e4m3_value(0x38) == 1
    assert significand_class(0x3F) == (7, 0) and e4m3_value(0x3F) == Fraction(15, 8)
    assert significand_class(0x7E) == (6, 8) and e4m3_value(0x7E) == 448
    assert significand_class(1) == (0, -9)  # smallest subnormal code: 2^-9
    assert significand_class(3) == (4, -8)  # 3 * 2^-9 = 1.5 * 2^-8
    assert significand_class(5) == (2, -7)  # 5 * 2^-9 = 1.25 * 2^-7
