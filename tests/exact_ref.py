"""Brute-force reference in exact rational arithmetic (fractions.Fraction), tiny inputs only.

An independent second implementation used to pin the float64 oracle: every rounding
is a nearest search over the whole finite value set of the target format with explicit
tie handling, every quotient is exact, and binary32 rounding is done on rationals.
It reuses nothing from oracle/.
"""
from fractions import Fraction as Fr
import math

# E2M1 magnitudes by code 0..7 (OCP MX v1.0: bias 1, one mantissa bit)
E2M1 = [Fr(0), Fr(1, 2), Fr(1), Fr(3, 2), Fr(2), Fr(3), Fr(4), Fr(6)]


def _e4m3_values():
    vals = []
    for code in range(127):                 # 0x7F is NaN
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(Fr(m, 8) * Fr(1, 64))
        else:
            vals.append((1 + Fr(m, 8)) * Fr(2) ** (e - 7))
    return vals


E4M3 = _e4m3_values()


def nearest_even(grid, a):
    """Index of the nearest grid value to a >= 0; on an exact tie the even index;
    beyond the last value, the last index."""
    best, best_d = None, None
    for i, g in enumerate(grid):
        d = abs(a - g)
        if best is None or d < best_d or (d == best_d and i % 2 == 0):
            best, best_d = i, d
    return best


def round_binary(fr, p=24, emin=-126):
    """Round a rational to the nearest binary float with p-bit significand (ties to
    even), subnormals below 2^emin; returns a Fraction.  No overflow handling."""
    if fr == 0:
        return Fr(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fr(2) ** (e - p + 1)
    q = a / ulp
    n = math.floor(q)
    rem = q - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32(fr):
    return round_binary(fr, 24, -126)


def nvfp4_block_codes(xs, s_t):
    """Exact NVFP4 of one 16-element block under tensor scale s_t (Fractions).
    Returns (E4M3 code, list of 4-bit codes)."""
    amax = max(abs(v) for v in xs)
    if s_t == 0 or amax == 0:
        sb_code = 0
    else:
        sb_code = nearest_even(E4M3, amax / (6 * s_t))
    S = E4M3[sb_code] * s_t
    codes = []
    for v in xs:
        sign = 8 if (v < 0) else 0
        mag = 0 if S == 0 else nearest_even(E2M1, abs(v) / S)
        codes.append(sign | mag)
    return sb_code, codes


def nvfp4_tensor(rows, s_t=None):
    """Exact NVFP4 of a list of rows of Fractions (each row a multiple of 16 long)."""
    if s_t is None:
        amax = max(abs(v) for r in rows for v in r)
        s_t = f32(amax / 2688)
    codes, scales = [], []
    for r in rows:
        rc, rs = [], []
        for b in range(0, len(r), 16):
            sb, c = nvfp4_block_codes(r[b:b + 16], s_t)
            rs.append(sb)
            rc.extend(c)
        codes.append(rc)
        scales.append(rs)
    return s_t, codes, scales


def mxfp4_block_codes(xs):
    """Exact MXFP4 of one 32-element block: (E8M0 code, codes).  The scale is the
    largest power of two X with 4 X <= amax (i.e. amax / X in [4, 8))."""
    amax = max(abs(v) for v in xs)
    if amax == 0:
        e = -127
    else:
        e = 0
        while Fr(2) ** (e + 2) > amax:
            e -= 1
        while Fr(2) ** (e + 3) <= amax:
            e += 1
        e = max(-127, min(127, e))
    X = Fr(2) ** e
    codes = []
    for v in xs:
        sign = 8 if v < 0 else 0
        codes.append(sign | nearest_even(E2M1, abs(v) / X))
    return e + 127, codes


def e2m1_value(code):
    v = E2M1[code & 7]
    return -v if code & 8 else v
