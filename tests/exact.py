"""Exact-arithmetic helpers for pinning the oracle (tests only).

Everything here is written independently of oracle/w8_oracle.c: rational
arithmetic with fractions.Fraction, and PyTorch's own float8_e4m3fn dtype as
the library reference for the OCP E4M3FN code table.
"""
from fractions import Fraction
from math import floor

import numpy as np
import torch


def round_half_even(q: Fraction) -> int:
    fl = floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def round_fp32(q: Fraction) -> Fraction:
    """Correctly rounded (nearest, ties to even) IEEE binary32 value of q (no overflow)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # below 2^-126 the spacing stays 2^-149
    quantum = Fraction(2) ** (e - 23)
    return sign * round_half_even(a / quantum) * quantum


def torch_e4m3_table() -> np.ndarray:
    """float64 value of every code 0..255 according to torch.float8_e4m3fn."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


_TABLE = None


def e4m3_positive_values():
    """(codes, exact Fractions) of the finite non-negative E4M3FN values, by code."""
    global _TABLE
    if _TABLE is None:
        t = torch_e4m3_table()
        codes = [c for c in range(0x80) if np.isfinite(t[c])]
        _TABLE = (codes, [Fraction(float(t[c])) for c in codes])
    return _TABLE


def e4m3_nearest_code(v: Fraction, negative: bool) -> int:
    """Brute force: the finite E4M3FN code nearest to v (saturating at 448);
    on a tie the even code wins.  The sign bit follows `negative`."""
    codes, vals = e4m3_positive_values()
    a = abs(v)
    best_c, best_d = None, None
    for c, x in zip(codes, vals):
        d = abs(a - x)
        if best_d is None or d < best_d or (d == best_d and c % 2 == 0):
            best_c, best_d = c, d
    return best_c | (0x80 if negative else 0)


def int8_nearest(v: Fraction) -> int:
    r = round_half_even(v)
    return max(-127, min(127, r))


def quantize_group_exact(x_fp32, is_int8: bool):
    """Fraction brute force of one quantization group: (codes uint8 list, scale)."""
    xs = [Fraction(float(v)) for v in np.asarray(x_fp32, dtype=np.float32)]
    qmax = 127 if is_int8 else 448
    amax = max(abs(v) for v in xs)
    s = Fraction(1) if amax == 0 else round_fp32(amax / qmax)
    codes = []
    for raw, v in zip(np.asarray(x_fp32, dtype=np.float32), xs):
        q = round_fp32(v / s)
        if is_int8:
            codes.append(int8_nearest(q) & 0xFF)
        else:
            codes.append(e4m3_nearest_code(q, bool(np.signbit(raw)) if q == 0 else q < 0))
    return codes, s
