"""Exact-rational model of IEEE 754 binary32 addition and multiplication.

A checker for the oracle that does not use the machine's float arithmetic:
each operation is computed exactly with ``fractions.Fraction`` and rounded once
to binary32 with an explicit round-to-nearest-even (IEEE 754-2019 s4.3.1),
gradual underflow (s7.5), overflow to infinity, and the sign rules for zero
results (s6.3).  Values are carried as 32-bit patterns (Python ints).

Special values: an infinity is ('inf', sign); NaN is the sentinel ``NAN``.
NaN payloads are not modelled (the fold's inputs are finite; where a NaN
arises only its NaN-ness is compared).
"""
from __future__ import annotations

from fractions import Fraction

NAN = 0x7FC00000  # quiet NaN pattern used for every NaN result
_EXP_MIN = -126   # smallest normal exponent
_MANT = 23        # fraction bits
_MAX_EXP = 127


def is_nan(bits: int) -> bool:
    return (bits & 0x7F800000) == 0x7F800000 and (bits & 0x7FFFFF) != 0


def is_inf(bits: int) -> bool:
    return (bits & 0x7FFFFFFF) == 0x7F800000


def sign_of(bits: int) -> int:
    return (bits >> 31) & 1


def value(bits: int) -> Fraction:
    """Exact value of a finite binary32 pattern."""
    if is_nan(bits) or is_inf(bits):
        raise ValueError("not finite: %08x" % bits)
    s = -1 if sign_of(bits) else 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0:  # zero or subnormal: m * 2^-149
        return s * Fraction(m, 1 << 149)
    return s * Fraction((1 << 23) | m) * Fraction(2) ** (e - 127 - 23)


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e <= a < 2^(e+1) must hold; adjust by at most one
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_rne(q: Fraction, zero_sign: int = 0) -> int:
    """Round the exact rational ``q`` to binary32, ties to even.

    ``zero_sign`` is the sign bit to give an exact zero (the caller decides it
    from the operation's sign rule)."""
    if q == 0:
        return zero_sign << 31
    sign = 1 if q < 0 else 0
    a = -q if sign else q
    e = max(_floor_log2(a), _EXP_MIN)
    quantum = Fraction(2) ** (e - _MANT)
    scaled = a / quantum
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and (n & 1)):
        n += 1
    if n == 0:  # underflow to zero (a product can do this; a sum cannot)
        return sign << 31
    rounded = n * quantum
    if rounded >= Fraction(2) ** (_MAX_EXP + 1):
        return (sign << 31) | 0x7F800000
    if rounded < Fraction(2) ** _EXP_MIN:  # subnormal result
        m = rounded / Fraction(1, 1 << 149)
        assert m.denominator == 1
        return (sign << 31) | int(m)
    e2 = _floor_log2(rounded)
    frac = rounded / Fraction(2) ** (e2 - _MANT) - (1 << _MANT)
    assert frac.denominator == 1 and 0 <= frac < (1 << _MANT)
    return (sign << 31) | ((e2 + 127) << 23) | int(frac)


def add(a: int, b: int) -> int:
    """binary32 a + b, round to nearest even."""
    if is_nan(a) or is_nan(b):
        return NAN
    if is_inf(a) or is_inf(b):
        if is_inf(a) and is_inf(b) and sign_of(a) != sign_of(b):
            return NAN
        return a if is_inf(a) else b
    q = value(a) + value(b)
    # exact zero: -0 only when both operands are -0
    zs = 1 if (q == 0 and a == 0x80000000 and b == 0x80000000) else 0
    return round_rne(q, zs)


def mul(a: int, b: int) -> int:
    """binary32 a * b, round to nearest even."""
    if is_nan(a) or is_nan(b):
        return NAN
    s = sign_of(a) ^ sign_of(b)
    if is_inf(a) or is_inf(b):
        other = b if is_inf(a) else a
        if not is_inf(other) and (other & 0x7FFFFFFF) == 0:
            return NAN  # inf * 0
        return (s << 31) | 0x7F800000
    return round_rne(value(a) * value(b), s)


def fold(slot_bits: list[list[int]]) -> list[int]:
    """Fixed-order fold of W slots of bit patterns: acc = s0, acc = acc + s_r."""
    W = len(slot_bits)
    n = len(slot_bits[0])
    out = []
    for i in range(n):
        acc = slot_bits[0][i]
        for r in range(1, W):
            acc = add(acc, slot_bits[r][i])
        out.append(acc)
    return out


def fold_scaled(slot_bits: list[list[int]], inv_bits: int) -> list[int]:
    return [mul(x, inv_bits) for x in fold(slot_bits)]


def same(a: int, b: int) -> bool:
    """Bit equality, except that any two NaNs compare equal (payload unpinned)."""
    if is_nan(a) or is_nan(b):
        return is_nan(a) and is_nan(b)
    return a == b
