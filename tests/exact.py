"""Exact-arithmetic helpers for pinning the oracle.

These do not use the oracle's code: bf16 patterns are decoded field by field
into exact fractions, and rounding to bf16 is done on exact rationals with an
explicit round-half-to-even rule. Square roots are evaluated with ``decimal`` at
high precision.
"""

from __future__ import annotations

import decimal
from fractions import Fraction

BF16_INF = 0x7F80
PREC = 70


def bf16_fields_value(bits: int):
    """Exact value of a bf16 pattern from its sign / exponent / fraction fields.

    Returns a Fraction, or the floats inf / -inf / nan for the special patterns.
    """
    bits &= 0xFFFF
    sign = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        if f:
            return float("nan")
        return float("inf") * sign
    if e == 0:
        return sign * Fraction(f, 128) * Fraction(1, 2**126)
    return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)


def _round_half_even(q: Fraction) -> int:
    fl = q.numerator // q.denominator
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_exact_to_bf16(v) -> int:
    """Round an exact rational (Fraction, int or Decimal) to bf16; return the bits.

    Ties go to the even significand; magnitudes at or above 2**128 after
    rounding become infinity; values under 2**-126 use the subnormal spacing
    2**-133.
    """
    v = Fraction(v)
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    # exponent E with 2**E <= a < 2**(E+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    eff = max(e, -126)
    spacing = Fraction(2) ** (eff - 7)
    n = _round_half_even(a / spacing)
    if eff == -126 and n < 128:  # subnormal (or zero)
        return sign | n
    # normal: n in [128, 256]
    if n == 256:
        eff += 1
        n = 128
    if eff > 127:
        return sign | BF16_INF
    return sign | ((eff + 127) << 7) | (n - 128)


def midpoint_distance(v) -> Fraction:
    """Relative distance of exact v from the nearest bf16 rounding midpoint."""
    v = abs(Fraction(v))
    if v == 0:
        return Fraction(1)
    e = v.numerator.bit_length() - v.denominator.bit_length()
    while Fraction(2) ** e > v:
        e -= 1
    while Fraction(2) ** (e + 1) <= v:
        e += 1
    spacing = Fraction(2) ** (max(e, -126) - 7)
    q = v / spacing
    frac = q - (q.numerator // q.denominator)
    return abs(frac - Fraction(1, 2)) * spacing / v


def dec_sqrt(q: Fraction) -> decimal.Decimal:
    with decimal.localcontext() as ctx:
        ctx.prec = PREC
        return (decimal.Decimal(q.numerator) / decimal.Decimal(q.denominator)).sqrt()


def dec_to_fraction(d: decimal.Decimal) -> Fraction:
    return Fraction(d)


def exact_rmsnorm_row(xs, ws, eps) -> list:
    """Exact-as-possible RMSNorm of one row of exact values (Fractions).

    mean(x^2) is exact; the square root and the division use ``PREC`` decimal
    digits. Returns a list of Fractions (pre-rounding values).
    """
    n = len(xs)
    ms = sum((x * x for x in xs), Fraction(0)) / n
    denom = ms + Fraction(eps)
    root = dec_sqrt(denom)
    out = []
    with decimal.localcontext() as ctx:
        ctx.prec = PREC
        for x, w in zip(xs, ws):
            num = x * w
            d = decimal.Decimal(num.numerator) / decimal.Decimal(num.denominator) / root
            out.append(Fraction(d))
    return out


def _dec(q: Fraction) -> decimal.Decimal:
    return decimal.Decimal(q.numerator) / decimal.Decimal(q.denominator)


def exact_layernorm_row(xs, ws, bs, eps) -> list:
    """LayerNorm of one row of exact values: exact mean and variance, 70-digit root."""
    n = len(xs)
    mu = sum(xs, Fraction(0)) / n
    var = sum(((x - mu) ** 2 for x in xs), Fraction(0)) / n
    root = dec_sqrt(var + Fraction(eps))
    out = []
    with decimal.localcontext() as ctx:
        ctx.prec = PREC
        for x, w, b in zip(xs, ws, bs):
            out.append(Fraction(_dec((x - mu) * w) / root) + b)
    return out


def exact_l2norm_row(xs, eps) -> list:
    """x / max(||x||_2, eps) for one row of exact values, 70-digit root."""
    ss = sum((x * x for x in xs), Fraction(0))
    root = dec_sqrt(ss)
    e = decimal.Decimal(Fraction(eps).numerator) / decimal.Decimal(Fraction(eps).denominator)
    with decimal.localcontext() as ctx:
        ctx.prec = PREC
        d = max(root, e)
        return [Fraction(_dec(x) / d) for x in xs]


def f16_fields_value(bits: int):
    """Exact value of an IEEE binary16 pattern from its fields (Fraction or float special)."""
    bits &= 0xFFFF
    sign = -1 if bits >> 15 else 1
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 0x1F:
        return float("nan") if f else float("inf") * sign
    if e == 0:
        return sign * Fraction(f, 1024) * Fraction(1, 2**14)
    return sign * (1 + Fraction(f, 1024)) * Fraction(2) ** (e - 15)


def round_exact_to_f16(v) -> int:
    """Round an exact rational to binary16 (nearest, ties to even); return the bits."""
    v = Fraction(v)
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    if a == 0:
        return sign
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    eff = max(e, -14)
    n = _round_half_even(a / Fraction(2) ** (eff - 10))
    if eff == -14 and n < 1024:  # subnormal (or zero)
        return sign | n
    if n == 2048:
        eff += 1
        n = 1024
    if eff > 15:
        return sign | 0x7C00
    return sign | ((eff + 15) << 10) | (n - 1024)
