"""Exact rational brute force of the BitDelta definitions, for tiny inputs.

An independent pin for the C oracle: every value is decoded from its bit
fields into a ``fractions.Fraction``, sums are exact, and rounding to fp32 /
bf16 is done by comparing exact rationals against the representable
neighbours (round to nearest, ties to even), not by bit manipulation.

Definitions from "BitDelta : servir 14 modèles Zen depuis un seul cluster
GPU" (hanzo-blog, 2026-02-28): "Mathematical foundation" (Δ's sign, α as the
mean absolute delta), "Serving architecture" (W_eff = W_base + α·sign(Δ),
y = x·W_effᵀ), "Infrastructure details" (8 signs per byte, fp32 α per output
dimension).  Readings as in the oracle: sign(0) = +1, LSB-first bytes, fp32
sum rounded once to bf16.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction


def f32_value(bits: int) -> Fraction:
    """Exact value of a finite fp32 bit pattern."""
    sign = -1 if (bits >> 31) & 1 else 1
    exp = (bits >> 23) & 0xFF
    man = bits & 0x7FFFFF
    if exp == 0xFF:
        raise ValueError("not finite")
    if exp == 0:
        return sign * Fraction(man, 1 << 149)
    return sign * Fraction((1 << 23) | man) * Fraction(2) ** (exp - 150)


def bf16_value(bits: int) -> Fraction:
    return f32_value((bits & 0xFFFF) << 16)


def float_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def _round_to(v: Fraction, mant_bits: int, emin: int, emax: int):
    """Round v to a binary format with mant_bits significand bits (incl. the
    hidden one), minimum normal exponent emin, maximum exponent emax.
    Returns the rounded Fraction or +-inf (as a float)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q = a / ulp
    lo = math.floor(q)
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    largest = (Fraction(2) - Fraction(2) ** (1 - mant_bits)) * Fraction(2) ** emax
    if r > largest:
        return sign * math.inf
    return sign * r


def round_f32(v: Fraction):
    return _round_to(v, 24, -126, 127)


def round_bf16(v: Fraction):
    return _round_to(v, 8, -126, 127)


def sign_bit(delta: float) -> int:
    """1 encodes +1, 0 encodes -1; zero of either sign encodes +1."""
    return 0 if Fraction(delta) < 0 else 1


def pack_row(deltas):
    """LSB-first bytes of one row of finite floats (length a multiple of 8)."""
    out = []
    for j in range(0, len(deltas), 8):
        byte = 0
        for b in range(8):
            byte += sign_bit(deltas[j + b]) * (2 ** b)
        out.append(byte)
    return out


def delta_pair(ft_bits: int, base_bits: int):
    """Δ = W_ft − W_base of two bf16 patterns: the exact difference, rounded
    once to fp32 (nearest, ties to even)."""
    return round_f32(bf16_value(ft_bits) - bf16_value(base_bits))


def alpha_exact(values) -> Fraction:
    """Exact mean of |Δ| over the given floats."""
    return sum((abs(Fraction(v)) for v in values), Fraction(0)) / len(values)


def weff(wbase_bits: int, bit: int, alpha_f32: float):
    """W_eff value: fp32 sum of the bf16 base and ±α, rounded once to bf16."""
    w = bf16_value(wbase_bits)
    a = Fraction(alpha_f32)
    s = round_f32(w + (a if bit else -a))
    if isinstance(s, float):
        return s
    return round_bf16(s)


def linear(x_bits, w_bits, signs, alpha_vals, per_row: bool):
    """Exact y[m][n] as Fractions; x_bits [M][K], w_bits [N][K] are bf16
    patterns, signs [N][K/8] bytes, alpha_vals fp32 floats ([N] or [1])."""
    n_out = len(w_bits)
    k = len(w_bits[0])
    weffs = []
    for n in range(n_out):
        a = alpha_vals[n] if per_row else alpha_vals[0]
        row = []
        for kk in range(k):
            bit = (signs[n][kk // 8] >> (kk % 8)) & 1
            row.append(weff(w_bits[n][kk], bit, a))
        weffs.append(row)
    y = []
    for xrow in x_bits:
        xs = [bf16_value(v) for v in xrow]
        y.append([sum((xs[kk] * weffs[n][kk] for kk in range(k)), Fraction(0))
                  for n in range(n_out)])
    return y, weffs
