"""Exact rational rounding to binary floating-point formats (test helper).

Independent of the oracle and of the library: values are converted to
Fractions and rounded to nearest, ties to even, with Python's exact integer
arithmetic, so a pin built on it cannot share a rounding slip with the code
it checks.
"""
from fractions import Fraction

import numpy as np

from gqa_kv_cache_decode_amd import inputs


def frac_round(x: Fraction, mant_bits: int, min_exp: int, max_exp: int):
    """x rounded to a binary float with mant_bits significant bits, nearest even.

    Exponents of the leading bit from min_exp (subnormals below) to max_exp;
    returns a Fraction, or None on overflow to infinity.
    """
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    # a in [2^e, 2^(e+1)); last kept bit has weight 2^(e - mant_bits + 1)
    q = Fraction(2) ** (max(e, min_exp) - mant_bits + 1)
    n, r = divmod(a, q)
    if r > q / 2 or (r == q / 2 and n % 2 == 1):
        n += 1
    v = n * q
    if v >= Fraction(2) ** (max_exp + 1):
        return None
    return sign * v


def bf16_bits(v):
    """bf16 bit pattern of an exactly representable Fraction (None: +inf)."""
    if v is None:
        return 0x7F80  # overflow of a positive value
    return int(inputs.f32_to_bf16_bits(np.array([float(v)], dtype=np.float32))[0])


def bf16_value(bits):
    return Fraction(float(inputs.bf16_bits_to_f32(np.array([bits], dtype=np.uint16))[0]))


def round_bf16_exact(x: float) -> int:
    """The double x rounded once to bf16 (nearest even), as a bit pattern; the sign is kept (also of zero)."""
    sign = 0x8000 if np.signbit(x) else 0
    want = frac_round(abs(Fraction(float(x))), 8, -126, 127)
    return (0x7F80 if want is None else bf16_bits(want)) | sign
