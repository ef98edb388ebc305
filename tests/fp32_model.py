"""Exact model of FP32 arithmetic on the host, for checking instruction
sequences of the kernels on the CPU.

Every operation is carried out exactly on rationals and rounded once to the
nearest FP32 value, ties to even, with gradual underflow and overflow to
infinity (IEEE 754 binary32, the mode the kernels run in).  Values are Python
floats holding FP32 numbers (or +-inf / nan).  The native transcendental
instructions (reciprocal, exp2, log2) are approximations of at most about one
ulp; the model takes their correctly rounded value, and callers that depend
on the approximation also try the neighbouring FP32 values.

Test infrastructure: nothing here is used by the product path.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

INF = float("inf")
NAN = float("nan")
_TWO = Fraction(2)


def _frac(x) -> Fraction:
    return x if isinstance(x, Fraction) else Fraction(float(x))


def rn(q) -> float:
    """Round a rational (or a finite float) to the nearest FP32 value, ties to
    even; results of magnitude 2^128 - 2^103 and up become infinities."""
    q = _frac(q)
    if q == 0:
        return 0.0
    s = -1.0 if q < 0 else 1.0
    a = -q if q < 0 else q
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    while _TWO ** e > a:
        e -= 1
    while _TWO ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                  # subnormals share the quantum 2^-149
    quantum = _TWO ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= _TWO ** 128:
        return s * INF
    return s * float(val)


def is_fp32(x: float) -> bool:
    return math.isnan(x) or math.isinf(x) or float(np.float32(x)) == x


def _special(*xs):
    return any(math.isnan(x) or math.isinf(x) for x in xs)


def mul(a: float, b: float) -> float:
    if _special(a, b):
        return a * b
    return rn(_frac(a) * _frac(b))


def add(a: float, b: float) -> float:
    if _special(a, b):
        return a + b
    return rn(_frac(a) + _frac(b))


def fma(a: float, b: float, c: float) -> float:
    """a * b + c rounded once."""
    if _special(a, b, c):
        return a * b + c
    return rn(_frac(a) * _frac(b) + _frac(c))


def rcp(b: float) -> float:
    """Correctly rounded 1 / b (the native reciprocal is within an ulp of it)."""
    return rn(Fraction(1) / _frac(b))


def exp2(x: float) -> float:
    """2^x to FP32.  Exact where x is an integer; elsewhere the binary64 value
    rounded (the native instruction is within an ulp; callers here only use
    the result's magnitude and its being zero, finite or not)."""
    if math.isnan(x):
        return NAN
    if x == -INF or x < -160.0:
        return 0.0
    if x >= 128.0:
        return INF
    if x == int(x):
        return rn(_TWO ** int(x))
    return rn(Fraction(2.0 ** x))


def ulp_neighbours(x: float):
    """x and the FP32 values just below and above it."""
    f = np.float32(x)
    return (float(np.nextafter(f, np.float32(-np.inf))), float(f), float(np.nextafter(f, np.float32(np.inf))))


def frexp(x: float):
    """(mantissa in [1/2, 1), exponent) of a nonzero finite x, as v_frexp_mant / v_frexp_exp."""
    m, e = math.frexp(x)
    return m, e


def ldexp(x: float, e: int) -> float:
    if _special(x) or x == 0.0:
        return x
    return rn(_frac(x) * _TWO ** e)


def rint(x: float) -> float:
    return float(round(x)) if abs(x) < 2.0 ** 23 else x  # round() is ties-to-even
