"""Exact rational arithmetic for pinning the oracle's rounding points.

Independent of ``oracle/``: every value is a ``fractions.Fraction`` and every
rounding is written out here from the definition of a binary floating-point
format (round to nearest, ties to the even significand), so a test can work a
float32 / bfloat16 / E4M3 chain step by step and compare the oracle's NumPy
evaluation with it bit for bit.  ``exp`` comes from the ``decimal`` module at
60 significant digits, far more than the 24 bits a float32 rounding needs
(``rn`` refuses to decide when a value lies closer to a rounding midpoint than
that precision can resolve).
"""
from decimal import Decimal, localcontext
from fractions import Fraction

#: relative precision of the exp values below (60 decimal digits)
EXP_REL_ERR = Fraction(1, 10 ** 55)


def _exponent(a):
    """floor(log2(a)) for a rational a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rn(q, p, emin, err=Fraction(0)):
    """Round the rational q to the nearest value of a binary format with a
    p-bit significand (implicit bit included) whose smallest normal exponent
    is emin (values below 2^emin share the spacing 2^(emin - p + 1)); ties go
    to the even significand.  No upper limit.  ``err`` is a relative
    uncertainty of q: rounding is refused (AssertionError) if q might lie on
    the other side of a midpoint."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_exponent(a), emin)
    ulp = Fraction(2) ** (e - (p - 1))
    n = a / ulp
    f = n.numerator // n.denominator
    r = n - f
    if err:
        assert abs(r - Fraction(1, 2)) * ulp > err * a, "too close to a rounding midpoint"
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return sign * f * ulp


def rn32(q, err=Fraction(0)):
    """float32: 24-bit significand, smallest normal 2^-126."""
    return rn(q, 24, -126, err)


def rn_bf16(q):
    """bfloat16: 8-bit significand, smallest normal 2^-126."""
    return rn(q, 8, -126)


def rn_e4m3(q):
    """OCP E4M3 ("fn"): 4-bit significand, smallest normal 2^-6 (subnormal
    step 2^-9); magnitudes that round above 448 saturate to 448."""
    v = rn(q, 4, -6)
    return max(min(v, Fraction(448)), Fraction(-448))


def e4m3_value(code):
    """Value of an E4M3 byte code, written from the format's bit fields."""
    code = int(code)
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    assert not (e == 15 and m == 7), "NaN code"
    if e == 0:
        return s * Fraction(m, 512)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def exp(q):
    """e^q as a rational, to 60 significant decimal digits."""
    q = Fraction(q)
    with localcontext() as ctx:
        ctx.prec = 60
        return Fraction((Decimal(q.numerator) / Decimal(q.denominator)).exp())


def f32(x):
    """A float32-representable float (or numpy scalar) as a Fraction."""
    return Fraction(float(x))
