"""OCP E4M3 ("fn" variant) codec -- test infrastructure, see ``oracle/__init__``.

The format, as [DF] part 1 "Per-tile FP8 scaling" and [TP] section V (FP8
detail 3, "E4M3 everywhere") describe it: one sign bit, four exponent bits,
three mantissa bits, largest magnitude 448, eight steps per binade.  Exponent
field 0 holds the subnormals m * 2^-9 (m = 0..7); field e = 1..15 holds
(1 + m/8) * 2^(e-7), except that S.1111.111 is NaN (there is no infinity).
That gives 127 non-negative finite values, 2^-9 .. 448.

Rounding (the plainest reading of [DF]'s emulator, which rounds the scaled
value half-to-even on a grid of step 2^(e-3) with e clamped to [-6, 8]):
round to nearest, ties to the even code, magnitudes above 448 saturate to 448,
the sign of the input is kept (so -0.0 and tiny negatives give 0x80).  Codes
0x7F and 0xFF are never produced.

The encoder is written twice, independently: ``encode_search`` looks the value
up in the table of representable values; ``encode_arith`` derives the code from
the binary exponent.  Tests require the two to agree.
"""
import numpy as np

MAX_E4M3 = 448.0
NAN_CODES = (0x7F, 0xFF)


def _decode_one(c):
    s = -1.0 if (c >> 7) & 1 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: value of every byte code, float64 (NaN for 0x7F and 0xFF)
TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
#: the 127 non-negative finite values, in code order (which is value order)
POS_VALUES = TABLE[:127].copy()


def decode(codes):
    """Byte codes -> float64 values."""
    return TABLE[np.asarray(codes, dtype=np.uint8)]


def encode_search(v):
    """Nearest representable value by table search; ties to the even code."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    i = np.searchsorted(POS_VALUES, a, side="left")   # POS[i-1] < a <= POS[i]
    hi = np.minimum(i, 126)
    lo = np.maximum(i - 1, 0)
    d_hi = POS_VALUES[hi] - a
    d_lo = a - POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= MAX_E4M3, 126, code)          # saturate
    code = np.where(a == 0.0, 0, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def encode_arith(v):
    """Code from the binary exponent: step 2^(e-3) for e = floor(log2|v|) in
    [-6, 8]; a fixed step of 2^-9 below 2^-6 (the subnormals)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    mant, ex = np.frexp(a)                    # a = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1               # floor(log2 a) for a > 0
    normal = a >= 2.0 ** -6
    e_n = np.minimum(e, 8)
    q_n = np.rint(np.ldexp(np.minimum(a, 1024.0), -(e_n - 3)))  # exact, half-even
    carry = q_n >= 16                          # rounded up into the next binade
    e_n = np.where(carry, e_n + 1, e_n)
    q_n = np.where(carry, 8, q_n)
    code_n = ((e_n + 7) << 3) | (q_n.astype(np.int64) - 8)
    code_n = np.where((e_n > 8) | ((e_n == 8) & (q_n > 14)), 126, code_n)
    q_s = np.rint(np.ldexp(np.minimum(a, 1.0), 9)).astype(np.int64)  # 0..8 below 2^-6
    code = np.where(normal, code_n, q_s)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


encode = encode_search


def round_to_e4m3(v):
    """The value an input rounds to, float64."""
    return decode(encode(v))
