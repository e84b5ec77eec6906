"""Pins of the rounding-faithful ("Q") oracle chain against exact rational
arithmetic.

The "Q" precision of the oracle reproduces every rounding point of the FP8
expert path: the block-scaled GEMM result rounded to float32, SiLU with each
float32 operation rounded, the SwiGLU product rounded to float32, the 1x128
requantisation of h (m = fl32(448 / amax), d = fl32(amax / 448),
code = E4M3(fl32(h * m))), the expert output rounded to bfloat16, and the
combine as float32 fused multiply-adds in slot order from the shared row
("DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction,
and FP8 Training at 671B Scale", section V, Figure 6 and FP8 details 1-2;
"DeepSeek-V3 Technical Report" (deepforge), part 1 "Per-tile FP8 scaling";
"DeepSeek-V3, explained.", glossary).

Here each chain is worked with ``fractions.Fraction`` and roundings written
from the formats' definitions (tests/exact.py), and the oracle's NumPy
evaluation must equal it bit for bit.  Each test also shows that its inputs
discriminate: dropping or moving any one rounding point changes a result on
them, so a mistake of that kind in the oracle would fail the test.
"""
from fractions import Fraction

import numpy as np

import exact as X
from oracle import e4m3, ffn

# Where NumPy's float64 evaluation of a step is not exact (exp, a division, the
# float64 GEMM accumulation) it is within 2^-45 of the exact value, so the
# float32 rounding of that step is decided only when the exact value lies
# farther than that from a rounding midpoint.  Products and sums of float32
# values are exact in float64 and need no margin (they may fall on a tie).
MARGIN = Fraction(1, 2 ** 45)


def _silu32_exact(v, drop=None):
    """SiLU of a float32 value v with each float32 operation rounded:
    e = fl32(exp(-v)), den = fl32(1 + e), sg = fl32(1 / den), out = fl32(v sg).
    ``drop`` names one rounding to leave out (to show the inputs see it)."""
    def r(q, name, err=Fraction(0)):
        return q if drop == name else X.rn32(q, err)
    e = r(X.exp(-v), "e", MARGIN)
    den = r(1 + e, "den")
    sg = r(1 / den, "sg", MARGIN)
    return r(v * sg, "out")


def _silu_inputs():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.uniform(-20, 20, 400), rng.standard_normal(400) * 3,
                        np.exp(rng.uniform(-12, 3, 200)) * rng.choice([-1, 1], 200),
                        [0.0, -0.0, 1.0, -1.0, 88.0, -87.0]])
    return v.astype(np.float32).astype(np.float64)


def test_silu32_equals_the_exact_float32_chain():
    v = _silu_inputs()
    got = ffn.silu32(v)
    want = np.array([float(_silu32_exact(X.f32(x))) for x in v])
    assert np.array_equal(got, want)
    # the inputs discriminate: leaving out any one of the four roundings
    # changes the float32 result on some of them
    for drop in ("e", "den", "sg"):
        alt = np.array([float(X.rn32(_silu32_exact(X.f32(x), drop))) for x in v])
        assert np.count_nonzero(alt != want) > 0, drop
    unrounded = [_silu32_exact(X.f32(x), "out") for x in v]
    assert sum(q != X.rn32(q) for q in unrounded) > 0
    # and float64 SiLU rounded once differs from the float32 chain somewhere
    assert np.count_nonzero(ffn.fl32(ffn.silu64(v)) != want) > 0


def _e4m3_int(codes):
    """E4M3 codes -> their values times 2^9 (integers), from the bit fields."""
    return np.array([int(X.e4m3_value(c) * 512) for c in range(256) if c not in (0x7F, 0xFF)]
                    + [0, 0], np.int64)[_code_index(codes)]


def _code_index(codes):
    # position of each code in the list built above (NaN codes never occur)
    idx = np.asarray(codes, np.int64)
    return np.where(idx < 0x7F, idx, np.where(idx < 0xFF, idx - 1, 254))


def _random_codes(rng, shape):
    c = rng.integers(0, 256, shape)
    c = np.where((c & 0x7F) == 0x7F, c - 1, c)          # no NaN codes
    return c.astype(np.uint8)


def _block_gemm_exact(aq, ad, bq, bd, magnitude=False):
    """sum_kb (sum_{h in kb} v(A) v(B)) d_A[r, kb] d_B[c // 128, kb] exactly:
    the block sums on the integer grid of 2^-9 (int64 matmul, exact), the
    scales as Fractions.  With ``magnitude`` also returns the same sum over
    |block sum| (what a float64 evaluation's rounding error is relative to)."""
    ai = _e4m3_int(aq)
    bi = _e4m3_int(bq)
    R, K = ai.shape
    N = bi.shape[0]
    out = [[Fraction(0)] * N for _ in range(R)]
    mag = [[Fraction(0)] * N for _ in range(R)]
    for kb in range(K // 128):
        s = ai[:, kb * 128:(kb + 1) * 128] @ bi[:, kb * 128:(kb + 1) * 128].T
        for r in range(R):
            for c in range(N):
                t = Fraction(int(s[r, c]), 2 ** 18) * X.f32(ad[r, kb]) * X.f32(bd[c // 128, kb])
                out[r][c] += t
                mag[r][c] += abs(t)
    return (out, mag) if magnitude else out


def _rn32_of_sum(v, mag):
    """float32 rounding of an exact sum whose float64 evaluation may be off
    by up to 2^-45 of the sum of magnitudes."""
    return X.rn32(v, MARGIN * mag / abs(v) if v else Fraction(0))


def _expert_case():
    rng = np.random.default_rng(5)
    R, H, I = 3, 256, 128
    xq = _random_codes(rng, (R, H))
    xd = rng.uniform(2 ** -9, 2 ** -6, (R, H // 128)).astype(np.float32)
    w1q = _random_codes(rng, (2 * I, H))
    w1d = rng.uniform(2 ** -14, 2 ** -11, (2 * I // 128, H // 128)).astype(np.float32)
    w2q = _random_codes(rng, (H, I))
    w2d = rng.uniform(2 ** -12, 2 ** -9, (H // 128, I // 128)).astype(np.float32)
    return xq, xd, w1q, w1d, w2q, w2d


def _q_chain_exact(case, a_round=True):
    xq, xd, w1q, w1d, w2q, w2d = case
    a, amag = _block_gemm_exact(xq, xd, w1q, w1d, magnitude=True)
    R = len(a)
    I = len(a[0]) // 2
    a32 = [[_rn32_of_sum(v, mg) if a_round else v for v, mg in zip(row, mrow)]
           for row, mrow in zip(a, amag)]
    h = [[X.rn32(_silu32_exact(X.rn32(a32[r][c])) * a32[r][I + c])
          for c in range(I)] for r in range(R)]
    hq_val, hd = [], []
    for r in range(R):                                     # I = 128: one tile per row
        amax = max(abs(v) for v in h[r])
        m = X.rn32(Fraction(448) / amax, MARGIN)
        hd.append(X.rn32(amax / Fraction(448), MARGIN))
        hq_val.append([X.rn_e4m3(X.rn32(v * m)) for v in h[r]])
    return dict(a=a, h=h, hq_val=hq_val, hd=hd)


def test_expert_ffn_q_equals_the_exact_chain():
    case = _expert_case()
    xq, xd, w1q, w1d, w2q, w2d = case
    res = ffn.expert_ffn(*case, precision="Q")
    ref = _q_chain_exact(case)
    R, I = len(ref["h"]), len(ref["h"][0])
    # GEMM1 in float64 is the exact block sum to float64 accuracy (relative
    # to the sum of the terms' magnitudes)
    a_exact = np.array([[float(v) for v in row] for row in ref["a"]])
    a_mag = np.array([[float(v) for v in row]
                      for row in _block_gemm_exact(xq, xd, w1q, w1d, magnitude=True)[1]])
    assert np.all(np.abs(res["a"] - a_exact) <= 1e-15 * a_mag)
    # h: float32 SwiGLU of the float32-rounded GEMM result, bit for bit
    h_want = np.array([[float(v) for v in row] for row in ref["h"]])
    assert np.array_equal(res["h"], h_want)
    # requantisation: scales and code values exact
    assert np.array_equal(res["hd"][:, 0].astype(np.float64), [float(d) for d in ref["hd"]])
    got_vals = [[X.e4m3_value(c) for c in row] for row in res["hq"]]
    assert got_vals == ref["hq_val"]
    # GEMM2 over those codes, rounded to float32 and then to bfloat16
    hq = res["hq"]
    out_exact, out_mag = _block_gemm_exact(hq, res["hd"], w2q, w2d, magnitude=True)
    out32 = [[_rn32_of_sum(v, mg) for v, mg in zip(row, mrow)] for row, mrow in zip(out_exact, out_mag)]
    out_want = np.array([[float(X.rn_bf16(v)) for v in row] for row in out32])
    assert np.array_equal(res["out"], out_want)

    # the inputs discriminate:
    # (1) without the float32 rounding of the GEMM result, h changes
    h_noround = _q_chain_exact(case, a_round=False)["h"]
    n1 = sum(h_noround[r][c] != ref["h"][r][c] for r in range(R) for c in range(I))
    assert n1 > 0
    # (2) the float64 expert ("D") gives a different h and output here
    resd = ffn.expert_ffn(*case, precision="D")
    assert np.count_nonzero(resd["h"] != res["h"]) > 0
    # (3) the bf16 rounding of the output matters on these rows
    out_f32 = np.array([[float(v) for v in row] for row in out32])
    assert np.count_nonzero(out_f32 != out_want) > 0
    # (4) gate and up are not interchangeable
    swapped = (xq, xd, np.concatenate([w1q[I:], w1q[:I]]),
               np.concatenate([w1d[1:], w1d[:1]]), w2q, w2d)
    assert not np.array_equal(ffn.expert_ffn(*swapped, precision="Q")["h"], res["h"])


def _combine_exact(out_rows, gate, row_of, shared_row0, fused=True, order=None):
    T, k = row_of.shape
    H = out_rows.shape[1]
    y = np.zeros((T, H))
    for t in range(T):
        for c in range(H):
            acc = X.f32(out_rows[shared_row0 + t, c])
            for j in (order or range(k)):
                g = X.f32(np.float32(gate[t, j]))
                o = X.f32(out_rows[row_of[t, j], c])
                acc = X.rn32(acc + g * o) if fused else X.rn32(acc + X.rn32(g * o))
            y[t, c] = float(X.rn_bf16(acc))
    return y


def test_combine_q_equals_the_exact_fma_chain():
    rng = np.random.default_rng(9)
    T, k, H = 16, 4, 64
    R = T * k + T
    out_rows = ffn.bf16_round(rng.standard_normal((R, H)) * np.exp(rng.uniform(-3, 3, (R, 1))))
    gate = rng.dirichlet(np.ones(k), T).astype(np.float32)
    row_of = rng.permutation(T * k).reshape(T, k).astype(np.int64)
    # one element where the slot order decides the float32 sum: terms
    # 2^8, 2^-18, -2^8, 2^-18 from a zero shared row (2^-18 is below half an
    # ulp of 2^8, so it survives only when added after the cancellation)
    gate[0] = 0.25
    out_rows[T * k + 0, 0] = 0.0
    for j, v in enumerate((2.0 ** 10, 2.0 ** -16, -2.0 ** 10, 2.0 ** -16)):
        out_rows[row_of[0, j], 0] = v
    # and one where only a fused multiply-add keeps the low bits of g * o:
    # shared -(1 + 2^-7), gate 1 + 2^-23, slot value 1 + 2^-7, other slots 0
    gate[1, 0] = np.float32(1.0 + 2.0 ** -23)
    out_rows[T * k + 1, 0] = -(1.0 + 2.0 ** -7)
    out_rows[row_of[1, 0], 0] = 1.0 + 2.0 ** -7
    for j in range(1, k):
        out_rows[row_of[1, j], 0] = 0.0
    got = ffn.combine(out_rows, gate, row_of, T * k, "Q")
    want = _combine_exact(out_rows, gate, row_of, T * k)
    assert np.array_equal(got, want)
    # a separately rounded product, or another slot order, gives other bits
    assert np.count_nonzero(_combine_exact(out_rows, gate, row_of, T * k, fused=False) != want) > 0
    rev = list(range(k))[::-1]
    assert np.count_nonzero(_combine_exact(out_rows, gate, row_of, T * k, order=rev) != want) > 0


def test_exact_helpers_against_known_values():
    """The rational rounding helpers themselves, on values with known
    answers (so the pins above rest on something checked)."""
    assert X.rn32(Fraction(1) + Fraction(1, 2 ** 24)) == 1                     # tie to even
    assert X.rn32(Fraction(1) + Fraction(3, 2 ** 24)) == 1 + Fraction(1, 2 ** 22)
    assert X.rn32(Fraction(1, 3)) == Fraction(float(np.float32(1 / 3)))
    assert X.rn32(Fraction(2) ** -149 * Fraction(3, 2)) == Fraction(2) ** -148  # subnormal tie
    assert X.rn_bf16(Fraction(1) + Fraction(1, 2 ** 8)) == 1
    assert X.rn_bf16(Fraction(1) + Fraction(3, 2 ** 8)) == 1 + Fraction(1, 2 ** 6)
    assert X.rn_e4m3(Fraction(460)) == 448 and X.rn_e4m3(Fraction(470)) == 448
    assert X.rn_e4m3(Fraction(3, 2 ** 10)) == Fraction(2, 2 ** 9)              # subnormal tie
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert float(X.e4m3_value(c)) == e4m3.TABLE[c] or (c == 0x80 and e4m3.TABLE[c] == 0)
    assert abs(X.exp(Fraction(1)) - Fraction("2.718281828459045235360287471352662497757")) \
        < Fraction(1, 10 ** 38)
