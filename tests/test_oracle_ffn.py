"""Pins of the oracle's block-scaled FP8 GEMM, SwiGLU expert and combine.

Sources: "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
Prediction, and FP8 Training at 671B Scale", section V (Figure 6: FP8 inputs,
FP32 accumulation, BF16 outputs; FP8 detail 1: 1x128 / 128x128 scales) and
section II (each token uses the shared expert plus its routed experts);
"DeepSeek-V3, explained.", glossary (the shared expert is added at full
weight, routed weights sum to 1).
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import e4m3, ffn, quant

ONE = int(e4m3.encode(1.0))


def _int_codes(rng, shape, lo=-8, hi=8):
    """Codes of integer values in [lo, hi] (all exactly representable)."""
    ints = rng.integers(lo, hi + 1, shape)
    return e4m3.encode(ints.astype(np.float64)), ints.astype(np.int64)


@pytest.mark.parametrize("R,N,K", [(5, 128, 384), (130, 256, 128), (1, 384, 512)])
def test_single_scale_reduces_to_integer_matmul(R, N, K):
    rng = np.random.default_rng(R + N + K)
    aq, ai = _int_codes(rng, (R, K))
    bq, bi = _int_codes(rng, (N, K))
    ad = np.full((R, K // 128), 2.0 ** -3, np.float32)
    bd = np.full((N // 128, K // 128), 2.0 ** -5, np.float32)
    got = ffn.block_scaled_gemm(aq, ad, bq, bd)
    want = (ai @ bi.T).astype(np.float64) * 2.0 ** -8          # exact integers
    np.testing.assert_array_equal(got, want)


def test_block_scales_enter_per_row_and_per_column_block():
    R, N, K = 3, 256, 384
    rng = np.random.default_rng(1)
    aq = np.full((R, K), ONE, np.uint8)
    bq = np.full((N, K), ONE, np.uint8)
    ad = rng.uniform(0.5, 2, (R, K // 128)).astype(np.float32)
    bd = rng.uniform(0.5, 2, (N // 128, K // 128)).astype(np.float32)
    got = ffn.block_scaled_gemm(aq, ad, bq, bd)
    for r in range(R):
        for c in (0, 127, 128, 255):
            want = sum(128.0 * float(ad[r, kb]) * float(bd[c // 128, kb]) for kb in range(3))
            assert abs(got[r, c] - want) <= 1e-12 * want


def test_scale_of_one_block_only_touches_that_block():
    R, N, K = 2, 128, 256
    rng = np.random.default_rng(2)
    aq, ai = _int_codes(rng, (R, K))
    aq[:, 128:] = 0
    ai[:, 128:] = 0
    bq, bi = _int_codes(rng, (N, K))
    ad = np.array([[0.25, 1e30], [0.5, 1e30]], np.float32)   # block 1 scales are huge
    bd = np.array([[2.0, 1e30]], np.float32)
    got = ffn.block_scaled_gemm(aq, ad, bq, bd)
    want = (ai[:, :128] @ bi[:, :128].T) * np.array([[0.5], [1.0]])
    np.testing.assert_array_equal(got, want)


def test_silu_closed_forms():
    v = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(ffn.silu64(v), v * expit(v), rtol=1e-14, atol=1e-300)
    assert ffn.silu64(np.array([0.0]))[0] == 0.0
    v32 = ffn.fl32(v)
    np.testing.assert_allclose(ffn.silu32(v32), ffn.silu64(v32), rtol=3e-7, atol=1e-30)


def test_bf16_rounding():
    e = 2.0 ** -7
    vals = np.array([1.0 + e / 2, 1.0 + 1.5 * e, 1.0 + 0.49 * e, -(1.0 + e / 2), 3.0])
    want = np.array([1.0, 1.0 + 2 * e, 1.0, -1.0, 3.0])
    np.testing.assert_array_equal(ffn.bf16_round(vals), want)


def _const_expert(H, I, dx, dg, du, dw2):
    """Codes of 1.0 everywhere; W1 = [gate; up] with per-block scales."""
    xq = np.full((len(dx), H), ONE, np.uint8)
    xd = np.array(dx, np.float32)
    w1q = np.full((2 * I, H), ONE, np.uint8)
    w1d = np.zeros((2 * I // 128, H // 128), np.float32)
    w1d[: I // 128] = dg
    w1d[I // 128:] = du
    w2q = np.full((H, I), ONE, np.uint8)
    w2d = np.full((H // 128, I // 128), dw2, np.float32)
    return xq, xd, w1q, w1d, w2q, w2d


def test_swiglu_expert_closed_form_and_gate_up_order():
    H, I = 256, 128
    dx = [[0.01, 0.02], [0.005, 0.0]]
    dg, du, dw2 = 0.03, -0.07, 0.002
    res = ffn.expert_ffn(*_const_expert(H, I, dx, dg, du, dw2), precision="D")
    for r in range(2):
        a_g = 128 * sum(dx[r]) * np.float64(np.float32(dg))
        a_u = 128 * sum(dx[r]) * np.float64(np.float32(du))
        a_g = sum(128 * float(np.float32(d)) * float(np.float32(dg)) for d in dx[r])
        a_u = sum(128 * float(np.float32(d)) * float(np.float32(du)) for d in dx[r])
        h = a_g * expit(a_g) * a_u
        np.testing.assert_allclose(res["a"][r, :I], a_g, rtol=1e-14)
        np.testing.assert_allclose(res["a"][r, I:], a_u, rtol=1e-14)
        np.testing.assert_allclose(res["h"][r], h, rtol=1e-7)
        assert np.all(res["hq"][r] == e4m3.encode(np.sign(h) * 448.0))
        hd = np.float32(abs(np.float32(h)) / 448.0)
        assert res["hd"][r, 0] == hd
        out = 128 * np.sign(h) * 448.0 * float(hd) * float(np.float32(dw2))
        np.testing.assert_allclose(res["out"][r], out, rtol=1e-14)
    # swapping gate and up changes the result: the order is pinned
    swapped = ffn.expert_ffn(*_const_expert(H, I, dx, du, dg, dw2), precision="D")
    assert not np.allclose(swapped["h"][0], res["h"][0], rtol=1e-3)


def test_zero_input_gives_exact_zero():
    H, I = 256, 128
    rng = np.random.default_rng(3)
    w1 = rng.standard_normal((2 * I, H)) * 0.02
    w2 = rng.standard_normal((H, I)) * 0.02
    w1q, w1d = quant.quant_128x128(ffn.fl32(w1))
    w2q, w2d = quant.quant_128x128(ffn.fl32(w2))
    xq, xd = quant.quant_1x128(np.zeros((4, H)))
    for p in ("D", "Q"):
        res = ffn.expert_ffn(xq, xd, w1q, w1d, w2q, w2d, p)
        assert np.all(res["out"] == 0.0) and np.all(res["hq"] == 0) and np.all(res["hd"] == 1.0)


def test_combine_closed_form():
    out = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0], [0.5, -0.5], [0.25, 0.75]])
    gate = np.array([[0.75, 0.25], [1.0, 0.0]])
    row_of = np.array([[0, 2], [1, 0]])
    y = ffn.combine(out, gate, row_of, 3, "D")
    np.testing.assert_array_equal(y, [[0.5 + 0.75 + 25.0, -0.5 + 1.5 + 50.0],
                                      [0.25 + 10.0, 0.75 + 20.0]])
    yq = ffn.combine(out, gate, row_of, 3, "Q")
    np.testing.assert_array_equal(yq, ffn.bf16_round(y))


def test_combine_k1_and_no_shared():
    rng = np.random.default_rng(4)
    out = ffn.bf16_round(rng.standard_normal((6, 8)))
    row_of = np.array([[2], [0], [1]])
    y = ffn.combine(out, np.ones((3, 1)), row_of, 3, "D")
    np.testing.assert_array_equal(y, out[3:6] + out[[2, 0, 1]])
    y0 = ffn.combine(out, np.full((3, 1), 0.5), row_of, -1, "D")
    np.testing.assert_array_equal(y0, 0.5 * out[[2, 0, 1]])
