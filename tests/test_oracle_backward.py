"""Pins of the oracle's FP8 backward GEMMs (Dgrad, Wgrad) and its token-tile
quantiser.

Source: "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
Prediction, and FP8 Training at 671B Scale", section V, Figure 6 (forward,
input-gradient and weight-gradient GEMMs of a linear layer all in FP8 with
FP32 accumulation) and details 1-4; "DeepSeek-V3 Technical Report"
(deepforge), part 1 "FP8 training, from first principles".  The products are
pinned against the exact float64 products of operands the quantisers
reproduce exactly, against the E4M3 rounding bound on random operands, and
against element-by-element loops; the token-tile quantiser against the 1x128
quantiser on transposed blocks and a per-tile loop.
"""
import numpy as np

from oracle import backward, e4m3, quant


def _exact_values(rng, rows, cols, exps, brows, bcols):
    """Values E4M3 holds exactly once divided by their block's power of two:
    random finite codes with one +448 per (brows x bcols) block, block (i, j)
    scaled by 2^exps[i, j], so every quantiser block this test uses sees
    amax = 448 * 2^p and reproduces the values exactly."""
    codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, codes & 0xF0, codes).astype(np.uint8)
    v = e4m3.decode(codes)
    for i in range(rows // brows):
        for j in range(cols // bcols):
            v[i * brows, j * bcols] = 448.0
    return v * np.repeat(np.repeat(2.0 ** np.asarray(exps, np.float64), brows, 0), bcols, 1)


def test_transpose_blocks_is_the_transposed_weight():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((2, 256, 384)) * np.exp2(rng.integers(-8, 0, (2, 1, 1)))
    wq, wd = quant.quant_128x128(w)
    tq, td = backward.transpose_blocks(wq, wd)
    assert tq.shape == (2, 384, 256) and td.shape == (2, 3, 2)
    np.testing.assert_array_equal(quant.dequant_128x128(tq, td),
                                  np.swapaxes(quant.dequant_128x128(wq, wd), -1, -2))
    # quantising the transposed weight gives the same codes and scales
    q2, d2 = quant.quant_128x128(np.swapaxes(w, -1, -2))
    np.testing.assert_array_equal(q2, tq)
    np.testing.assert_array_equal(d2, td)


def test_dgrad_exact_on_e4m3_operands():
    rng = np.random.default_rng(2)
    R, N, K = 48, 256, 384
    dy = _exact_values(rng, R, N, rng.integers(-12, -4, (R, N // 128)), 1, 128)
    w = _exact_values(rng, N, K, rng.integers(-14, -8, (N // 128, K // 128)), 128, 128)
    wq, wd = quant.quant_128x128(w)
    dx, dyq, dyd = backward.dgrad(dy, wq, wd)
    exact = dy @ w
    scale = np.abs(dy) @ np.abs(w)
    assert np.max(np.abs(dx - exact) / scale) < 1e-13


def test_dgrad_within_the_e4m3_error_bound():
    rng = np.random.default_rng(3)
    R, N, K = 64, 384, 256
    dy = rng.standard_normal((R, N)) * np.exp2(rng.integers(-6, 6, (R, N // 128))).repeat(128, 1)
    w = rng.standard_normal((N, K)) * np.exp2(rng.integers(-9, -3, (N // 128, K // 128))).repeat(128, 0).repeat(128, 1)
    wq, wd = quant.quant_128x128(w)
    dx, _, _ = backward.dgrad(dy, wq, wd)
    ddy = np.abs(dy).reshape(R, N // 128, 128).max(2) / 448.0
    dw = np.abs(w).reshape(N // 128, 128, K // 128, 128).max((1, 3)) / 448.0
    e_dy = np.abs(dy) * (2.0 ** -4 + 2.0 ** -20) + ddy.repeat(128, 1) * 2.0 ** -10 * (1 + 1e-6)
    e_w = np.abs(w) * (2.0 ** -4 + 2.0 ** -20) + dw.repeat(128, 0).repeat(128, 1) * 2.0 ** -10 * (1 + 1e-6)
    bound = e_dy @ np.abs(w) + (np.abs(dy) + e_dy) @ e_w
    ratio = np.abs(dx - dy @ w) / bound
    assert np.max(ratio) <= 1.0 and np.max(ratio) > 1e-3


def test_padded_offsets_and_layout():
    off = np.array([0, 0, 130, 258, 259, 259, 600])
    pad = backward.padded_offsets(off)
    np.testing.assert_array_equal(pad, [0, 0, 256, 384, 512, 512, 896])
    rng = np.random.default_rng(4)
    x = rng.standard_normal((600, 128))
    xq, xd, p2 = backward.quant_tokens(x, off)
    np.testing.assert_array_equal(p2, pad)
    assert xq.shape == (128, 896) and xd.shape == (128, 7)
    # padding positions hold code 0; real positions hold the token's code
    assert np.all(xq[:, 130:256] == 0) and np.all(xq[:, 384 + 1:512] == 0)
    # group 3 has one token (row 258): its tile's amax is that token alone
    np.testing.assert_array_equal(xd[:, 3], (np.abs(x[258]) / 448.0).astype(np.float32))


def test_quant_tokens_equals_row_quantiser_on_transposed_blocks():
    """A group whose length is a multiple of 128 is quantised exactly like the
    1x128 activation quantiser applied to the group's transposed rows."""
    rng = np.random.default_rng(5)
    off = np.array([0, 256, 384])
    x = rng.standard_normal((384, 200)) * np.exp2(rng.integers(-5, 5, (1, 200)))
    xq, xd, pad = backward.quant_tokens(x, off)
    for g in range(2):
        r0, r1 = off[g], off[g + 1]
        q, d = quant.quant_1x128(x[r0:r1].T)
        np.testing.assert_array_equal(xq[:, r0:r1], q)
        np.testing.assert_array_equal(xd[:, r0 // 128:r1 // 128], d)


def test_quant_tokens_ragged_tile_by_loop():
    rng = np.random.default_rng(6)
    off = np.array([0, 70, 70, 333])
    x = rng.standard_normal((333, 8)) * 3.0
    xq, xd, pad = backward.quant_tokens(x, off)
    for g in range(3):
        r0, r1 = off[g], off[g + 1]
        for t0 in range(r0, r1, 128):
            t1 = min(t0 + 128, r1)
            col = pad[g] + (t0 - r0)
            for c in range(8):
                amax = max(abs(v) for v in x[t0:t1, c])
                m = np.float32(448.0 / amax)
                assert xd[c, col // 128] == np.float32(amax / 448.0)
                for i, t in enumerate(range(t0, t1)):
                    want = e4m3.encode(np.array([float(np.float32(x[t, c] * np.float64(m)))]))[0]
                    assert xq[c, col + i] == want
                assert np.all(xq[c, col + (t1 - t0):col + 128] == 0)


def test_wgrad_exact_on_e4m3_operands_and_loop():
    """Operands that every token tile reproduces exactly: dW_g equals the
    exact float64 dY_g^T X_g; one element also by an explicit loop."""
    rng = np.random.default_rng(7)
    off = np.array([0, 128, 128, 384])
    N, K = 128, 256
    dy = np.zeros((384, N))
    x = np.zeros((384, K))
    for g in range(3):
        r0, r1 = off[g], off[g + 1]
        for t0 in range(r0, r1, 128):
            dy[t0:t0 + 128] = _exact_values(rng, N, 128, rng.integers(-10, -4, (N, 1)), 1, 128).T
            x[t0:t0 + 128] = _exact_values(rng, K, 128, rng.integers(-8, -2, (K, 1)), 1, 128).T
    dw, _, _, pad = backward.wgrad(dy, x, off)
    for g in range(3):
        r0, r1 = off[g], off[g + 1]
        exact = dy[r0:r1].T @ x[r0:r1]
        scale = np.abs(dy[r0:r1]).T @ np.abs(x[r0:r1]) + 1e-300
        assert np.max(np.abs(dw[g] - exact) / scale) < 1e-13
    assert np.all(dw[1] == 0.0)                       # an empty expert
    acc = sum(dy[t, 5] * x[t, 9] for t in range(128, 384))
    assert abs(dw[2, 5, 9] - acc) <= 1e-12 * abs(acc)


def test_wgrad_within_the_e4m3_error_bound():
    rng = np.random.default_rng(8)
    off = np.array([0, 100, 357, 357, 500])
    N, K = 128, 128
    dy = rng.standard_normal((500, N)) * np.exp2(rng.integers(-4, 4, (1, N)))
    x = rng.standard_normal((500, K)) * np.exp2(rng.integers(-4, 4, (1, K)))
    x[17] *= 50.0                                           # an outlier token
    dw, _, _, pad = backward.wgrad(dy, x, off)
    for g in range(4):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            assert np.all(dw[g] == 0.0)
            continue
        a, b = dy[r0:r1], x[r0:r1]
        # per token tile and channel: the tile amax gives the scale
        ea, eb = np.zeros_like(a), np.zeros_like(b)
        for t0 in range(0, r1 - r0, 128):
            sl = slice(t0, min(t0 + 128, r1 - r0))
            ea[sl] = np.abs(a[sl]) * (2.0 ** -4 + 2.0 ** -20) + np.abs(a[sl]).max(0) / 448.0 * 2.0 ** -10 * (1 + 1e-6)
            eb[sl] = np.abs(b[sl]) * (2.0 ** -4 + 2.0 ** -20) + np.abs(b[sl]).max(0) / 448.0 * 2.0 ** -10 * (1 + 1e-6)
        bound = ea.T @ np.abs(b) + (np.abs(a) + ea).T @ eb
        ratio = np.abs(dw[g] - a.T @ b) / bound
        assert np.max(ratio) <= 1.0 and np.max(ratio) > 1e-3
