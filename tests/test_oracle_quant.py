"""Pins of the oracle's 1x128 / 128x128 quantisers.

Sources: "DeepSeek-V3 Technical Report" (deepforge.srivtx.xyz), part 1
"Per-tile FP8 scaling" (scale = 448 / amax, worked tile) and part 4 "Build it
yourself" (per-tensor vs per-128-tile success criteria); "DeepSeek-V3:
Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction, and FP8
Training at 671B Scale", section V, FP8 detail 1 (1x128 activation tiles,
128x128 weight blocks, a local outlier rescales only its own group).
"""
import json
import os

import numpy as np

from oracle import e4m3, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def test_worked_example_from_the_page():
    g = json.load(open(os.path.join(GOLDEN, "quantize_tile_worked_example.json")))
    tile = np.zeros((1, 128))
    tile[0, :4] = _f32(g["input"])
    codes, d = quant.quant_1x128(tile)
    assert list(codes[0, :4]) == g["e4m3_codes"]
    assert np.array_equal(e4m3.decode(codes[0, :4]), g["e4m3_values"])
    assert np.all(codes[0, 4:] == 0)
    deq = quant.dequant_1x128(codes, d)[0, :4]
    # the page divides by a float64 scale; the oracle multiplies by the float32
    # factor d = fl32(amax / 448) and starts from float32 inputs
    np.testing.assert_allclose(deq, g["dequantised"], rtol=2e-7, atol=0)


def test_every_nonzero_tile_reaches_448_and_error_bounds():
    rng = np.random.default_rng(2)
    x = _f32(rng.standard_normal((37, 512)) * np.exp(rng.uniform(-8, 8, (37, 1))))
    codes, d = quant.quant_1x128(x)
    tiles = codes.reshape(37, 4, 128)
    assert np.all(np.any((tiles & 0x7F) == 0x7E, axis=-1))
    xh = quant.dequant_1x128(codes, d)
    m = _f32(448.0 / np.abs(x.reshape(37, 4, 128)).max(-1))
    scaled = np.abs(x) * np.repeat(m, 128, axis=-1)
    err = np.abs(xh - x)
    normal = scaled >= 2.0 ** -6
    # half an E4M3 step relative (2^-4) plus float32 slack from fl32(x*m), d != 1/m
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -21) * np.abs(x[normal]))
    dd = np.repeat(d.astype(np.float64), 128, axis=-1)
    assert np.all(err[~normal] <= 2.0 ** -10 * dd[~normal] * (1 + 2.0 ** -21) + 1e-300)


def test_on_grid_tile_round_trips_exactly():
    vals = e4m3.POS_VALUES[1:]
    rng = np.random.default_rng(3)
    x = rng.choice(vals, (4, 128)) * rng.choice([-1.0, 1.0], (4, 128))
    x[:, 5] = 448.0                                          # amax = 448 -> m = d = 1
    codes, d = quant.quant_1x128(x)
    assert np.all(d == 1.0)
    assert np.array_equal(quant.dequant_1x128(codes, d), x)


def test_scale_is_per_tile_and_online():
    rng = np.random.default_rng(4)
    x = _f32(rng.standard_normal((2, 256)))
    c0, d0 = quant.quant_1x128(x)
    x2 = x.copy()
    x2[0, 3] = 1000.0                      # outlier in tile (0, 0) only
    c1, d1 = quant.quant_1x128(x2)
    assert d1[0, 0] == np.float32(1000.0 / 448.0)
    assert d1[0, 1] == d0[0, 1] and d1[1, 0] == d0[1, 0] and d1[1, 1] == d0[1, 1]
    assert np.array_equal(c1[:, 128:], c0[:, 128:]) and np.array_equal(c1[1], c0[1])


def test_zero_and_tiny_tiles():
    x = np.zeros((1, 256))
    x[0, 130] = 1e-39                      # fl32(448 / 1e-39) overflows
    codes, d = quant.quant_1x128(_f32(x))
    assert np.all(codes == 0) and np.all(d == 1.0)


def _rel_l2(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_build_it_yourself_criteria_per_tensor_vs_per_tile():
    """One large outlier and values near 1e-5: one scale for the whole vector
    leaves the non-outlier tile with relative error above 0.5; one scale per
    128 brings it below 0.05 (read normwise, over that tile)."""
    rng = np.random.default_rng(5)
    v = _f32(rng.standard_normal(256) * 1e-5)
    v[7] = 100.0                                            # outlier in tile 0
    # per tensor: the same rule with a single 256-wide group
    codes_t, d_t = quant._quant_groups(v.reshape(1, 256))
    vt = e4m3.decode(codes_t[0]) * float(d_t[0])
    codes_b, d_b = quant.quant_1x128(v.reshape(1, 256))
    vb = quant.dequant_1x128(codes_b, d_b)[0]
    quiet = slice(128, 256)
    assert _rel_l2(vt[quiet], v[quiet]) > 0.5
    assert _rel_l2(vb[quiet], v[quiet]) < 0.05


def test_weight_blocks_are_128x128():
    rng = np.random.default_rng(6)
    w = _f32(rng.standard_normal((2, 256, 384)) * 0.006)
    w[1, 130, 260] = 5.0                    # block (1, 1, 2)
    codes, d = quant.quant_128x128(w)
    assert d.shape == (2, 2, 3)
    blocks = np.abs(w).reshape(2, 2, 128, 3, 128).max(axis=(2, 4))
    np.testing.assert_array_equal(d, _f32(blocks / 448.0).astype(np.float32))
    # each block is the 1x128 rule applied to the block's 16384 values
    blk = w[1, 128:256, 256:384]
    cb, db = quant._quant_groups(blk.reshape(1, -1))
    assert np.array_equal(codes[1, 128:256, 256:384].reshape(-1), cb[0])
    wh = quant.dequant_128x128(codes, d)
    assert np.max(np.abs(wh - w) / np.maximum(np.abs(w), 1e-30)
                  * (np.abs(w) >= 2.0 ** -6 * np.repeat(np.repeat(d, 128, 1), 128, 2))) <= 2.0 ** -4 + 2.0 ** -21
