"""Fine-grained FP8 quantisers -- test infrastructure, see ``oracle/__init__``.

What is computed ([VE] recipe step 7; [TP] section V, FP8 detail 1 and the
"online" scaling of Figure 6; [DF] part 1 "Per-tile FP8 scaling"):

  * one scale per 1x128 tile of an activation matrix (one row, 128 consecutive
    columns of the contraction dimension), and one per 128x128 block of a
    weight matrix;
  * the scale is recomputed from the tile itself: scale = 448 / amax, the
    stored code is E4M3(x * scale), and the dequantised value is
    code_value / scale.

Readings where the pages leave a step open:
  * the multiplier m = fl32(448 / amax) and x * m are each one correctly
    rounded float32 operation (the kernel's precision), and the code is taken
    from that float32 product;
  * the stored factor is the dequantisation factor d = fl32(amax / 448), so
    dequantisation is a multiply;
  * a tile whose amax is 0, or so small that fl32(448 / amax) overflows, is
    stored as all-zero codes (0x00) with d = 1.0.

All float32 roundings below are done by computing in float64 and rounding
once; for one +, -, *, / of float32 operands that equals the correctly rounded
float32 result, because float64 carries more than 2 * 24 + 2 bits.
"""
import numpy as np

from . import e4m3

TILE = 128
FP8_MAX = 448.0


def _fl32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def _quant_groups(xg):
    """xg: float64 [..., n] with each trailing group sharing one scale.
    Returns (codes uint8 same shape, d float32 [...])."""
    amax = np.max(np.abs(xg), axis=-1)                         # exact
    with np.errstate(divide="ignore", over="ignore"):
        m = _fl32(FP8_MAX / amax)                              # fl32(448/amax)
    zero = (amax == 0.0) | ~np.isfinite(m)
    m64 = np.where(zero, 0.0, m.astype(np.float64))
    d = np.where(zero, np.float32(1.0), _fl32(amax / FP8_MAX))
    scaled = _fl32(xg * m64[..., None])                        # fl32(x * m)
    codes = e4m3.encode(scaled.astype(np.float64))
    codes = np.where(zero[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, d.astype(np.float32)


def quant_1x128(x):
    """Activation quantiser.  x: [rows, cols] values (float32-representable),
    cols % 128 == 0.  Returns (codes uint8 [rows, cols],
    d float32 [rows, cols / 128])."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = x.shape
    assert cols % TILE == 0
    codes, d = _quant_groups(x.reshape(rows, cols // TILE, TILE))
    return codes.reshape(rows, cols), d


def quant_128x128(w):
    """Weight quantiser.  w: [..., rows, cols], both multiples of 128.
    Returns (codes uint8 like w, d float32 [..., rows / 128, cols / 128])."""
    w = np.asarray(w, dtype=np.float64)
    *lead, rows, cols = w.shape
    assert rows % TILE == 0 and cols % TILE == 0
    rb, cb = rows // TILE, cols // TILE
    blocks = w.reshape(*lead, rb, TILE, cb, TILE)
    blocks = np.moveaxis(blocks, -3, -2).reshape(*lead, rb, cb, TILE * TILE)
    codes, d = _quant_groups(blocks)
    codes = codes.reshape(*lead, rb, cb, TILE, TILE)
    codes = np.moveaxis(codes, -2, -3).reshape(*lead, rows, cols)
    return codes, d


def dequant_1x128(codes, d):
    """x_hat[r, c] = value(code[r, c]) * d[r, c // 128], float64."""
    v = e4m3.decode(codes)
    return v * np.repeat(np.asarray(d, np.float64), TILE, axis=-1)


def dequant_128x128(codes, d):
    """w_hat[.., r, c] = value(code) * d[.., r // 128, c // 128], float64."""
    v = e4m3.decode(codes)
    dd = np.repeat(np.repeat(np.asarray(d, np.float64), TILE, axis=-2), TILE, axis=-1)
    return v * dd
