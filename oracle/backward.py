"""FP8 backward GEMMs of a block-scaled linear layer (Dgrad, Wgrad) -- test
infrastructure, see ``oracle/__init__``.

What is computed ([TP] section V, Figure 6: the three GEMMs of a linear layer,
forward, input gradient and weight gradient, all take FP8 inputs cast right
before the GEMM and accumulate in FP32; detail 3: E4M3 on every tensor with
fine-grained scales; detail 4 and [DF] part 1 "FP8 training, from first
principles": gradients are kept in higher precision).  For a linear layer Y = X W^T with X [R, K] (tokens x
input channels) and W [N, K]:

  Dgrad  dX = dY W      [R, K], contraction over the N output channels
  Wgrad  dW = dY^T X    [N, K], contraction over the R tokens

Readings where the pages leave a step open:
  * Dgrad: dY is an activation-like tensor with tokens as rows, so it takes the
    activation rule, one scale per 1x128 tile (one token, 128 consecutive
    channels of the contraction); W keeps its 128x128 blocks, used transposed
    (a 128x128 block transposes into a 128x128 block with the same scale, so
    the transposed codes and scales are exact).
  * Wgrad: both operands are activation-like, and the contraction now runs
    over tokens, so each is quantised with one scale per tile of 128
    consecutive tokens of one channel (1x128 along the contraction, as in
    every other FP8 product here).  Tokens are the rows of the expert-grouped
    layout; a tile never spans two experts, and a group's last tile holds the
    remaining tokens only (its amax is over those; the missing positions are
    zero codes).  Group g's tiles start at padded offset P_g = sum over
    earlier groups of 128 * ceil(R_g' / 128).
  * Wgrad is emitted in float32 (gradients in higher precision); Dgrad in
    bf16 or float32 as the forward GEMM's epilogues.
  * Each product is, as in the forward GEMM, the float64 dot product of the
    dequantised operands (the block sums are exact in float64, see ``ffn``).
"""
import numpy as np

from . import quant as _quant

TILE = _quant.TILE


def transpose_blocks(wq, wd):
    """Codes [..., R, C] and 128x128 scales [..., R/128, C/128] of W ->
    the same of W^T: codes [..., C, R], scales [..., C/128, R/128]."""
    return (np.ascontiguousarray(np.swapaxes(np.asarray(wq), -1, -2)),
            np.ascontiguousarray(np.swapaxes(np.asarray(wd), -1, -2)))


def dgrad(dy, wq, wd):
    """dX = dY W for one expert.  dy [R, N] values, wq/wd the 128x128
    quantised W [N, K].  Returns (dX float64 [R, K], dy codes, dy scales)."""
    dyq, dyd = _quant.quant_1x128(dy)
    dx = _quant.dequant_1x128(dyq, dyd) @ _quant.dequant_128x128(wq, wd)
    return dx, dyq, dyd


def padded_offsets(offsets):
    """Group row offsets [G+1] -> padded token offsets [G+1] (multiples of 128)."""
    off = np.asarray(offsets, np.int64)
    lens = np.diff(off)
    return np.concatenate([[0], np.cumsum((lens + TILE - 1) // TILE * TILE)]).astype(np.int64)


def quant_tokens(x, offsets):
    """Token-tile quantiser.  x [R, C] values in expert-grouped row order,
    offsets [G+1] the groups' first rows.  Returns (codes uint8 [C, Rpad]:
    column P_g + j of channel c is token offsets[g] + j of group g, zero past
    the group's end; scales float32 [C, Rpad / 128]; padded offsets [G+1])."""
    x = np.asarray(x, np.float64)
    R, C = x.shape
    off = np.asarray(offsets, np.int64)
    pad = padded_offsets(off)
    xt = np.zeros((C, int(pad[-1])), np.float64)
    for g in range(off.size - 1):
        r0, r1 = int(off[g]), int(off[g + 1])
        xt[:, pad[g]:pad[g] + (r1 - r0)] = x[r0:r1].T
    codes, d = _quant._quant_groups(xt.reshape(C, -1, TILE))
    return codes.reshape(C, -1), d, pad


def dequant_tokens(codes, d):
    return _quant.dequant_1x128(codes, d)


def wgrad(dy, x, offsets):
    """dW_g = dY_g^T X_g for every group g.  dy [R, N], x [R, K] values in
    expert-grouped row order.  Returns (dW float64 [G, N, K], the token-tile
    codes and scales of dY^T and X^T, padded offsets)."""
    aq, ad, pad = quant_tokens(dy, offsets)
    bq, bd, _ = quant_tokens(x, offsets)
    a = dequant_tokens(aq, ad)
    b = dequant_tokens(bq, bd)
    G = pad.size - 1
    out = np.zeros((G, a.shape[0], b.shape[0]), np.float64)
    for g in range(G):
        sl = slice(int(pad[g]), int(pad[g + 1]))
        out[g] = a[:, sl] @ b[:, sl].T
    return out, (aq, ad), (bq, bd), pad
