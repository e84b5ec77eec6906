"""Block-scaled FP8 GEMM, SwiGLU expert and gate-weighted combine -- test
infrastructure, see ``oracle/__init__``.

What is computed:
  * An FP8 linear layer takes E4M3 operands with one scale per 1x128 tile of
    the activation and per 128x128 block of the weight, accumulates in high
    precision and emits BF16 ([TP] section V, Figure 6 and FP8 details 1-2;
    [VE] recipe step 7).  Because the scales change every 128 elements of the
    contraction, the product is a sum over 128-deep blocks kb of the block's
    exact code-value dot product times d_A[r, kb] * d_B[c // 128, kb]:

        C[r, c] = sum_kb ( sum_{h in kb} v(A[r, h]) v(B[c, h]) ) d_A[r, kb] d_B[c//128, kb]

    Each inner block sum is exact in float64: an E4M3 x E4M3 product is a
    multiple of 2^-18 below 2^18, and 128 of them need fewer than 53 bits, so
    the library matmul used for it cannot round, whatever its order.
  * Each expert, routed or shared, is an FFN of intermediate size I ([VE]
    recipe step 3; [TP] section II).  Its form is SwiGLU (the plainest reading;
    the pages name no activation):  out = W2 (SiLU(W_gate u) * (W_up u)),
    SiLU(v) = v * sigmoid(v), no biases.  W1 = [W_gate; W_up] is [2I, H]
    (gate rows first), W2 is [H, I].  Both GEMMs are FP8; the intermediate h
    is itself an FP8 operand, quantised 1x128 from fl32(h).
  * The layer output of token t is the shared expert's output at full weight
    plus the gate-weighted routed outputs ([VE] glossary: "the shared expert
    ... is always added at full weight"; [TP] Figure 2, "summed into the
    block output").  The residual is not part of it.

Two precisions:
  * "D" (dequantised reference): everything after the codes in float64, no
    bf16 rounding anywhere.
  * "Q" (rounding-faithful): the GEMM1 output rounded to float32, SiLU and the
    product in float32 (each op rounded, exp taken in float64 and rounded),
    each expert output rounded to bf16, the combine as float32 fused
    multiply-adds in slot order starting from the shared row, then bf16.
"""
import numpy as np

from . import e4m3
from .quant import quant_1x128, TILE


def fl32(v):
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def bf16_round(v):
    """float32 -> bfloat16 (round to nearest even), returned as float64."""
    f = np.ascontiguousarray(np.asarray(v, np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def block_scaled_gemm(aq, ad, bq, bd):
    """aq uint8 [R, K], ad float32 [R, K/128]; bq uint8 [N, K],
    bd float32 [N/128, K/128].  Returns C float64 [R, N] per the formula in
    the module docstring."""
    a = e4m3.decode(aq)
    b = e4m3.decode(bq)
    ad = np.asarray(ad, np.float64)
    bd = np.asarray(bd, np.float64)
    R, K = a.shape
    N = b.shape[0]
    out = np.zeros((R, N), dtype=np.float64)
    for kb in range(K // TILE):
        sl = slice(kb * TILE, (kb + 1) * TILE)
        part = a[:, sl] @ b[:, sl].T                      # exact block sum
        col_scale = np.repeat(bd[:, kb], TILE)            # d_B[c // 128, kb]
        out += part * (ad[:, kb][:, None] * col_scale[None, :])
    return out


def silu64(v):
    v = np.asarray(v, np.float64)
    return v / (1.0 + np.exp(-v))


def silu32(v32):
    """SiLU with each float32 operation rounded: e = fl32(exp(-v)),
    den = fl32(1 + e), sg = fl32(1 / den), out = fl32(v * sg)."""
    e = fl32(np.exp(-v32))
    den = fl32(1.0 + e)
    sg = fl32(1.0 / den)
    return fl32(v32 * sg)


def expert_ffn(xq, xd, w1q, w1d, w2q, w2d, precision="D"):
    """One expert over a set of rows.

    xq/xd: [R, H] codes and [R, H/128] scales of the rows (already gathered);
    w1q/w1d: [2I, H] codes (gate rows then up rows) and [2I/128, H/128];
    w2q/w2d: [H, I] and [H/128, I/128].
    Returns dict(a=[R, 2I] float64, h=[R, I] float64 (what is quantised),
    hq, hd, out=[R, H] float64 (bf16 values in precision "Q"))."""
    a = block_scaled_gemm(xq, xd, w1q, w1d)
    I = a.shape[1] // 2
    if precision == "D":
        h = fl32(silu64(a[:, :I]) * a[:, I:])
    elif precision == "Q":
        a32 = fl32(a)
        h = fl32(silu32(a32[:, :I]) * a32[:, I:])
    else:
        raise ValueError(precision)
    hq, hd = quant_1x128(h)
    out = block_scaled_gemm(hq, hd, w2q, w2d)
    if precision == "Q":
        out = bf16_round(out)
    return dict(a=a, h=h, hq=hq, hd=hd, out=out)


def combine(out_rows, gate, row_of, shared_row0, precision="D"):
    """y[t] = out[shared_row0 + t] + sum_j gate[t, j] * out[row_of[t, j]].
    shared_row0 < 0 means there is no shared expert."""
    out_rows = np.asarray(out_rows, np.float64)
    gate = np.asarray(gate, np.float64)
    row_of = np.asarray(row_of, np.int64)
    T, k = row_of.shape
    H = out_rows.shape[1]
    if precision == "D":
        y = out_rows[shared_row0 + np.arange(T)].copy() if shared_row0 >= 0 \
            else np.zeros((T, H))
        for j in range(k):
            y += gate[:, j][:, None] * out_rows[row_of[:, j]]
        return y
    if precision == "Q":
        g32 = fl32(gate)
        acc = fl32(out_rows[shared_row0 + np.arange(T)]) if shared_row0 >= 0 \
            else np.zeros((T, H))
        for j in range(k):
            acc = fl32(acc + g32[:, j][:, None] * out_rows[row_of[:, j]])
        return bf16_round(acc)
    raise ValueError(precision)
