"""Sigmoid router, biased top-k and unbiased gates -- test infrastructure.

What is computed ([TP] section III: the affinity equation, the selection
equation for g' and the normalisation equation for g; [VE] recipe step 4 and
the glossary for u_t, e_i, b_i, K_r; [DF] "Balancing without a balance loss"):

  s[t, i]  = sigmoid(u_t . e_i)                 each expert scored on its own
  chosen   = the K_r experts with the largest s[t, i] + b[i]
  g'[t, i] = s[t, i] if i is chosen else 0      (the bias never enters g')
  g[t, i]  = g'[t, i] / sum_j g'[t, j]          (so the chosen gates sum to 1)

Readings where the pages leave a step open:
  * the router is x @ W_r^T with no router bias, temperature or extra scale;
    here in float64 (bf16 x bf16 products are exact), sigmoid in float64;
  * the scores that take part in selection and gating are float32, s32 =
    fl32(s); the biased key is one float32 add, key = fl32(s32 + b);
  * ties are broken by the lower expert index, and the k chosen experts are
    listed in (key descending, index ascending) order;
  * gates are computed in float64 from the float32 scores.

Group-limited selection ([VE] recipe step 5; [DF] "Balancing without a balance
loss", last sentences; [TP] section V, "Custom all-to-all kernels"): the N
experts are split into G equal groups of consecutive indices (one group per
node); a group's score is the sum of its K_r / M highest keys; only the M best
groups are eligible, and the K_r experts are the best keys among them.
Opt-in FP8 router.  The pages keep the gating network in BF16/FP32 ([TP]
section V, FP8 detail 4; [VE] recipe step 7); the FP8 option applies the
block-scaled product of [TP] section V (details 1-2, Figure 6) to the router:
x quantised 1x128, W_r quantised 128x128 (its rows are the experts), and
  z[t, i] = sum_c d_x[t, c] d_W[i / 128, c] sum_{h in block c} q_x[t, h] q_W[i, h]
in float64; scores, selection and gates then follow as above.

Readings where the pages leave a step open:
  * the keys are the biased keys (selection, including the group ranking, is
    where the bias acts; the gates stay unbiased);
  * the group score is a float32 sum of the group's K_r / M highest keys taken
    in descending order, and K_r must be a multiple of M;
  * groups are ranked by (score descending, group index ascending).
"""
import numpy as np

from . import ffn as _ffn
from . import quant as _quant


def router_logits(x, w_r):
    """z[t, i] = sum_h x[t, h] * W_r[i, h] in float64.  W_r row i is e_i."""
    return np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T


def sigmoid(z):
    """1 / (1 + exp(-z)) in float64, evaluated without overflow."""
    z = np.asarray(z, np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def router_logits_fp8(xq, xd, wq, wd):
    """z [T, N] float64 from quantised operands: x codes [T, H] with 1x128
    scales [T, H/128], W_r codes [N, H] with 128x128 scales [N/128, H/128]."""
    return _ffn.block_scaled_gemm(xq, xd, wq, wd)


def route_fp8(x, w_r, bias, k, n_groups=1, topk_groups=1):
    """Routing through the opt-in FP8 router: x and W_r quantised by the
    oracle's own quantisers, logits from the block-scaled product, then the
    same sigmoid, selection and gates as ``route``.  Returns
    (s64, s32, idx, gate, (xq, xd, wq, wd))."""
    xq, xd = _quant.quant_1x128(x)
    wq, wd = _quant.quant_128x128(w_r)
    s64 = sigmoid(router_logits_fp8(xq, xd, wq, wd))
    s32 = s64.astype(np.float32)
    idx = select_topk_grouped(s32, bias, k, n_groups, topk_groups)
    return s64, s32, idx, gates(s32, idx), (xq, xd, wq, wd)


def router_scores(x, w_r):
    """Float64 affinities s = sigmoid(x @ W_r^T)."""
    return sigmoid(router_logits(x, w_r))


def biased_keys(s32, bias):
    """key = fl32(s32 + b), one float32 add per (token, expert)."""
    s = np.asarray(s32, np.float32).astype(np.float64)
    b = np.asarray(bias, np.float32).astype(np.float64)
    return (s + b[None, :]).astype(np.float32)


def select_topk(s32, bias, k):
    """Indices [T, k] int32 of the k largest biased keys per token, ordered by
    (key descending, index ascending)."""
    key = biased_keys(s32, bias)
    order = np.argsort(-key, axis=1, kind="stable")   # stable: index asc on ties
    return order[:, :k].astype(np.int32)


def group_scores(key, n_groups, per_group):
    """Float32 score of every group: the sum of its `per_group` largest keys,
    added in descending order.  key [T, N] float32 -> [T, G] float32."""
    key = np.asarray(key, np.float32)
    T, N = key.shape
    gs = N // n_groups
    top = -np.sort(-key.reshape(T, n_groups, gs), axis=2)[:, :, :per_group]
    acc = top[:, :, 0].astype(np.float32)
    for j in range(1, per_group):
        acc = (acc.astype(np.float64) + top[:, :, j].astype(np.float64)).astype(np.float32)
    return acc


def select_topk_grouped(s32, bias, k, n_groups, topk_groups):
    """Group-limited selection: indices [T, k] int32 of the k largest biased
    keys among the experts of the `topk_groups` best groups (groups ranked by
    the float32 sum of their k / topk_groups largest keys, ties to the lower
    group), ordered by (key descending, index ascending)."""
    key = biased_keys(s32, bias)
    T, N = key.shape
    if n_groups <= 1 or topk_groups >= n_groups:
        return select_topk(s32, bias, k)
    assert N % n_groups == 0 and k % topk_groups == 0
    gs = N // n_groups
    gsc = group_scores(key, n_groups, k // topk_groups)
    gorder = np.argsort(-gsc, axis=1, kind="stable")[:, :topk_groups]
    allowed = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(allowed, gorder, True, axis=1)
    allowed = np.repeat(allowed, gs, axis=1)
    order = np.lexsort((np.broadcast_to(np.arange(N), key.shape), -key.astype(np.float64),
                        ~allowed), axis=1)
    return order[:, :k].astype(np.int32)


def gates(s32, idx):
    """g[t, j] = s32[t, idx[t, j]] / sum_j' s32[t, idx[t, j']], float64.
    The bias is not an argument: it cannot reach the gate."""
    s = np.asarray(s32, np.float32).astype(np.float64)
    sel = np.take_along_axis(s, np.asarray(idx, np.int64), axis=1)
    tot = sel.sum(axis=1, keepdims=True)
    k = sel.shape[1]
    return np.where(tot > 0, sel / np.where(tot > 0, tot, 1.0), 1.0 / k)


def route(x, w_r, bias, k):
    """Full routing in the oracle's own precision.  Returns
    (s64 [T,N] float64, s32 [T,N] float32, idx [T,k] int32, gate [T,k] float64)."""
    s64 = router_scores(x, w_r)
    s32 = s64.astype(np.float32)
    idx = select_topk(s32, bias, k)
    return s64, s32, idx, gates(s32, idx)


def topk_margin(s64, bias, k):
    """Float64 gap between the k-th and (k+1)-th largest s + b per token
    (inf when k equals the number of experts).  A token with a tiny gap can be
    routed either way by any finite-precision evaluation of the router."""
    key = np.asarray(s64, np.float64) + np.asarray(bias, np.float64)[None, :]
    n = key.shape[1]
    if k >= n:
        return np.full(key.shape[0], np.inf)
    part = -np.sort(-key, axis=1)
    return part[:, k - 1] - part[:, k]
