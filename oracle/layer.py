"""The whole DeepSeekMoE forward layer chained from the oracle pieces -- test
infrastructure, see ``oracle/__init__``.

Order of the steps as the pages give them ([TP] section III flowchart, forward
pass then the per-step control loop; [TP] section V Figure 6 for each FP8
linear): affinity -> biased top-k -> unbiased gates -> per-expert token
groups -> FP8 expert FFNs (routed and shared) -> gate-weighted sum -> bias
update from this step's token counts.  Weights are quantised 128x128 from
their current values ("online" scaling, [TP] section V; done once per weight
update, here once per call).

Only for inputs the CPU finishes quickly (the tiny layer, or a sample of rows
of a large one through ``expert_rows``).
"""
import numpy as np

from . import route as _route
from . import permute as _permute
from . import quant as _quant
from . import ffn as _ffn
from . import bias as _bias


def quantise_weights(w1, w2):
    """w1 [G, 2I, H] (gate rows then up rows), w2 [G, H, I] ->
    dict(w1q, w1d, w2q, w2d) in the same (natural) row order."""
    w1q, w1d = _quant.quant_128x128(w1)
    w2q, w2d = _quant.quant_128x128(w2)
    return dict(w1q=w1q, w1d=w1d, w2q=w2q, w2d=w2d)


def expert_rows(xq, xd, tokens, wq, g, precision="D"):
    """FFN of expert g (N = shared) for the given tokens' rows."""
    return _ffn.expert_ffn(xq[tokens], xd[tokens], wq["w1q"][g], wq["w1d"][g],
                           wq["w2q"][g], wq["w2d"][g], precision)


def moe_layer(x, w_r, bias, w1, w2, k, gamma, precision="D", idx=None, wq=None, n_groups=1,
              topk_groups=1, router_fp8=False):
    """x [T, H], w_r [N, H], bias [N] float32, w1 [N+1, 2I, H],
    w2 [N+1, H, I] (expert N is the shared one).  ``idx`` overrides the
    oracle's own routing (to line it up with a routing decided elsewhere);
    ``wq`` supplies already-quantised weights; n_groups > 1 selects with the
    group-limited rule (``route.select_topk_grouped``); router_fp8 scores
    with the opt-in FP8 router (``route.route_fp8``).  Returns a dict of
    every intermediate."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    N = w_r.shape[0]
    if router_fp8:
        s64, s32, idx_o, gate_o, _ = _route.route_fp8(x, w_r, bias, k)
    else:
        s64, s32, idx_o, gate_o = _route.route(x, w_r, bias, k)
    if n_groups > 1:
        idx_o = _route.select_topk_grouped(s32, bias, k, n_groups, topk_groups)
        gate_o = _route.gates(s32, idx_o)
    if idx is None:
        idx = idx_o
        gate = gate_o
    else:
        idx = np.asarray(idx, np.int32)
        gate = _route.gates(s32, idx)
    counts, offsets, row_of, token_of = _permute.permute(idx, N, True)
    xq, xd = _quant.quant_1x128(x)
    if wq is None:
        wq = quantise_weights(w1, w2)
    R = T * k + T
    out = np.zeros((R, H), dtype=np.float64)
    hq = np.zeros((R, wq["w2q"].shape[-1]), dtype=np.uint8)
    hd = np.zeros((R, wq["w2q"].shape[-1] // _quant.TILE), dtype=np.float32)
    for g in range(N + 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 == r0:
            continue
        res = expert_rows(xq, xd, token_of[r0:r1], wq, g, precision)
        out[r0:r1] = res["out"]
        hq[r0:r1] = res["hq"]
        hd[r0:r1] = res["hd"]
    y = _ffn.combine(out, gate, row_of, T * k, precision)
    new_bias = _bias.bias_update(bias, counts, T, k, gamma)
    return dict(s64=s64, s32=s32, idx=idx, gate=gate, counts=counts,
                offsets=offsets, row_of=row_of, token_of=token_of, xq=xq,
                xd=xd, hq=hq, hd=hd, out=out, y=y, bias=new_bias, **wq)
