"""End-to-end parity of the layer (MoELayer.forward, the path bench.py times)
against the CPU oracle.

Bars: routing indices, counts, permutation maps, FP8 activation codes and the
bias update bit-exact (routing on tokens whose top-k gap is clear of the
router's float32 error); the output within normwise max relative error 2e-2 of
the float64 oracle on the same dequantised FP8 operands ("D").

Against the rounding-faithful oracle ("Q": float32 GEMM results, float32
SwiGLU, bf16 expert outputs, float32 combine) the bar is 1e-3 relative L2:
  * on every token whose k + 1 expert rows carry exactly the oracle's h codes;
  * on every token against the same oracle fed the GPU's own h codes (GEMM2 and
    combine from those codes), which isolates the codes the MFMA moved;
  * a token with moved codes may differ from the oracle's own result by at
    most 1e-3 plus exactly what those moved codes change (the difference
    between the two oracle runs, per token).
The gfx950 FP8 MFMA sums each group of 8 products on a grid 2^-13 below the
group's largest (test_mfma_block_sum_precision_probe), so a few h values that
lie within that error of an E4M3 rounding midpoint land on the neighbouring
code; check_h bounds where that may happen (the MFMA band propagated through
SwiGLU) and how often (H_FLIP_MAX_FRAC).

At the DeepSeek-V3 shape (H 7168, 256 routed experts top-8 plus 1 shared,
I 2048) the oracle recomputes a sample the CPU can afford: all routing, the
expert FFN of the least and most loaded routed experts plus a slice of the
shared expert's rows, and the full output y of sampled tokens from their k + 1
experts regenerated on the host.
"""
import numpy as np
import pytest

import synth
from helpers import (bf16_from_dev, bf16_to_dev, bf16_values, check_h, flip_cap,
                     device_tensor, log, max_rel, rel_l2, swiglu_band, to_dev)
from oracle import ffn, layer as olayer, quant, route

pytestmark = pytest.mark.gpu

D_BAR = 2e-2        # normwise max relative error vs the float64 oracle
Q_BAR = 1e-3        # relative L2 vs the rounding-faithful oracle

torch = pytest.importorskip("torch")


def _moe():
    import fp8_block_scaled_sigmoid_amd as moe
    return moe


def _run_small(w, x_bits=None):
    moe = _moe()
    x_b = synth.generate(w.x_spec(), w.seed) if x_bits is None else x_bits
    wr_b = w.router_weight()
    w1_b = synth.generate(w.w1_spec(), w.seed)
    w2_b = synth.generate(w.w2_spec(), w.seed)
    b = w.bias()
    log(f"layer {w.name} T={w.T} H={w.H} N={w.N} k={w.k} I={w.I}")
    weights = moe.MoEWeights(bf16_to_dev(wr_b), to_dev(b.copy()), w1_bf16=bf16_to_dev(w1_b),
                             w2_bf16=bf16_to_dev(w2_b))
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma)
    y = bf16_values(lay.forward(bf16_to_dev(x_b)))
    torch.cuda.synchronize()
    args = (synth.as_f64(x_b), synth.as_f64(wr_b), b, synth.as_f64(w1_b), synth.as_f64(w2_b),
            w.k, w.gamma)
    return lay, weights, y, args


def _check_small(lay, weights, y, args, k):
    q = olayer.moe_layer(*args, precision="Q")
    s64 = q["s64"]
    margin = route.topk_margin(s64, args[2], k)
    assert np.all(margin > 3e-5), "inputs too close to a routing tie for an exact check"
    assert np.array_equal(lay.idx.cpu().numpy(), q["idx"])
    assert np.array_equal(lay.counts.cpu().numpy(), q["counts"])
    assert np.array_equal(lay.offsets.cpu().numpy(), q["offsets"])
    assert np.array_equal(lay.row_of.cpu().numpy(), q["row_of"])
    assert np.array_equal(lay.token_of.cpu().numpy(), q["token_of"])
    assert np.array_equal(lay.xq.cpu().numpy(), q["xq"])
    assert np.array_equal(lay.xd.cpu().numpy(), q["xd"])
    np.testing.assert_allclose(lay.gate.cpu().numpy(), q["gate"], rtol=1e-5, atol=1e-6)
    assert np.array_equal(weights.bias.cpu().numpy(), q["bias"])
    # h: the re-quantised intermediate, within the propagated MFMA band
    hq = lay.hq.cpu().numpy()
    hd = lay.hd.cpu().numpy()
    wq = {kk: q[kk] for kk in ("w1q", "w1d", "w2q", "w2d")}
    n_h = 0
    row_moved = np.zeros(hq.shape[0], bool)
    for g in range(q["offsets"].size - 1):
        r0, r1 = q["offsets"][g], q["offsets"][g + 1]
        if r1 == r0:
            continue
        toks = q["token_of"][r0:r1]
        res = olayer.expert_rows(q["xq"], q["xd"], toks, wq, g, "Q")
        band = swiglu_band(q["xq"][toks], q["xd"][toks], wq["w1q"][g], wq["w1d"][g], res["h"],
                           res["a"])
        n_h += check_h(hq[r0:r1], hd[r0:r1], res, band)
        row_moved[r0:r1] = np.any(hq[r0:r1] != res["hq"], axis=1)
    check_y_q(y, q, hq, hd, row_moved)
    d = olayer.moe_layer(*args, precision="D")
    err_d = max_rel(y, d["y"])
    print(f"normwise max rel vs D = {err_d:.3e}, h codes differing = {n_h} of {hq.size}")
    assert n_h <= flip_cap(hq.size)
    assert err_d <= D_BAR


def check_y_q(y, q, hq, hd, row_moved):
    """The three rounding-faithful bars on y (module docstring).  ``q`` is the
    oracle's "Q" layer, hq/hd the GPU's h codes and scales, row_moved marks
    the expert rows whose h codes differ from the oracle's."""
    from oracle import ffn as offn
    T, k = q["row_of"].shape
    R = q["offsets"][-1]
    out_fed = np.zeros_like(q["out"])
    for g in range(q["offsets"].size - 1):
        r0, r1 = q["offsets"][g], q["offsets"][g + 1]
        if r1 > r0:
            out_fed[r0:r1] = offn.bf16_round(offn.block_scaled_gemm(hq[r0:r1], hd[r0:r1],
                                                                    q["w2q"][g], q["w2d"][g]))
    y_fed = offn.combine(out_fed, q["gate"], q["row_of"], T * k, "Q")
    rows_t = np.concatenate([q["row_of"], T * k + np.arange(T)[:, None]], 1)
    moved = np.any(row_moved[rows_t], axis=1)
    clean = ~moved
    err_fed = rel_l2(y, y_fed)
    err_clean = rel_l2(y[clean], q["y"][clean]) if clean.any() else 0.0
    print(f"rel L2 vs Q: {err_clean:.3e} on {clean.sum()} tokens with the oracle's h codes; "
          f"{err_fed:.3e} on all {T} tokens vs Q fed the GPU's h codes; "
          f"{moved.sum()} tokens with moved codes")
    assert err_clean <= Q_BAR
    assert err_fed <= Q_BAR
    for t in np.nonzero(moved)[0]:
        shift = np.linalg.norm(y_fed[t] - q["y"][t])
        assert np.linalg.norm(y[t] - q["y"][t]) <= shift + Q_BAR * np.linalg.norm(q["y"][t]) + 1e-30
    return clean.sum(), moved.sum()


def test_layer_tiny():
    w = synth.WORKLOADS["tiny"]
    _check_small(*_run_small(w), w.k)


@pytest.mark.parametrize("T,H,N,k,I", [(300, 512, 32, 4, 256), (40, 256, 16, 1, 128),
                                       (17, 384, 16, 16, 128), (1, 256, 16, 2, 128)])
def test_layer_small_variants(T, H, N, k, I):
    """Small layers of other shapes.  The seed is redrawn (before any GPU
    work) until every token's top-k gap is clear of the router's float32
    error, so the exact routing check always runs."""
    for seed in range(T, T + 50):
        w = synth.Workload(f"v{T}", T=T, H=H, N=N, k=k, I=I, x_std=1.0, wr_dist=synth.NORMAL,
                           wr_param=0.05, bias_half=0.1, w_std=0.02, seed=seed)
        x_b = synth.generate(w.x_spec(), w.seed)
        s64 = route.router_scores(synth.as_f64(x_b), synth.as_f64(w.router_weight()))
        if np.all(route.topk_margin(s64, w.bias(), k) > 3e-5):
            break
    else:
        raise AssertionError("no seed with a clear top-k margin")
    lay, weights, y, args = _run_small(w, x_b)
    _check_small(lay, weights, y, args, k)


def test_layer_tiny_group_limited():
    """The tiny layer with group-limited routing: 16 experts in 4 groups of
    4, the best 2 groups eligible, top-2 -- through MoELayer, against the
    oracle layer with the same rule."""
    moe = _moe()
    w = synth.WORKLOADS["tiny"]
    x_b = synth.generate(w.x_spec(), w.seed)
    wr_b = w.router_weight()
    w1_b = synth.generate(w.w1_spec(), w.seed)
    w2_b = synth.generate(w.w2_spec(), w.seed)
    b = w.bias()
    log("layer tiny group-limited G=4 M=2")
    weights = moe.MoEWeights(bf16_to_dev(wr_b), to_dev(b.copy()), w1_bf16=bf16_to_dev(w1_b),
                             w2_bf16=bf16_to_dev(w2_b))
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma, n_groups=4, topk_groups=2)
    y = bf16_values(lay.forward(bf16_to_dev(x_b)))
    torch.cuda.synchronize()
    args = (synth.as_f64(x_b), synth.as_f64(wr_b), b, synth.as_f64(w1_b), synth.as_f64(w2_b),
            w.k, w.gamma)
    # selection on the GPU's own scores is the group-limited rule, bit-exact
    s_gpu = lay.scores.cpu().numpy()
    idx = lay.idx.cpu().numpy()
    assert np.array_equal(idx, route.select_topk_grouped(s_gpu, b, w.k, 4, 2))
    q = olayer.moe_layer(*args, precision="Q", idx=idx)
    assert np.array_equal(lay.counts.cpu().numpy(), q["counts"])
    assert np.array_equal(lay.row_of.cpu().numpy(), q["row_of"])
    assert np.array_equal(weights.bias.cpu().numpy(), q["bias"])
    hq_g, hd_g = lay.hq.cpu().numpy(), lay.hd.cpu().numpy()
    check_y_q(y, q, hq_g, hd_g, np.any(hq_g != q["hq"], axis=1))
    d = olayer.moe_layer(*args, precision="D", idx=idx)
    assert max_rel(y, d["y"]) <= D_BAR
    # and the oracle's own group-limited routing agrees wherever the float64
    # group and expert margins are clear of the router's float32 error
    mine = olayer.moe_layer(*args, precision="Q", n_groups=4, topk_groups=2)["idx"]
    agree = np.all(np.sort(mine, 1) == np.sort(idx, 1), axis=1)
    assert agree.mean() > 0.95


def test_layer_fp8_router():
    """A small layer with the opt-in FP8 router (128 experts top-4): routing on
    the GPU's own scores is the selection rule bit for bit, the scores sit in
    the FP8 router's band around the oracle's FP8 router, and the rest of the
    layer matches the oracle given that routing."""
    moe = _moe()
    w = synth.Workload("fp8r", T=300, H=512, N=128, k=4, I=256, x_std=1.0, wr_dist=synth.NORMAL,
                       wr_param=0.05, bias_half=0.1, w_std=0.02, seed=7)
    x_b = synth.generate(w.x_spec(), w.seed)
    wr_b = w.router_weight()
    w1_b = synth.generate(w.w1_spec(), w.seed)
    w2_b = synth.generate(w.w2_spec(), w.seed)
    b = w.bias()
    log("layer fp8 router T=300 H=512 N=128 k=4")
    weights = moe.MoEWeights(bf16_to_dev(wr_b), to_dev(b.copy()), w1_bf16=bf16_to_dev(w1_b),
                             w2_bf16=bf16_to_dev(w2_b), router_fp8=True)
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma, router_fp8=True)
    y = bf16_values(lay.forward(bf16_to_dev(x_b)))
    torch.cuda.synchronize()
    args = (synth.as_f64(x_b), synth.as_f64(wr_b), b, synth.as_f64(w1_b), synth.as_f64(w2_b),
            w.k, w.gamma)
    s_gpu = lay.scores.cpu().numpy()
    idx = lay.idx.cpu().numpy()
    assert np.array_equal(idx, route.select_topk(s_gpu, b, w.k))
    q = olayer.moe_layer(*args, precision="Q", idx=idx, router_fp8=True)
    xq, xd, wq, wd = route.route_fp8(args[0], args[1], b, w.k)[4]
    mag = route.router_logits_fp8(xq & 0x7F, xd, wq & 0x7F, wd)   # sum |d_x d_W q_x q_W|
    assert np.all(np.abs(s_gpu - q["s64"]) <= 0.25e-4 * mag + 2e-7)
    np.testing.assert_allclose(lay.gate.cpu().numpy(), q["gate"], rtol=1e-4, atol=1e-6)
    assert np.array_equal(lay.xq.cpu().numpy(), q["xq"])
    assert np.array_equal(lay.counts.cpu().numpy(), q["counts"])
    assert np.array_equal(lay.row_of.cpu().numpy(), q["row_of"])
    assert np.array_equal(weights.bias.cpu().numpy(), q["bias"])
    hq_g, hd_g = lay.hq.cpu().numpy(), lay.hd.cpu().numpy()
    check_y_q(y, q, hq_g, hd_g, np.any(hq_g != q["hq"], axis=1))
    d = olayer.moe_layer(*args, precision="D", idx=idx, router_fp8=True)
    err_d = max_rel(y, d["y"])
    print(f"normwise max rel vs D = {err_d:.3e}")
    assert err_d <= D_BAR


def test_layer_zero_input():
    w = synth.WORKLOADS["tiny"]
    zero = np.zeros((w.T, w.H), np.uint16)
    lay, weights, y, args = _run_small(w, zero)
    assert np.all(y == 0.0)
    assert np.all(lay.xq.cpu().numpy() == 0) and np.all(lay.xd.cpu().numpy() == 1.0)


# --------------------------------------------------------------------------- V3 shape


def _build_v3(w):
    """Weights generated and quantised on the device (22.6 GB of bf16 never
    reaches the host); the host regenerates the sampled experts only."""
    moe = _moe()
    log(f"v3 weights {w.name}")
    w1 = device_tensor(w.w1_spec(), w.seed)
    w1q, w1d = moe.fp8_quant_128x128(w1, interleave_gate_up=True)
    del w1
    w2 = device_tensor(w.w2_spec(), w.seed)
    w2q, w2d = moe.fp8_quant_128x128(w2)
    del w2
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    wr_b = w.router_weight()
    b = w.bias()
    weights = moe.MoEWeights(bf16_to_dev(wr_b), to_dev(b.copy()), w1q=w1q, w1d=w1d, w2q=w2q,
                             w2d=w2d)
    return weights, wr_b, b


def _expert_oracle(w, g):
    H, I = w.H, w.I
    w1 = synth.as_f64(synth.generate(w.w1_spec(), w.seed,
                                     rows=np.arange(g * 2 * I, (g + 1) * 2 * I)))
    w2 = synth.as_f64(synth.generate(w.w2_spec(), w.seed, rows=np.arange(g * H, (g + 1) * H)))
    w1q, w1d = quant.quant_128x128(w1)
    w2q, w2d = quant.quant_128x128(w2)
    return w1q, w1d, w2q, w2d


def _check_tokens_end_to_end(w, lay, y, wr_b, b0, n_tokens):
    """The full output row y[t] of a few tokens against the oracle, from
    scratch: the token's x row and its k + 1 experts (the k routed ones the
    oracle itself picks, and the shared one) regenerated on the host and
    quantised by the oracle, the expert FFNs and the combine run by the
    oracle in both precisions.  Tokens are the first ones whose top-k gap is
    clear of the router's float32 error.  Bars: normwise max relative error
    <= 2e-2 vs "D"; relative L2 <= 1e-3 vs "Q" when the GPU's h codes of the
    token's rows are the oracle's, otherwise within 1e-3 of "Q" fed the GPU's
    own h codes for those rows."""
    T, k, N = w.T, w.k, w.N
    xb = synth.generate(w.x_spec(), w.seed, rows=np.arange(min(T, 64)))
    s64 = route.router_scores(synth.as_f64(xb), synth.as_f64(wr_b))
    clear = np.nonzero(route.topk_margin(s64, b0, k) > 3e-5)[0][:n_tokens]
    assert clear.size == n_tokens
    idx_gpu = lay.idx.cpu().numpy()
    row_of = lay.row_of.cpu().numpy()
    hq_all = lay.hq.cpu().numpy()
    hd_all = lay.hd.cpu().numpy()
    y_gpu = bf16_values(y)
    cache = {}
    for t in clear:
        idx_o = route.select_topk(s64[t:t + 1].astype(np.float32), b0, k)[0]
        assert np.array_equal(idx_gpu[t], idx_o)
        gate_o = route.gates(s64[t:t + 1].astype(np.float32), idx_o[None])[0]
        xq, xd = quant.quant_1x128(synth.as_f64(xb[t:t + 1]))
        rows = [int(r) for r in row_of[t]] + [T * k + int(t)]
        experts = [int(e) for e in idx_o] + [N]
        outs_q, outs_d, outs_fed, moved = [], [], [], False
        for g, r in zip(experts, rows):
            if g not in cache:
                log(f"oracle expert {g} for token {t}")
                cache[g] = _expert_oracle(w, g)
            w1q, w1d, w2q, w2d = cache[g]
            rq = ffn.expert_ffn(xq, xd, w1q, w1d, w2q, w2d, "Q")
            rd = ffn.expert_ffn(xq, xd, w1q, w1d, w2q, w2d, "D")
            outs_q.append(rq["out"][0])
            outs_d.append(rd["out"][0])
            outs_fed.append(ffn.bf16_round(ffn.block_scaled_gemm(hq_all[r:r + 1], hd_all[r:r + 1],
                                                                 w2q, w2d))[0])
            moved |= bool(np.any(hq_all[r] != rq["hq"][0]))
        # combine in slot order from the shared row (one token, the oracle's gates)
        ones = np.arange(k)[None]
        yq = ffn.combine(np.array(outs_q), gate_o[None], ones, k, "Q")[0]
        yd = ffn.combine(np.array(outs_d), gate_o[None], ones, k, "D")[0]
        yf = ffn.combine(np.array(outs_fed), gate_o[None], ones, k, "Q")[0]
        e_d = max_rel(y_gpu[t], yd)
        e_fed = rel_l2(y_gpu[t], yf)
        e_q = rel_l2(y_gpu[t], yq)
        print(f"token {t}: experts {experts}; max rel vs D {e_d:.2e}; rel L2 vs Q {e_q:.2e}, vs Q fed "
              f"the GPU's h codes {e_fed:.2e}; h codes moved: {moved}")
        assert e_d <= D_BAR
        assert e_fed <= Q_BAR
        if moved:
            assert np.linalg.norm(y_gpu[t] - yq) <= np.linalg.norm(yf - yq) + Q_BAR * np.linalg.norm(yq)
        else:
            assert e_q <= Q_BAR


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_layer_v3_shape_sampled(name):
    moe = _moe()
    w = synth.WORKLOADS[name]
    weights, wr_b, b0 = _build_v3(w)
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma)
    x = device_tensor(w.x_spec(), w.seed)
    log(f"v3 forward {name}")
    y = lay.forward(x)
    torch.cuda.synchronize()
    idx = lay.idx.cpu().numpy()
    gate = lay.gate.cpu().numpy()
    counts = lay.counts.cpu().numpy()
    offsets = lay.offsets.cpu().numpy()
    row_of = lay.row_of.cpu().numpy()
    token_of = lay.token_of.cpu().numpy()
    T, k, N = w.T, w.k, w.N

    # routing on a token sample, in the oracle's own precision
    sample = np.arange(T) if T <= 2048 else np.sort(np.random.default_rng(0).choice(T, 2048, False))
    xb = synth.generate(w.x_spec(), w.seed, rows=sample)
    assert np.array_equal(bf16_from_dev(x[torch.from_numpy(sample).cuda()]), xb)
    s64 = route.router_scores(synth.as_f64(xb), synth.as_f64(wr_b))
    assert np.max(np.abs(lay.scores.cpu().numpy()[sample] - s64)) < 1e-5
    clear = route.topk_margin(s64, b0, k) > 3e-5
    assert clear.mean() > 0.97
    idx_o = route.select_topk(s64.astype(np.float32), b0, k)
    assert np.array_equal(idx[sample][clear], idx_o[clear])
    np.testing.assert_allclose(gate[sample], route.gates(s64.astype(np.float32), idx[sample]),
                               rtol=1e-5, atol=1e-6)
    # activation codes on the sample: bit-exact
    xq_o, xd_o = quant.quant_1x128(synth.as_f64(xb))
    assert np.array_equal(lay.xq.cpu().numpy()[sample], xq_o)
    assert np.array_equal(lay.xd.cpu().numpy()[sample], xd_o)

    # permutation: properties of the GPU's own routing (bit-exactness of the
    # permutation itself is covered at this size by test_permute_bit_exact)
    assert counts.sum() == T * k and np.array_equal(np.bincount(idx.ravel(), minlength=N), counts)
    assert np.array_equal(np.sort(row_of.ravel()), np.arange(T * k))
    assert np.array_equal(token_of[row_of], np.repeat(np.arange(T)[:, None], k, 1))
    for e in range(N):
        assert np.all(np.diff(token_of[offsets[e]:offsets[e + 1]]) > 0)

    # expert FFN on sampled experts, compared row by row
    xq_all = lay.xq.cpu().numpy()
    xd_all = lay.xd.cpu().numpy()
    hq = lay.hq.cpu().numpy()
    out_rows = lay.out_rows
    live = np.nonzero(counts)[0]
    experts = [int(live[np.argmin(counts[live])]), int(np.argmax(counts)), N]
    for g in experts:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        rows = np.arange(r0, r1) if g < N else np.concatenate([np.arange(r0, r0 + 32),
                                                               np.arange(r1 - 32, r1)])
        toks = token_of[rows]
        # the oracle quantises the rows it needs from the generator's x
        xr = synth.generate(w.x_spec(), w.seed, rows=toks)
        xq_r, xd_r = quant.quant_1x128(synth.as_f64(xr))
        assert np.array_equal(xq_all[toks], xq_r) and np.array_equal(xd_all[toks], xd_r)
        log(f"oracle expert {g} rows={rows.size}")
        w1q, w1d, w2q, w2d = _expert_oracle(w, g)
        resq = ffn.expert_ffn(xq_r, xd_r, w1q, w1d, w2q, w2d, "Q")
        resd = ffn.expert_ffn(xq_r, xd_r, w1q, w1d, w2q, w2d, "D")
        band = swiglu_band(xq_r, xd_r, w1q, w1d, resq["h"], resq["a"])
        hd_r = lay.hd.cpu().numpy()[rows]
        n_h = check_h(hq[rows], hd_r, resq, band)
        got = bf16_values(out_rows[torch.from_numpy(rows).cuda()])
        # expert rows against the oracle fed the GPU's own h codes, and, on
        # rows whose codes all equal the oracle's, against its own result
        fed = ffn.bf16_round(ffn.block_scaled_gemm(hq[rows], hd_r, w2q, w2d))
        same = ~np.any(hq[rows] != resq["hq"], axis=1)
        eq_fed = rel_l2(got, fed)
        eq_same = rel_l2(got[same], resq["out"][same]) if same.any() else 0.0
        ed = max_rel(got, resd["out"])
        print(f"expert {g}: rows {rows.size}, rel L2 vs Q fed the GPU's h codes {eq_fed:.2e}, "
              f"vs Q on the {same.sum()} rows with the oracle's codes {eq_same:.2e}, "
              f"max rel vs D {ed:.2e}, h codes differing {n_h}")
        assert eq_fed <= Q_BAR and eq_same <= Q_BAR and ed <= D_BAR

    if name == "decode":
        _check_tokens_end_to_end(w, lay, y, wr_b, b0, n_tokens=2)

    # combine: y is the shared row plus the gate-weighted routed rows (float
    # FMA chain in slot order), checked on a token sample
    ts = np.arange(0, T, max(1, T // 256))
    ob = bf16_values(out_rows)
    acc = ob[T * k + ts]
    for j in range(k):
        acc = ffn.fl32(acc + ffn.fl32(gate[ts, j])[:, None] * ob[row_of[ts, j]])
    yv = bf16_values(y)[ts]
    assert np.all(np.abs(yv - ffn.bf16_round(acc)) <= np.abs(yv) * 2.0 ** -7 + 1e-30)
    # bias: one float32 step of +-gamma or 0 by the integer load comparison
    want_b = (b0.astype(np.float64) + np.where(N * counts > T * k, -np.float32(w.gamma),
              np.where(N * counts < T * k, np.float32(w.gamma), 0.0))).astype(np.float32)
    assert np.array_equal(weights.bias.cpu().numpy(), want_b)


def test_layer_skew_ten_batches():
    """The skewed-load stress workload at its full size (T = 32768 per batch,
    DeepSeek-V3 shape, Zipf(1.2) per-expert logit offsets, 1 % of the
    activation channels x100): ten successive batches (batch b draws x with
    seed offset b) through one MoELayer, the bias updated after each.  Every
    batch: selection bit-exact on the GPU's own scores with the bias of that
    batch, counts equal to the routing, the bias update bit-exact, routing and
    activation codes against the float64 oracle on a token sample; the
    per-expert load max/mean is printed after each batch.  Batch 0 also checks
    the most loaded expert's FFN on a row sample."""
    from oracle import bias as obias
    moe = _moe()
    w = synth.WORKLOADS["skew"]
    weights, wr_b, b = _build_v3(w)
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma)
    T, k, N = w.T, w.k, w.N
    rng = np.random.default_rng(4)
    bias = b.copy()
    ratios = []
    for batch in range(w.batches):
        x = device_tensor(w.x_spec(batch), w.seed)
        log(f"skew batch {batch}")
        y = lay.forward(x)
        torch.cuda.synchronize()
        s_gpu = lay.scores.cpu().numpy()
        idx = lay.idx.cpu().numpy()
        counts = lay.counts.cpu().numpy()
        assert np.array_equal(idx, route.select_topk(s_gpu, bias, k))
        np.testing.assert_allclose(lay.gate.cpu().numpy(), route.gates(s_gpu, idx), rtol=2e-6,
                                   atol=1e-7)
        assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=N))
        new_bias = obias.bias_update(bias, counts, T, k, w.gamma)
        assert np.array_equal(weights.bias.cpu().numpy(), new_bias)
        # routing and activation codes against the oracle on 256 sampled tokens
        sample = np.sort(rng.choice(T, 256, replace=False))
        xb = synth.generate(w.x_spec(batch), w.seed, rows=sample)
        s64 = route.router_scores(synth.as_f64(xb), synth.as_f64(wr_b))
        assert np.max(np.abs(s_gpu[sample] - s64)) < 1e-5
        clear = route.topk_margin(s64, bias, k) > 3e-5
        assert clear.mean() > 0.95
        idx_o = route.select_topk(s64.astype(np.float32), bias, k)
        assert np.array_equal(idx[sample][clear], idx_o[clear])
        xq_o, xd_o = quant.quant_1x128(synth.as_f64(xb))
        assert np.array_equal(lay.xq.cpu().numpy()[sample], xq_o)
        assert np.array_equal(lay.xd.cpu().numpy()[sample], xd_o)
        ratio = counts.max() / counts.mean()
        ratios.append(ratio)
        print(f"batch {batch}: per-expert load max/mean {ratio:.2f}, "
              f"experts above 10x mean {(counts > 10 * counts.mean()).sum()}, "
              f"empty experts {(counts == 0).sum()}")
        if batch == 0:
            g = int(np.argmax(counts))
            offsets = lay.offsets.cpu().numpy()
            token_of = lay.token_of.cpu().numpy()
            r0 = int(offsets[g])
            rows = r0 + np.sort(rng.choice(int(counts[g]), 48, replace=False))
            toks = token_of[rows]
            xr = synth.generate(w.x_spec(batch), w.seed, rows=toks)
            xq_r, xd_r = quant.quant_1x128(synth.as_f64(xr))
            log(f"oracle skew expert {g} rows {rows.size}")
            w1q, w1d, w2q, w2d = _expert_oracle(w, g)
            resq = ffn.expert_ffn(xq_r, xd_r, w1q, w1d, w2q, w2d, "Q")
            resd = ffn.expert_ffn(xq_r, xd_r, w1q, w1d, w2q, w2d, "D")
            hq_r = lay.hq.cpu().numpy()[rows]
            hd_r = lay.hd.cpu().numpy()[rows]
            check_h(hq_r, hd_r, resq, swiglu_band(xq_r, xd_r, w1q, w1d, resq["h"], resq["a"]))
            got = bf16_values(lay.out_rows[torch.from_numpy(rows).cuda()])
            fed = ffn.bf16_round(ffn.block_scaled_gemm(hq_r, hd_r, w2q, w2d))
            assert rel_l2(got, fed) <= Q_BAR
            assert max_rel(got, resd["out"]) <= D_BAR
        bias = new_bias
        del y
    # the Zipf offsets give a strongly skewed load (design intent: a few
    # experts above 10x the mean)
    assert ratios[0] > 10


def test_layer_v3_shape_64k_tokens():
    """A 65,536-token batch at the DeepSeek-V3 shape (the prefill recipe):
    589,824 expert rows, expert outputs of 8.5 GB.  Routing and activation
    codes against the oracle on a token sample, the permutation's
    invariants, one expert's FFN on a row sample (codes and rows within the
    bars), the combine on sampled tokens and the bias update."""
    moe = _moe()
    base = synth.WORKLOADS["prefill"]
    w = synth.Workload("prefill64k", T=65536, H=base.H, N=base.N, k=base.k, I=base.I,
                       x_std=base.x_std, wr_dist=base.wr_dist, wr_param=base.wr_param,
                       bias_half=base.bias_half, w_std=base.w_std, seed=base.seed)
    weights, wr_b, b0 = _build_v3(w)
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma)
    x = device_tensor(w.x_spec(), w.seed)
    log("v3 forward T=65536")
    y = lay.forward(x)
    torch.cuda.synchronize()
    T, k, N = w.T, w.k, w.N
    idx = lay.idx.cpu().numpy()
    counts = lay.counts.cpu().numpy()
    offsets = lay.offsets.cpu().numpy()
    row_of = lay.row_of.cpu().numpy()
    token_of = lay.token_of.cpu().numpy()
    gate = lay.gate.cpu().numpy()
    rng = np.random.default_rng(64)
    sample = np.sort(rng.choice(T, 512, replace=False))
    xb = synth.generate(w.x_spec(), w.seed, rows=sample)
    s64 = route.router_scores(synth.as_f64(xb), synth.as_f64(wr_b))
    assert np.max(np.abs(lay.scores.cpu().numpy()[sample] - s64)) < 1e-5
    clear = route.topk_margin(s64, b0, k) > 3e-5
    idx_o = route.select_topk(s64.astype(np.float32), b0, k)
    assert np.array_equal(idx[sample][clear], idx_o[clear])
    xq_o, xd_o = quant.quant_1x128(synth.as_f64(xb))
    assert np.array_equal(lay.xq.cpu().numpy()[sample], xq_o)
    assert np.array_equal(lay.xd.cpu().numpy()[sample], xd_o)
    assert counts.sum() == T * k and offsets[-1] == T * k + T
    assert np.array_equal(np.sort(row_of.ravel()), np.arange(T * k))
    assert np.array_equal(token_of[row_of], np.repeat(np.arange(T)[:, None], k, 1))
    assert np.array_equal(token_of[T * k:], np.arange(T))
    # the most loaded routed expert, on a sample of its rows (its last rows
    # sit far into the [R, H] output, past 2^31 bytes)
    g = int(np.argmax(counts))
    rows = int(offsets[g]) + np.sort(rng.choice(int(counts[g]), 32, replace=False))
    rows = np.concatenate([rows, np.arange(lay.R - 8, lay.R)])           # shared rows at the end
    toks = token_of[rows]
    log(f"oracle experts {g} and shared, {rows.size} rows")
    xr = synth.generate(w.x_spec(), w.seed, rows=toks)
    xq_r, xd_r = quant.quant_1x128(synth.as_f64(xr))
    hq = lay.hq.cpu().numpy()
    hd = lay.hd.cpu().numpy()
    got = bf16_values(lay.out_rows[torch.from_numpy(rows).cuda()])
    for sel, ge in ((slice(0, 32), g), (slice(32, None), N)):
        w1q, w1d, w2q, w2d = _expert_oracle(w, ge)
        resq = ffn.expert_ffn(xq_r[sel], xd_r[sel], w1q, w1d, w2q, w2d, "Q")
        resd = ffn.expert_ffn(xq_r[sel], xd_r[sel], w1q, w1d, w2q, w2d, "D")
        band = swiglu_band(xq_r[sel], xd_r[sel], w1q, w1d, resq["h"], resq["a"])
        check_h(hq[rows[sel]], hd[rows[sel]], resq, band)
        fed = ffn.bf16_round(ffn.block_scaled_gemm(hq[rows[sel]], hd[rows[sel]], w2q, w2d))
        assert rel_l2(got[sel], fed) <= Q_BAR
        assert max_rel(got[sel], resd["out"]) <= D_BAR
    # combine on the last tokens (their shared rows are the last rows of [R, H])
    ts = np.arange(T - 16, T)
    acc = bf16_values(lay.out_rows[torch.from_numpy(T * k + ts).cuda()])
    for j in range(k):
        acc = ffn.fl32(acc + ffn.fl32(gate[ts, j])[:, None] *
                       bf16_values(lay.out_rows[torch.from_numpy(row_of[ts, j]).cuda()]))
    yv = bf16_values(y)[ts]
    assert np.all(np.abs(yv - ffn.bf16_round(acc)) <= np.abs(yv) * 2.0 ** -7 + 1e-30)
    want_b = (b0.astype(np.float64) + np.where(N * counts > T * k, -np.float32(w.gamma),
              np.where(N * counts < T * k, np.float32(w.gamma), 0.0))).astype(np.float32)
    assert np.array_equal(weights.bias.cpu().numpy(), want_b)


@pytest.mark.parametrize("T,H,N,k,I", [(64, 256, 16, 2, 128), (200, 1024, 8, 3, 512),
                                       (48, 7168, 4, 2, 2048)])
def test_gemm2_combine_rounding_faithful(T, H, N, k, I):
    """GEMM2 + combine fed the same h codes on both sides (codes made by the
    oracle's quantiser from generated values): the rounding-faithful bar."""
    moe = _moe()
    rng = np.random.default_rng(T + H)
    idx = np.argsort(rng.uniform(size=(T, N)), 1)[:, :k].astype(np.int32)
    from oracle import permute as opermute
    counts, offsets, row_of, token_of = opermute.permute(idx, N, True)
    R = T * k + T
    h = synth.as_f64(synth.generate(synth.Spec(synth.T_ROWS, (R, I), synth.NORMAL, 0.3), T))
    hq, hd = quant.quant_1x128(h)
    w2 = synth.generate(synth.Spec(synth.T_W2, (N + 1, H, I), synth.NORMAL, 0.006), T)
    w2q, w2d = quant.quant_128x128(synth.as_f64(w2))
    gate = rng.uniform(0.05, 1, (T, k)).astype(np.float32)
    gate /= gate.sum(1, keepdims=True)
    log(f"gemm2+combine T={T} H={H} N={N} k={k} I={I}")
    out, _ = moe.moe_grouped_gemm_fp8(to_dev(hq), to_dev(hd), to_dev(w2q), to_dev(w2d),
                                      to_dev(offsets), R, moe.MOE_EPI_BF16)
    y = moe.moe_combine(out, to_dev(gate), to_dev(row_of), T * k)
    torch.cuda.synchronize()
    want_out = np.zeros((R, H))
    for g in range(N + 1):
        rr = slice(offsets[g], offsets[g + 1])
        if offsets[g + 1] > offsets[g]:
            want_out[rr] = ffn.bf16_round(ffn.block_scaled_gemm(hq[rr], hd[rr], w2q[g], w2d[g]))
    want_y = ffn.combine(want_out, gate.astype(np.float64), row_of, T * k, "Q")
    err_out = rel_l2(bf16_values(out), want_out)
    err = rel_l2(bf16_values(y), want_y)
    print(f"rel L2: expert rows {err_out:.3e}, y {err:.3e}")
    assert err_out <= Q_BAR and err <= Q_BAR


def test_layers_on_two_streams_from_two_threads():
    """The library keeps no state between calls: two layers (own weights and
    bias), each driven by its own host thread on its own stream (default
    priority) for three batches, give bit for bit what the same layers give
    when run one after the other."""
    import threading
    moe = _moe()
    w = synth.Workload("threads", T=300, H=512, N=32, k=4, I=256, x_std=1.0,
                       wr_dist=synth.NORMAL, wr_param=0.05, bias_half=0.1, w_std=0.02, seed=9)
    wr = bf16_to_dev(w.router_weight())
    w1 = bf16_to_dev(synth.generate(w.w1_spec(), w.seed))
    w2 = bf16_to_dev(synth.generate(w.w2_spec(), w.seed))
    b0 = to_dev(w.bias().copy())
    xs = [bf16_to_dev(synth.generate(w.x_spec(b), w.seed)) for b in range(6)]

    def make():
        weights = moe.MoEWeights(wr, b0.clone(), w1_bf16=w1, w2_bf16=w2)
        return moe.MoELayer(weights, w.T, w.k, w.gamma)

    # reference: layer A on batches 0-2, then layer B on batches 3-5
    ref = []
    for lay, batches in ((make(), xs[:3]), (make(), xs[3:])):
        ref.append([lay.forward(x).clone() for x in batches] + [lay.w.bias.clone()])
    torch.cuda.synchronize()

    layers = [make(), make()]
    torch.cuda.synchronize()          # weights and bias copies made on the default stream
    results = [None, None]
    errors = []

    def run(i):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                outs = [layers[i].forward(x, stream=st).clone() for x in xs[3 * i:3 * i + 3]]
                outs.append(layers[i].w.bias.clone())
            st.synchronize()
            results[i] = outs
        except Exception as e:                     # reported below
            errors.append(e)

    log("two layers, two streams, two host threads")
    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for i in range(2):
        for got, want in zip(results[i], ref[i]):
            assert torch.equal(got, want)


def test_layer_empty_batch():
    """T = 0 through the whole layer: every call is a no-op that succeeds, y
    is empty, and the bias stays put (zero load equals the zero target)."""
    moe = _moe()
    w = synth.WORKLOADS["tiny"]
    b = w.bias()
    weights = moe.MoEWeights(bf16_to_dev(w.router_weight()), to_dev(b.copy()),
                             w1_bf16=bf16_to_dev(synth.generate(w.w1_spec(), w.seed)),
                             w2_bf16=bf16_to_dev(synth.generate(w.w2_spec(), w.seed)))
    log("layer T=0")
    lay = moe.MoELayer(weights, 0, w.k, w.gamma)
    y = lay.forward(torch.empty(0, w.H, dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, w.H)
    assert np.array_equal(lay.counts.cpu().numpy(), np.zeros(w.N, np.int32))
    assert np.array_equal(weights.bias.cpu().numpy(), b)


@pytest.mark.parametrize("router_fp8", [False, True])
def test_layer_forward_graph_replay(router_fp8):
    """MoELayer.forward allocates nothing, clears nothing with a memset and
    syncs nothing, so one step can be captured in a HIP graph and replayed.
    Four replays, each on a new batch copied into the graph's input buffer
    (eager work and a synchronisation between replays), every one bit-exact
    against a twin layer run eagerly on the same batches -- output, routing,
    maps and the bias each step updates."""
    moe = _moe()
    w = synth.Workload("graph", T=300, H=512, N=128 if router_fp8 else 32, k=4, I=256, x_std=1.0,
                       wr_dist=synth.NORMAL, wr_param=0.05, bias_half=0.1, w_std=0.02, seed=7)
    wr = bf16_to_dev(w.router_weight())
    w1 = bf16_to_dev(synth.generate(w.w1_spec(), w.seed))
    w2 = bf16_to_dev(synth.generate(w.w2_spec(), w.seed))
    b0 = to_dev(w.bias().copy())
    layers = []
    for _ in range(2):
        weights = moe.MoEWeights(wr, b0.clone(), w1_bf16=w1, w2_bf16=w2, router_fp8=router_fp8)
        layers.append(moe.MoELayer(weights, w.T, w.k, w.gamma, router_fp8=router_fp8))
    eager, graphed = layers
    xs = [bf16_to_dev(synth.generate(w.x_spec(b), w.seed)) for b in range(4)]
    log(f"graph capture of MoELayer.forward router_fp8={router_fp8}")
    x_static = torch.empty_like(xs[0])
    x_static.copy_(xs[0])
    graphed.forward(x_static, update_bias=False)      # first launches outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_static = graphed.forward(x_static)
    torch.cuda.synchronize()
    graphed.w.bias.copy_(b0)                           # the capture itself ran nothing
    for b, x in enumerate(xs):
        y_e = eager.forward(x).clone()
        torch.cuda.synchronize()
        x_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_e), f"replay {b}: output differs"
        assert torch.equal(graphed.idx, eager.idx), f"replay {b}: routing differs"
        assert torch.equal(graphed.token_of, eager.token_of), f"replay {b}: row map differs"
        assert torch.equal(graphed.w.bias, eager.w.bias), f"replay {b}: bias differs"
    assert not torch.equal(eager.w.bias, b0)           # the bias did move
