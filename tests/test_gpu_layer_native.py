"""The one-call layer entry point (moe_layer_forward through the C ABI).

It enqueues the same kernels as MoELayer.forward, so every output -- y, the
routing, the counts, the scores and the updated bias -- must be bit-identical
to the step-by-step path on the same inputs; the tiny layer is also checked
against the oracle directly, to the end-to-end bars of the layer tests.
"""
import numpy as np
import pytest

import synth
from helpers import bf16_to_dev, bf16_values, log, max_rel, rel_l2, to_dev
from oracle import layer as olayer, route

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

D_BAR = 2e-2        # normwise max relative error vs the float64 oracle
E2E_Q_BAR = 5e-3    # relative L2 vs the rounding-faithful oracle, end to end


def _moe():
    import fp8_block_scaled_sigmoid_amd as moe
    return moe


def _weights(w, router_fp8=False, shared=True):
    moe = _moe()
    w1 = bf16_to_dev(synth.generate(w.w1_spec(), w.seed))
    w2 = bf16_to_dev(synth.generate(w.w2_spec(), w.seed))
    if not shared:                  # drop the shared expert (the last one)
        w1, w2 = w1[:w.N].contiguous(), w2[:w.N].contiguous()

    def make():
        return moe.MoEWeights(bf16_to_dev(w.router_weight()), to_dev(w.bias().copy()),
                              w1_bf16=w1, w2_bf16=w2, router_fp8=router_fp8)
    return make


def _outputs(T, N, k):
    return dict(scores=torch.empty(T, N, dtype=torch.float32, device="cuda"),
                idx=torch.empty(T, k, dtype=torch.int32, device="cuda"),
                gate=torch.empty(T, k, dtype=torch.float32, device="cuda"),
                counts=torch.empty(N, dtype=torch.int32, device="cuda"))


def test_native_layer_tiny_against_oracle():
    moe = _moe()
    w = synth.WORKLOADS["tiny"]
    x_b = synth.generate(w.x_spec(), w.seed)
    weights = _weights(w)()
    out = _outputs(w.T, w.N, w.k)
    log(f"moe_layer_forward tiny T={w.T} H={w.H} N={w.N} k={w.k} I={w.I}")
    y = bf16_values(moe.moe_layer_forward(weights, bf16_to_dev(x_b), w.k, w.gamma, **out))
    torch.cuda.synchronize()
    args = (synth.as_f64(x_b), synth.as_f64(w.router_weight()), w.bias(),
            synth.as_f64(synth.generate(w.w1_spec(), w.seed)),
            synth.as_f64(synth.generate(w.w2_spec(), w.seed)), w.k, w.gamma)
    q = olayer.moe_layer(*args, precision="Q")
    assert np.all(route.topk_margin(q["s64"], args[2], w.k) > 3e-5)
    assert np.array_equal(out["idx"].cpu().numpy(), q["idx"])
    assert np.array_equal(out["counts"].cpu().numpy(), q["counts"])
    np.testing.assert_allclose(out["gate"].cpu().numpy(), q["gate"], rtol=1e-5, atol=1e-6)
    assert np.array_equal(weights.bias.cpu().numpy(), q["bias"])
    assert rel_l2(y, q["y"]) <= E2E_Q_BAR
    assert max_rel(y, olayer.moe_layer(*args, precision="D")["y"]) <= D_BAR


CASES = [
    # name,           T,   H,   N,   k, I,   shared, groups, fp8 router, residual, update
    ("plain",         300, 512, 32,  4, 256, True,  (1, 1), False, False, True),
    ("ragged",        37,  384, 16,  16, 128, True, (1, 1), False, False, True),
    ("no_shared",     300, 512, 32,  4, 256, False, (1, 1), False, False, True),
    ("grouped",       300, 512, 32,  4, 256, True,  (4, 2), False, False, True),
    ("fp8_router",    300, 512, 128, 4, 256, True,  (1, 1), True,  False, True),
    ("fp8_grouped",   200, 256, 128, 8, 128, True,  (8, 4), True,  False, True),
    ("residual",      129, 256, 16,  2, 128, True,  (1, 1), False, True,  False),
    ("empty",         0,   256, 16,  2, 128, True,  (1, 1), False, False, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_native_layer_matches_step_by_step(case):
    name, T, H, N, k, I, shared, (ng, tg), fp8r, with_res, update = case
    moe = _moe()
    w = synth.Workload(f"native_{name}", T=T, H=H, N=N, k=k, I=I, x_std=1.0,
                       wr_dist=synth.NORMAL, wr_param=0.05, bias_half=0.1, w_std=0.02, seed=11)
    make = _weights(w, router_fp8=fp8r, shared=shared)
    ref_w, nat_w = make(), make()
    x = bf16_to_dev(synth.generate(w.x_spec(), w.seed)) if T else \
        torch.empty(0, H, dtype=torch.bfloat16, device="cuda")
    residual = bf16_to_dev(synth.generate(w.x_spec(1), w.seed)) if with_res else None
    log(f"moe_layer_forward {name} T={T} H={H} N={N} k={k} I={I}")
    lay = moe.MoELayer(ref_w, T, k, w.gamma, n_groups=ng, topk_groups=tg, router_fp8=fp8r)
    y_ref = lay.forward(x, update_bias=update)
    if with_res:
        y_ref = moe.moe_combine(lay.out_rows, lay.gate, lay.row_of,
                                T * k if shared else -1, residual=residual)
    out = _outputs(T, N, k)
    y = moe.moe_layer_forward(nat_w, x, k, w.gamma, n_groups=ng, topk_groups=tg,
                              router_fp8=fp8r, update_bias=update, residual=residual, **out)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, H)
    assert torch.equal(y, y_ref)
    assert torch.equal(out["idx"], lay.idx)
    assert torch.equal(out["gate"], lay.gate)
    assert torch.equal(out["scores"], lay.scores)
    assert torch.equal(out["counts"], lay.counts)
    assert torch.equal(nat_w.bias, ref_w.bias)
    if update and T and k < N:       # with k = N every expert is exactly on target
        assert not torch.equal(nat_w.bias, to_dev(w.bias().copy()))


def test_native_layer_workspace_reused_for_a_smaller_batch():
    """Two calls in a row on one workspace, the second with fewer tokens, and
    one call whose optional outputs all live in the workspace: each gives what
    the step-by-step path gives."""
    moe = _moe()
    w = synth.Workload("native_ws", T=300, H=512, N=32, k=4, I=256, x_std=1.0,
                       wr_dist=synth.NORMAL, wr_param=0.05, bias_half=0.1, w_std=0.02, seed=5)
    make = _weights(w)
    ref_w, nat_w = make(), make()
    ws = torch.empty(moe.moe_layer_workspace_bytes(w.T, w.H, w.N, w.k, w.I), dtype=torch.uint8,
                     device="cuda")
    log("moe_layer_forward on one workspace: T=300 then T=77")
    for b, T in enumerate((300, 77)):
        x = bf16_to_dev(synth.generate(w.x_spec(b), w.seed))[:T].contiguous()
        lay = moe.MoELayer(ref_w, T, w.k, w.gamma)
        y_ref = lay.forward(x)
        y = moe.moe_layer_forward(nat_w, x, w.k, w.gamma, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {b}"
        assert torch.equal(nat_w.bias, ref_w.bias), f"call {b}"


def test_native_layer_rejects_a_short_workspace():
    moe = _moe()
    w = synth.WORKLOADS["tiny"]
    weights = _weights(w)()
    x = bf16_to_dev(synth.generate(w.x_spec(), w.seed))
    need = moe.moe_layer_workspace_bytes(w.T, w.H, w.N, w.k, w.I)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    bias0 = weights.bias.clone()
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_forward(weights, x, w.k, w.gamma, ws=ws)
    assert e.value.code == 4                                # MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(weights.bias, bias0)                 # nothing was enqueued


def test_native_layer_graph_replay():
    """The one call captured in a HIP graph: four replays on new batches, each
    bit-exact against the step-by-step path run eagerly on the same batches."""
    moe = _moe()
    w = synth.Workload("native_graph", T=300, H=512, N=32, k=4, I=256, x_std=1.0,
                       wr_dist=synth.NORMAL, wr_param=0.05, bias_half=0.1, w_std=0.02, seed=3)
    make = _weights(w)
    ref_w, nat_w = make(), make()
    b0 = nat_w.bias.clone()
    eager = moe.MoELayer(ref_w, w.T, w.k, w.gamma)
    xs = [bf16_to_dev(synth.generate(w.x_spec(b), w.seed)) for b in range(4)]
    x_static = xs[0].clone()
    y_static = torch.empty_like(x_static)
    ws = torch.empty(moe.moe_layer_workspace_bytes(w.T, w.H, w.N, w.k, w.I), dtype=torch.uint8,
                     device="cuda")
    log("graph capture of moe_layer_forward")
    moe.moe_layer_forward(nat_w, x_static, w.k, w.gamma, update_bias=False, y=y_static, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer_forward(nat_w, x_static, w.k, w.gamma, y=y_static, ws=ws,
                              stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    nat_w.bias.copy_(b0)
    for b, x in enumerate(xs):
        y_e = eager.forward(x).clone()
        torch.cuda.synchronize()
        x_static.copy_(x)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_e), f"replay {b}: output differs"
        assert torch.equal(nat_w.bias, ref_w.bias), f"replay {b}: bias differs"


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_native_layer_v3_shape_matches_step_by_step(name):
    """At the DeepSeek-V3 shapes (H 7168, 256 routed experts top-8 + 1 shared,
    I 2048; T = 512 and 8192), one moe_layer_forward call gives bit for bit
    the step-by-step path's output, routing, counts and updated bias (which the
    layer tests hold against the oracle on sampled experts)."""
    from helpers import device_tensor
    moe = _moe()
    w = synth.WORKLOADS[name]
    log(f"moe_layer_forward v3 {name} T={w.T}")
    w1 = device_tensor(w.w1_spec(), w.seed)
    w1q, w1d = moe.fp8_quant_128x128(w1, interleave_gate_up=True)
    del w1
    w2 = device_tensor(w.w2_spec(), w.seed)
    w2q, w2d = moe.fp8_quant_128x128(w2)
    del w2
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    wr = bf16_to_dev(w.router_weight())
    b0 = to_dev(w.bias().copy())
    ref_w = moe.MoEWeights(wr, b0.clone(), w1q=w1q, w1d=w1d, w2q=w2q, w2d=w2d)
    nat_w = moe.MoEWeights(wr, b0.clone(), w1q=w1q, w1d=w1d, w2q=w2q, w2d=w2d)
    x = device_tensor(w.x_spec(), w.seed)
    lay = moe.MoELayer(ref_w, w.T, w.k, w.gamma)
    y_ref = lay.forward(x)
    out = _outputs(w.T, w.N, w.k)
    y = moe.moe_layer_forward(nat_w, x, w.k, w.gamma, **out)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(out["idx"], lay.idx)
    assert torch.equal(out["counts"], lay.counts)
    assert torch.equal(nat_w.bias, ref_w.bias)
    assert not torch.equal(nat_w.bias, b0)
