"""Pins of the oracle's bias update and of the whole tiny layer.

Sources: "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
Prediction, and FP8 Training at 671B Scale", section III ("How the bias is
set": overloaded -> b -= gamma, underloaded -> b += gamma; the per-step
control-loop flowchart); "DeepSeek-V3, explained.", recipe step 4 and the
paragraph after the glossary (gamma = 0 freezes the biases; the bias never
touches the gate weights).
"""
import numpy as np
import pytest

import synth
from oracle import bias, ffn, layer, permute, route


def test_update_closed_form_and_direction():
    b = np.array([0.5, -0.25, 0.0, 1e-3], np.float32)
    counts = np.array([5, 3, 4, 4])                  # T*k = 16 over N = 4: target 4
    nb = bias.bias_update(b, counts, T=8, k=2, gamma=1e-3)
    g = np.float32(1e-3)
    assert nb[0] == np.float32(b[0] - g)             # overloaded goes down
    assert nb[1] == np.float32(b[1] + g)             # underloaded goes up
    assert nb[2] == b[2] and nb[3] == b[3]           # on target: unchanged
    # the step is one float32 add, so b' - b is gamma only up to b's rounding
    d = nb.astype(np.float64) - b.astype(np.float64)
    assert np.all(np.abs(np.abs(d[:2]) - float(g)) <= np.spacing(np.abs(b[:2])))


def test_gamma_zero_freezes():
    rng = np.random.default_rng(1)
    b = rng.uniform(-1, 1, 64).astype(np.float32)
    counts = rng.integers(0, 100, 64)
    assert np.array_equal(bias.bias_update(b, counts, 50, 8, 0.0), b)


def test_non_integral_target_uses_exact_comparison():
    # T*k = 7, N = 3: the target 7/3 is not an integer; counts 2 < 7/3 < 3
    nb = bias.bias_update(np.zeros(3, np.float32), np.array([2, 3, 2]), T=7, k=1, gamma=0.5)
    assert nb.tolist() == [0.5, -0.5, 0.5]


def test_controller_balances_a_skewed_router():
    """Closing the loop (route -> counts -> update) on fixed skewed scores drives
    the load towards the balanced target, as the thermostat is meant to."""
    rng = np.random.default_rng(2)
    T, N, k = 512, 16, 2
    z = rng.standard_normal((T, N)) + np.linspace(2.0, -2.0, N)[None, :]
    s32 = route.sigmoid(z).astype(np.float32)
    b = np.zeros(N, np.float32)

    def imbalance(b):
        idx = route.select_topk(s32, b, k)
        c = np.bincount(idx.reshape(-1), minlength=N)
        return c.max() / (T * k / N), c

    start, _ = imbalance(b)
    for _ in range(400):
        _, c = imbalance(b)
        b = bias.bias_update(b, c, T, k, 1e-2)
    end, _ = imbalance(b)
    assert start > 3.0 and end < 1.3


def _tiny_inputs():
    w = synth.WORKLOADS["tiny"]
    x = synth.as_f64(synth.generate(w.x_spec(), w.seed))
    wr = synth.as_f64(w.router_weight())
    b = w.bias()
    w1 = synth.as_f64(synth.generate(w.w1_spec(), w.seed))
    w2 = synth.as_f64(synth.generate(w.w2_spec(), w.seed))
    return w, x, wr, b, w1, w2


def test_tiny_layer_invariants_and_precisions():
    w, x, wr, b, w1, w2 = _tiny_inputs()
    d = layer.moe_layer(x, wr, b, w1, w2, w.k, w.gamma, precision="D")
    q = layer.moe_layer(x, wr, b, w1, w2, w.k, w.gamma, precision="Q")
    assert d["counts"].sum() == w.T * w.k
    assert np.all(np.isfinite(d["y"])) and np.abs(d["y"]).max() > 0
    rel = np.linalg.norm(q["y"] - d["y"]) / np.linalg.norm(d["y"])
    assert rel < 1e-2
    # the output is the shared row plus the gate-weighted routed rows
    t = 5
    want = d["out"][w.T * w.k + t] + sum(d["gate"][t, j] * d["out"][d["row_of"][t, j]]
                                         for j in range(w.k))
    np.testing.assert_allclose(d["y"][t], want, rtol=1e-14)
    # bias moved by exactly +-gamma or 0
    step = d["bias"].astype(np.float64) - b.astype(np.float64)
    assert np.all(np.isclose(np.abs(step), np.float32(w.gamma), rtol=1e-3) | (step == 0))


def test_tiny_layer_zero_input_and_k1():
    w, x, wr, b, w1, w2 = _tiny_inputs()
    d = layer.moe_layer(np.zeros_like(x), wr, b, w1, w2, w.k, w.gamma)
    assert np.all(d["y"] == 0.0)
    d1 = layer.moe_layer(x, wr, b, w1, w2, 1, w.gamma, precision="Q")
    assert np.all(d1["gate"] == 1.0)
    T = w.T
    want = ffn.bf16_round(ffn.fl32(d1["out"][T:2 * T] + d1["out"][d1["row_of"][:, 0]]))
    np.testing.assert_array_equal(d1["y"], want)


def test_tiny_layer_weights_quantised_per_expert():
    w, x, wr, b, w1, w2 = _tiny_inputs()
    wq = layer.quantise_weights(w1, w2)
    assert wq["w1q"].shape == (w.G, 2 * w.I, w.H) and wq["w1d"].shape == (w.G, 2, 2)
    assert wq["w2q"].shape == (w.G, w.H, w.I) and wq["w2d"].shape == (w.G, 2, 1)
