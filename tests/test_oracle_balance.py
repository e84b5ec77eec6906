"""Pins of the sequence-wise balance statistic.

Source: "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
Prediction, and FP8 Training at 671B Scale", section III, "The one small loss
that remains" (L_Bal = alpha sum_i f_i P_i, alpha = 1e-4, per sequence)."""
import numpy as np

from oracle import balance, route


def test_perfectly_even_routing_gives_alpha():
    """Every expert chosen equally often with uniform gates 1/k: f_i = 1,
    P_i = 1/N, so L = alpha exactly (closed form)."""
    N, k, T = 16, 4, 32
    idx = np.array([[(4 * t + j) % N for j in range(k)] for t in range(T)])
    gate = np.full((T, k), 1.0 / k)
    L = balance.seq_balance_loss(idx, gate, [0, T], N, alpha=1e-4)
    assert abs(L[0] - 1e-4) < 1e-18


def test_collapsed_routing_gives_alpha_n_over_k():
    """All tokens on the same k experts with equal gates: f_i = N/k on those,
    P_i = 1/k, L = alpha * N / k (closed form)."""
    N, k, T = 256, 8, 100
    idx = np.tile(np.arange(k), (T, 1))
    gate = np.full((T, k), 1.0 / k)
    L = balance.seq_balance_loss(idx, gate, [0, T], N, alpha=2.0)
    assert abs(L[0] - 2.0 * N / k) < 1e-12


def test_hand_computed_example_and_sequence_split():
    """N = 4, k = 2, two tokens; counts (2, 1, 1, 0), masses (0.7+0.6, 0.3,
    0.4, 0): f = 4/(2*2) * counts = counts, P = masses / 2, so
    sum f P = 2*0.65 + 1*0.15 + 1*0.2 = 1.65.  Sequences are independent and
    an empty one gives 0."""
    idx = np.array([[0, 1], [0, 2], [3, 1]])
    gate = np.array([[0.7, 0.3], [0.6, 0.4], [0.5, 0.5]])
    L = balance.seq_balance_loss(idx, gate, [0, 2, 2, 3], 4, alpha=1.0)
    assert abs(L[0] - 1.65) < 1e-15
    assert L[1] == 0.0
    # one token with gates 0.5 on experts 3 and 1: f = 2 on each, P = 0.5
    assert abs(L[2] - 2.0) < 1e-15


def test_gates_from_the_router_sum_to_one_so_mass_is_one():
    """With the oracle's gates (normalised over the chosen experts) the gate
    masses of a sequence sum to 1 and f averages 1, whatever the routing."""
    rng = np.random.default_rng(1)
    s = rng.uniform(0, 1, (64, 32)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    idx = route.select_topk(s, b, 4)
    g = route.gates(s, idx)
    count = np.bincount(idx.ravel(), minlength=32)
    mass = np.bincount(idx.ravel(), weights=g.ravel(), minlength=32)
    assert abs(mass.sum() / 64 - 1.0) < 1e-12
    assert abs((32 / (4 * 64) * count).mean() - 1.0) < 1e-12
    L = balance.seq_balance_loss(idx, g, [0, 64], 32, alpha=1.0)[0]
    assert abs(L - np.sum(32 / (4 * 64) * count * mass / 64)) < 1e-12
