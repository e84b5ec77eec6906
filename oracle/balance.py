"""Sequence-wise balance statistic -- test infrastructure, see ``oracle/__init__``.

What is computed ([TP] section III, "The one small loss that remains": the
complementary sequence-wise balance loss L_Bal = alpha * sum_i f_i P_i with
alpha = 1e-4, over the T tokens of one sequence; [VE] recipe step 4: the
sequence-level balance loss with weight 0.0001; [DF] "Balancing without a
balance loss": a complementary sequence-wise loss with a very small weight).

Readings where the pages leave a step open:
  * f_i, the "per-expert normalised load", is the number of the sequence's
    (token, slot) assignments that chose expert i, normalised so that a
    perfectly even load gives 1:  f_i = N / (K_r T) * count_i;
  * P_i, the "mean gate mass", is the mean over the sequence's tokens of the
    gate weight expert i receives (0 where i is not chosen), so sum_i P_i = 1;
  * sequences are given by token offsets; an empty sequence has L = 0.
Everything in float64.
"""
import numpy as np


def seq_balance_loss(idx, gate, seq_offsets, n_experts, alpha=1e-4):
    """idx [T, k] int, gate [T, k] float, seq_offsets [S + 1] -> L [S] float64."""
    idx = np.asarray(idx, np.int64)
    gate = np.asarray(gate, np.float64)
    k = idx.shape[1]
    out = np.zeros(len(seq_offsets) - 1)
    for s in range(len(seq_offsets) - 1):
        t0, t1 = int(seq_offsets[s]), int(seq_offsets[s + 1])
        T = t1 - t0
        if T == 0:
            continue
        count = np.zeros(n_experts)
        mass = np.zeros(n_experts)
        for t in range(t0, t1):
            for j in range(k):
                count[idx[t, j]] += 1
                mass[idx[t, j]] += gate[t, j]
        f = n_experts / (k * T) * count
        P = mass / T
        out[s] = alpha * np.sum(f * P)
    return out
