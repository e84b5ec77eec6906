"""Sign-based bias update -- test infrastructure, see ``oracle/__init__``.

What is computed ([TP] section III, "How the bias is set" and the per-step
control-loop flowchart; [VE] recipe step 4 and the glossary for b_i and
gamma; [DF] "Balancing without a balance loss"): after each step every
expert's load is compared with the balanced target; an overloaded expert's
bias falls by gamma, an underloaded one's rises by gamma.  gamma = 0 freezes
the biases.  No gradient is involved.

Readings where the pages leave a step open:
  * the balanced target is T*k/N per expert; the comparison is done exactly in
    integers as N*c_i against T*k;
  * an expert exactly on target keeps its bias (the sign of a zero error is 0);
  * the bias is float32 and the update is one float32 add of fl32(gamma).
  (One page prints the update with the opposite sign; the prose of every page,
  including that one, says overloaded experts go down, which is what is done.)
"""
import numpy as np


def bias_update(bias, counts, T, k, gamma):
    """Returns the new float32 bias [N]."""
    b = np.asarray(bias, np.float32).astype(np.float64)
    c = np.asarray(counts, np.int64)
    N = c.shape[0]
    g = float(np.float32(gamma))
    load = N * c
    target = int(T) * int(k)
    step = np.where(load > target, -g, np.where(load < target, g, 0.0))
    return (b + step).astype(np.float32)
