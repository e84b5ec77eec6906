"""Per-expert counts and the token permutation -- test infrastructure.

What is computed.  No token is dropped and there is no capacity limit ([VE]
recipe step 5, last sentence; [DF] "Balancing without a balance loss"), so
every (token, slot) assignment gets its own row of the expert's group.  The
per-expert token counts are what the bias controller reads ([TP] section III,
flowchart: "token counts" flowing from TopK into "measure per-expert load").

  counts[e]    = #{(t, j) : idx[t, j] = e}
  offsets[e]   = sum_{e' < e} counts[e']           (offsets[N] = T*k)
  row_of[t, j] = offsets[e] + #{(t', j') before (t, j) in (t, j) order with
                 idx[t', j'] = e},  e = idx[t, j]
  token_of[row_of[t, j]] = t

Readings where the pages leave a step open:
  * rows of one group are ordered by token (then slot), so the result is
    unique and deterministic;
  * the shared expert, which every token uses at full weight ([VE] glossary,
    "FFN^(s)"), is appended as group N with rows T*k + t -> t, and
    offsets[N + 1] = T*k + T.  Without it, offsets[N + 1] = T*k.
"""
import numpy as np


def permute(idx, n_experts, with_shared=True):
    """idx: int [T, k].  Returns (counts int32 [N], offsets int32 [N+2],
    row_of int32 [T, k], token_of int32 [T*k (+T)])."""
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.reshape(-1)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int64)
    offsets = np.zeros(n_experts + 2, dtype=np.int64)
    offsets[1:n_experts + 1] = np.cumsum(counts)
    offsets[n_experts + 1] = T * k + (T if with_shared else 0)
    order = np.argsort(flat, kind="stable")   # expert-major, (t, j) ascending
    row_of_flat = np.empty(T * k, dtype=np.int64)
    row_of_flat[order] = np.arange(T * k)
    token_of = np.empty(T * k + (T if with_shared else 0), dtype=np.int64)
    token_of[row_of_flat] = np.arange(T * k) // k
    if with_shared:
        token_of[T * k:] = np.arange(T)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            row_of_flat.reshape(T, k).astype(np.int32), token_of.astype(np.int32))
