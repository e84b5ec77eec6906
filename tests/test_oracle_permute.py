"""Pins of the oracle's counts and token permutation.

Sources: "DeepSeek-V3, explained.", recipe step 5 (no tokens are dropped);
"DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction,
and FP8 Training at 671B Scale", section III flowchart (TopK feeds token
counts to the load measurement).
"""
import numpy as np
import pytest

from oracle import permute


def _brute(idx, n):
    """Pure-Python counting sort over (token, slot) pairs."""
    T, k = len(idx), len(idx[0])
    counts = [0] * n
    for t in range(T):
        for j in range(k):
            counts[idx[t][j]] += 1
    offsets = [0]
    for e in range(n):
        offsets.append(offsets[-1] + counts[e])
    fill = list(offsets[:n])
    row_of = [[None] * k for _ in range(T)]
    token_of = [None] * (T * k + T)
    for t in range(T):
        for j in range(k):
            e = idx[t][j]
            row_of[t][j] = fill[e]
            token_of[fill[e]] = t
            fill[e] += 1
    for t in range(T):
        token_of[T * k + t] = t
    offsets.append(T * k + T)
    return counts, offsets, row_of, token_of


def _random_idx(rng, T, n, k):
    return np.array([rng.choice(n, k, replace=False) for _ in range(T)], dtype=np.int32)


@pytest.mark.parametrize("T,n,k", [(1, 4, 1), (17, 8, 3), (64, 16, 2), (33, 5, 5)])
def test_matches_brute_force(T, n, k):
    rng = np.random.default_rng(T + n + k)
    idx = _random_idx(rng, T, n, k)
    counts, offsets, row_of, token_of = permute.permute(idx, n, True)
    bc, bo, br, bt = _brute(idx.tolist(), n)
    assert counts.tolist() == bc and offsets.tolist() == bo
    assert row_of.tolist() == br and token_of.tolist() == bt


def test_invariants_at_scale():
    rng = np.random.default_rng(1)
    T, n, k = 2000, 64, 6
    idx = _random_idx(rng, T, n, k)
    counts, offsets, row_of, token_of = permute.permute(idx, n, True)
    assert counts.sum() == T * k                                     # nothing dropped
    assert np.array_equal(np.sort(row_of.reshape(-1)), np.arange(T * k))   # bijection
    assert np.array_equal(token_of[row_of], np.repeat(np.arange(T)[:, None], k, 1))
    for e in range(n):
        toks = token_of[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(toks) > 0)                              # stable by token
        assert np.all(np.any(idx[toks] == e, axis=1))
    assert np.array_equal(token_of[T * k:], np.arange(T))
    assert offsets[n + 1] == T * k + T


def test_without_shared_group():
    idx = np.array([[1, 0], [0, 2]], dtype=np.int32)
    counts, offsets, row_of, token_of = permute.permute(idx, 3, False)
    assert counts.tolist() == [2, 1, 1]
    assert offsets.tolist() == [0, 2, 3, 4, 4]
    assert row_of.tolist() == [[2, 0], [1, 3]]
    assert token_of.tolist() == [0, 1, 0, 1]


def test_empty_experts_and_empty_batch():
    idx = np.array([[3, 3 - 1]], dtype=np.int32)
    counts, offsets, _, _ = permute.permute(idx, 6, True)
    assert counts.tolist() == [0, 0, 1, 1, 0, 0]
    c, o, r, t = permute.permute(np.zeros((0, 2), np.int32), 4, True)
    assert c.sum() == 0 and o.tolist() == [0] * 6 and r.shape == (0, 2) and t.size == 0
