"""Pins of the oracle's router, biased top-k and gates.

Source: "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token
Prediction, and FP8 Training at 671B Scale", section III: the affinity
equation s = Sigmoid(u . e), the selection equation (s + b in TopK), the gate
normalisation g = g' / sum g' and the bullet "the bias only enters the TopK
comparison"; "DeepSeek-V3, explained.", glossary (normalised weights sum to 1,
bias decides which experts are chosen and never how much they count).
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

from oracle import route


def _f32(v):
    return np.asarray(v, np.float64).astype(np.float32)


def test_sigmoid_closed_forms_and_library():
    assert route.sigmoid(np.array([0.0]))[0] == 0.5
    assert abs(route.sigmoid(np.array([np.log(3.0)]))[0] - 0.75) < 1e-15
    z = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(route.sigmoid(z) + route.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(route.sigmoid(z), expit(z), rtol=1e-14, atol=0)
    assert np.all(np.isfinite(route.sigmoid(np.array([-800.0, 800.0]))))


def test_router_logits_closed_form():
    T, H, N = 3, 256, 5
    x = np.ones((T, H)) * np.array([1.0, 2.0, -0.5])[:, None]
    w = np.arange(N)[:, None] / 256.0 * np.ones((N, H))
    z = route.router_logits(x, w)
    np.testing.assert_array_equal(z, np.array([1.0, 2.0, -0.5])[:, None] * np.arange(N)[None, :] * H / 256.0)
    # one-hot tokens pick out columns of W_r: z[t, i] = W_r[i, t]
    rng = np.random.default_rng(0)
    w = rng.standard_normal((N, H))
    np.testing.assert_array_equal(route.router_logits(np.eye(H)[:T], w), w[:, :T].T)


def _brute_topk(key, k):
    """The unique k-set S with: every member's key exceeds every non-member's,
    ties resolved to the lower index; listed by (key desc, index asc)."""
    n = key.size
    found = []
    for S in itertools.combinations(range(n), k):
        rest = [j for j in range(n) if j not in S]
        ok = all(key[i] > key[j] or (key[i] == key[j] and i < j) for i in S for j in rest)
        if ok:
            found.append(S)
    assert len(found) == 1
    S = list(found[0])
    S.sort(key=lambda i: (-key[i], i))
    return S


@pytest.mark.parametrize("n,k", [(6, 2), (8, 3), (7, 7), (9, 1)])
def test_topk_matches_brute_force(n, k):
    rng = np.random.default_rng(n * 10 + k)
    for trial in range(40):
        s = _f32(rng.uniform(0, 1, (1, n)))
        b = _f32(rng.uniform(-0.1, 0.1, n))
        if trial % 3 == 0:                                  # force ties
            s = _f32(np.round(s * 4) / 4)
            b = np.zeros(n, np.float32)
        idx = route.select_topk(s, b, k)[0]
        key = route.biased_keys(s, b)[0]
        assert list(idx) == _brute_topk(key, k)


def test_k_equals_n_is_plain_normalisation():
    rng = np.random.default_rng(7)
    s = _f32(rng.uniform(0.01, 1, (5, 6)))
    b = _f32(rng.uniform(-1, 1, 6))
    idx = route.select_topk(s, b, 6)
    assert all(sorted(r) == list(range(6)) for r in idx)
    g = route.gates(s, idx)
    full = s.astype(np.float64) / s.astype(np.float64).sum(1, keepdims=True)
    np.testing.assert_allclose(np.take_along_axis(full, idx.astype(np.int64), 1), g, rtol=1e-15)


def test_zero_bias_is_textbook_topk_of_sigmoid():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((50, 128))
    w = rng.standard_normal((16, 128)) * 0.1
    s64, s32, idx, g = route.route(x, w, np.zeros(16, np.float32), 4)
    ref = np.argsort(-s32.astype(np.float64), axis=1, kind="stable")[:, :4]
    assert np.array_equal(idx, ref)


def test_large_bias_forces_selection_but_not_the_gate():
    rng = np.random.default_rng(9)
    s = _f32(rng.uniform(0, 1, (100, 16)))
    b = np.zeros(16, np.float32)
    b[3] = 10.0
    idx = route.select_topk(s, b, 2)
    assert np.all(idx[:, 0] == 3)
    g = route.gates(s, idx)
    want = s[:, 3].astype(np.float64) / (s[:, 3].astype(np.float64)
                                         + np.take_along_axis(s, idx[:, 1:2].astype(np.int64), 1)[:, 0])
    np.testing.assert_array_equal(g[:, 0], want)


def test_gates_are_invariant_to_bias_that_keeps_the_selection():
    rng = np.random.default_rng(10)
    s = _f32(rng.uniform(0, 1, (200, 16)))
    b1 = _f32(rng.uniform(-0.05, 0.05, 16))
    b2 = _f32(b1 + rng.uniform(-1e-3, 1e-3, 16))
    i1, i2 = route.select_topk(s, b1, 4), route.select_topk(s, b2, 4)
    same = np.all(np.sort(i1, 1) == np.sort(i2, 1), axis=1)
    assert same.sum() > 150
    g1 = route.gates(s, np.sort(i1, 1))
    g2 = route.gates(s, np.sort(i2, 1))
    assert np.array_equal(g1[same], g2[same])


def test_gates_sum_to_one_and_are_positive():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 64))
    w = rng.standard_normal((32, 64)) * 0.2
    _, s32, idx, g = route.route(x, w, _f32(rng.uniform(-0.1, 0.1, 32)), 8)
    assert np.all(g > 0)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(route.biased_keys(s32, _f32(np.zeros(32)))[0]) != np.inf)


def test_order_is_key_descending():
    rng = np.random.default_rng(12)
    s = _f32(rng.uniform(0, 1, (100, 32)))
    b = _f32(rng.uniform(-0.05, 0.05, 32))
    idx = route.select_topk(s, b, 8)
    key = np.take_along_axis(route.biased_keys(s, b), idx.astype(np.int64), 1)
    assert np.all(np.diff(key.astype(np.float64), axis=1) <= 0)


def test_margin():
    s = np.array([[0.9, 0.5, 0.4, 0.1]])
    b = np.array([0.0, 0.0, 0.05, 0.0])
    assert abs(route.topk_margin(s, b, 2)[0] - (0.5 - 0.45)) < 1e-15
    assert route.topk_margin(s, b, 4)[0] == np.inf


# ---------------------------------------------------------------- group-limited selection
# Sources: "DeepSeek-V3, explained.", recipe step 5 (nodes ranked by the sum of
# the highest affinities they hold, the 8 experts taken from the top 4 nodes);
# "DeepSeek-V3 Technical Report" (deepforge), "Balancing without a balance
# loss" (at most 4 nodes, chosen by the sum of each node's top K_r / M scores).


def _brute_grouped(key, k, G, M):
    """Enumerate every set of M groups, keep the sets whose minimum group score
    beats (or ties with a lower index) every excluded group, and take the top k
    keys inside the winning set -- written independently of the oracle."""
    N = key.size
    gs = N // G
    r = k // M
    scores = []
    for g in range(G):
        top = sorted(key[g * gs:(g + 1) * gs].tolist(), reverse=True)[:r]
        acc = np.float32(top[0])
        for v in top[1:]:
            acc = np.float32(acc + np.float32(v))
        scores.append(acc)
    best = None
    for groups in itertools.combinations(range(G), M):
        ok = all((scores[a] > scores[b]) or (scores[a] == scores[b] and a < b)
                 for a in groups for b in range(G) if b not in groups)
        if ok:
            assert best is None
            best = groups
    cand = [e for e in range(N) if e // gs in best]
    cand.sort(key=lambda e: (-float(key[e]), e))
    return cand[:k]


@pytest.mark.parametrize("N,G,M,k", [(16, 4, 2, 4), (16, 8, 4, 8), (24, 6, 3, 3), (32, 8, 4, 8)])
def test_grouped_topk_matches_brute_force(N, G, M, k):
    rng = np.random.default_rng(N * 100 + G * 10 + M)
    s = rng.uniform(0, 1, (60, N)).astype(np.float32)
    b = rng.uniform(-0.2, 0.2, N).astype(np.float32)
    s[::7] = np.round(s[::7] * 4) / 4          # plenty of exact ties
    idx = route.select_topk_grouped(s, b, k, G, M)
    key = route.biased_keys(s, b)
    for t in range(s.shape[0]):
        assert idx[t].tolist() == _brute_grouped(key[t], k, G, M), t


def test_grouped_topk_reduces_to_plain_topk():
    rng = np.random.default_rng(8)
    s = rng.uniform(0, 1, (50, 64)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, 64).astype(np.float32)
    plain = route.select_topk(s, b, 8)
    assert np.array_equal(route.select_topk_grouped(s, b, 8, 8, 8), plain)   # every group
    assert np.array_equal(route.select_topk_grouped(s, b, 8, 1, 1), plain)   # one group


def test_grouped_topk_limits_the_groups_and_keeps_gates_unbiased():
    """A token whose plain top-8 spans 8 groups gets 8 experts from 4 groups;
    the chosen experts are the top keys of the chosen groups; the gates are
    the unbiased scores normalised, whatever the bias."""
    N, G, M, k = 256, 8, 4, 8
    s = np.full((1, N), 0.1, np.float32)
    # group g holds one strong expert 32 g (score 0.9 - 0.01 g) and, for even
    # g, a second one of 0.5: even groups score higher by their second key
    for g in range(G):
        s[0, 32 * g] = 0.9 - 0.01 * g
        if g % 2 == 0:
            s[0, 32 * g + 1] = 0.5
    b = np.zeros(N, np.float32)
    plain = route.select_topk(s, b, k)[0]
    assert len({e // 32 for e in plain}) == 8
    idx = route.select_topk_grouped(s, b, k, G, M)[0]
    assert {e // 32 for e in idx} == {0, 2, 4, 6}
    assert idx.tolist() == [0, 64, 128, 192, 1, 65, 129, 193]
    # a bias that only reorders inside the chosen set leaves the gates alone
    b2 = b.copy()
    b2[[0, 64, 128, 192, 1, 65, 129, 193]] += 0.001
    idx2 = route.select_topk_grouped(s, b2, k, G, M)
    g1 = route.gates(s, idx[None, :])
    g2 = route.gates(s, idx2)
    assert sorted(idx2[0].tolist()) == sorted(idx.tolist())
    np.testing.assert_allclose(np.sort(g1[0]), np.sort(g2[0]), rtol=0, atol=0)
    # a large bias on a weak group's expert pulls that group in (selection
    # uses the biased keys, group ranking included)
    b3 = b.copy()
    b3[32 * 7 + 5] = 2.0
    idx3 = route.select_topk_grouped(s, b3, k, G, M)[0]
    assert 32 * 7 + 5 in idx3 and 7 in {e // 32 for e in idx3}


# --------------------------------------------------------------------------- opt-in FP8 router
# "DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction,
# and FP8 Training at 671B Scale", section V, FP8 details 1-2 (1x128 activation
# tiles, 128x128 weight blocks) applied to the router's product.

from oracle import e4m3  # noqa: E402


def _e4m3_tiles(rng, rows, cols, exps, block_rows):
    """Values that E4M3 holds exactly once divided by their block's power of
    two: random finite codes, one +448 per block (so amax = 448 * 2^p and the
    quantiser's scale is exactly 2^p), block (r // block_rows, c // 128)
    scaled by 2^exps[r // block_rows, c // 128]."""
    codes = rng.integers(0, 256, (rows, cols)).astype(np.uint8)
    codes = np.where((codes & 0x7F) == 0x7F, codes & 0xF0, codes).astype(np.uint8)
    v = e4m3.decode(codes)
    for rb in range(rows // block_rows):
        for cb in range(cols // 128):
            v[rb * block_rows, cb * 128] = 448.0
    scale = np.repeat(np.repeat(2.0 ** np.asarray(exps, np.float64), block_rows, 0), 128, 1)
    return v * scale


def test_fp8_router_is_exact_on_e4m3_operands():
    """Operands that the quantisers reproduce exactly: the FP8 logits equal the
    plain float64 product, and the routing equals the bf16-free oracle's."""
    rng = np.random.default_rng(21)
    T, H, N, k = 40, 512, 256, 8
    x = _e4m3_tiles(rng, T, H, rng.integers(-9, -3, (T, H // 128)), 1)
    w = _e4m3_tiles(rng, N, H, np.array([[-14, -13, -12, -11], [-12, -15, -11, -13]]), 128)
    b = rng.uniform(-0.05, 0.05, N).astype(np.float32)
    s64f, s32f, idxf, gatef, (xq, xd, wq, wd) = route.route_fp8(x, w, b, k)
    np.testing.assert_array_equal(e4m3.decode(xq) * np.repeat(xd.astype(np.float64), 128, 1), x)
    z = route.router_logits(x, w)
    zf = route.router_logits_fp8(xq, xd, wq, wd)
    scale = np.abs(x) @ np.abs(w).T
    assert np.max(np.abs(zf - z) / scale) < 1e-13
    s64, s32, idx, gate = route.route(x, w, b, k)
    clear = route.topk_margin(s64, b, k) > 1e-9
    assert clear.mean() > 0.99
    assert np.array_equal(idxf[clear], idx[clear])


def test_fp8_router_dequantised_dot_brute_force():
    """The block-scaled sum equals the dot product of the dequantised operands,
    written out element by element (tiny case, two weight block rows)."""
    rng = np.random.default_rng(22)
    T, H, N = 2, 256, 256
    x = rng.standard_normal((T, H)) * np.repeat([[1.0, 30.0]], T, 0).repeat(128, 1)
    w = rng.standard_normal((N, H)) * 0.02
    w[128:] *= 7.0
    _, _, _, _, (xq, xd, wq, wd) = route.route_fp8(x, w, np.zeros(N, np.float32), 2)
    zf = route.router_logits_fp8(xq, xd, wq, wd)
    xv, wv = e4m3.decode(xq), e4m3.decode(wq)
    for t in range(T):
        for i in range(0, N, 37):
            acc = 0.0
            for h in range(H):
                acc += (xv[t, h] * float(xd[t, h // 128])) * (wv[i, h] * float(wd[i // 128, h // 128]))
            assert abs(zf[t, i] - acc) <= 1e-12 * (abs(acc) + 1.0)


def test_fp8_router_within_the_e4m3_error_bound():
    """Random operands with tile- and block-dependent magnitudes: the FP8
    logits differ from the exact product by no more than the E4M3 rounding
    allows (relative 2^-4 on normal codes, 2^-10 of the scale below them),
    with the scales computed here from each block's amax."""
    rng = np.random.default_rng(23)
    T, H, N = 64, 768, 256
    x = rng.standard_normal((T, H)) * np.exp2(rng.integers(-6, 6, (T, H // 128))).repeat(128, 1)
    x[:, 5] *= 100.0                                    # an outlier channel
    wexp = rng.integers(-9, -3, (N // 128, H // 128))
    w = rng.standard_normal((N, H)) * np.exp2(wexp).repeat(128, 0).repeat(128, 1)
    _, _, _, _, (xq, xd, wq, wd) = route.route_fp8(x, w, np.zeros(N, np.float32), 8)
    zf = route.router_logits_fp8(xq, xd, wq, wd)
    z = route.router_logits(x, w)
    dx = np.abs(x).reshape(T, H // 128, 128).max(2) / 448.0
    dw = np.abs(w).reshape(N // 128, 128, H // 128, 128).max((1, 3)) / 448.0
    ex = np.abs(x) * (2.0 ** -4 + 2.0 ** -20) + dx.repeat(128, 1) * 2.0 ** -10 * (1 + 1e-6)
    ew = np.abs(w) * (2.0 ** -4 + 2.0 ** -20) + dw.repeat(128, 0).repeat(128, 1) * 2.0 ** -10 * (1 + 1e-6)
    bound = ex @ np.abs(w).T + (np.abs(x) + ex) @ ew.T
    ratio = np.abs(zf - z) / bound
    assert np.max(ratio) <= 1.0
    assert np.max(ratio) > 1e-3          # the error is real: the check is not vacuous
