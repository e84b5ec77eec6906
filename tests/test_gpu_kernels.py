"""GPU parity of each C entry point against the CPU oracle, on the same seeded
inputs.  Integer results (codes, indices, maps, counts, bias) must match bit
for bit; float results within the stated tolerances."""
import numpy as np
import pytest

import synth
from helpers import (bf16_from_dev, bf16_to_dev, bf16_values, check_h, codes_agree_up_to_ties, flip_cap, swiglu_band,
                     device_tensor, log, rel_l2, to_dev)
from oracle import balance as obalance
from oracle import bias as obias
from oracle import e4m3, ffn, permute as opermute, quant, route

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a device"
    import fp8_block_scaled_sigmoid_amd as moe
    moe.lib()
    return moe


def _moe():
    import fp8_block_scaled_sigmoid_amd as moe
    return moe


# --------------------------------------------------------------------------- generator


@pytest.mark.parametrize("name", ["tiny", "prefill", "skew"])
def test_device_generator_matches_host(name):
    w = synth.WORKLOADS[name]
    rows = np.array([0, 1, 7, w.T - 1])
    log(f"synth x {name}")
    x = device_tensor(w.x_spec(), w.seed)
    got = bf16_from_dev(x)[rows]
    assert np.array_equal(got, synth.generate(w.x_spec(), w.seed, rows=rows))
    spec = w.wr_spec()
    t = device_tensor(spec, w.seed)
    assert np.array_equal(bf16_from_dev(t), synth.generate(spec, w.seed))
    bspec = synth.Spec(synth.T_BIAS, (w.N,), synth.UNIFORM, 0.05, dtype="f32")
    tb = device_tensor(bspec, w.seed, dtype="f32")
    assert np.array_equal(tb.cpu().numpy(), synth.generate(bspec, w.seed))


# --------------------------------------------------------------------------- quantisers


def _adversarial_rows(H):
    """Rows exercising the zero-tile, overflow, sign-of-zero and subnormal rules."""
    rows = np.zeros((6, H), np.float32)
    rows[1, :] = -0.0
    rows[2, :128] = np.float32(1e-37)               # fl32(448 / amax) overflows
    rows[3, :128] = np.linspace(-3e-38, 3e-38, 128)  # tiny, with float32 subnormals
    rows[3, 5] = np.float32(2e-36)
    rows[4, :] = np.where(np.arange(H) % 2, 448.0, -448.0)
    rows[5, :] = np.linspace(-1, 1, H)
    rows[5, 17] = 1e4                                # outlier in tile 0
    return rows


@pytest.mark.parametrize("name,rows", [("tiny", None), ("decode", None), ("prefill", 37)])
def test_quant_1x128_bf16_bit_exact(name, rows):
    moe = _moe()
    w = synth.WORKLOADS[name]
    r = np.arange(w.T if rows is None else rows)
    bits = synth.generate(w.x_spec(), w.seed, rows=r)
    adv = synth.f32_to_bf16_bits(_adversarial_rows(w.H))
    bits = np.concatenate([bits, adv])
    log(f"fp8_quant_1x128 bf16 {name} rows={bits.shape[0]}")
    q, d = moe.fp8_quant_1x128(bf16_to_dev(bits))
    torch.cuda.synchronize()
    wq, wd = quant.quant_1x128(synth.as_f64(bits))
    assert np.array_equal(q.cpu().numpy(), wq)
    assert np.array_equal(d.cpu().numpy(), wd)


def test_quant_1x128_f32_encoder_sweep():
    """Tiles whose amax is 448 have m = d = 1, so every other element's code is
    the E4M3 encoding of that very float: sweep float32 values up to 448 plus
    every rounding tie and its neighbours, both signs."""
    moe = _moe()
    bits = np.arange(0, 0x43E00000, 97, dtype=np.uint64).astype(np.uint32)
    sweep = bits.view(np.float32)
    pos = e4m3.POS_VALUES
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    near = [mids]
    for dirn in (np.inf, -np.inf):
        cur = mids
        for _ in range(2):
            cur = np.nextafter(cur, np.float32(dirn))
            near.append(cur)
    vals = np.concatenate([sweep] + near)
    vals = np.concatenate([vals, -vals])
    vals = vals[np.abs(vals) <= 448.0]
    per = 127
    n_t = (vals.size + per - 1) // per
    pad = np.zeros(n_t * per, np.float32)
    pad[:vals.size] = vals
    tiles = np.concatenate([np.full((n_t, 1), 448.0, np.float32), pad.reshape(n_t, per)], 1)
    x = tiles.reshape(-1, 1024) if tiles.size % 1024 == 0 else np.concatenate(
        [tiles.reshape(-1), np.full((-tiles.size) % 1024, 448.0, np.float32)]).reshape(-1, 1024)
    log(f"fp8_quant_1x128 f32 encoder sweep values={vals.size}")
    q, d = moe.fp8_quant_1x128(to_dev(x))
    torch.cuda.synchronize()
    assert np.all(d.cpu().numpy() == 1.0)
    assert np.array_equal(q.cpu().numpy(), e4m3.encode(x.astype(np.float64)))


def _encode_positive_chunk(lo_hi):
    lo, hi = lo_hi
    pos = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return e4m3.encode_arith(pos.astype(np.float64)).astype(np.uint8)


def test_quant_1x128_f32_every_float32_up_to_448():
    """The hardware E4M3 conversion against the oracle on every float32 of
    magnitude at most 448 (1.14 G patterns per sign, both signs, -0
    included): tiles whose maximum is 448 have m = d = 1, so each code is the
    encoding of that very float.  Negative codes are the positive ones with
    the sign bit, as the format defines them.  The oracle's codes are computed
    on host threads ahead of the device chunks; about half a minute."""
    from concurrent.futures import ThreadPoolExecutor
    moe = _moe()
    top = 0x43E00000 + 1                      # bit patterns 0 .. 448.0
    step = 1 << 24
    per = 127
    bad = 0
    ranges = [(lo, min(lo + step, top)) for lo in range(0, top, step)]
    log(f"fp8_quant_1x128 f32 every float32 up to 448: {len(ranges)} chunks")
    with ThreadPoolExecutor(max_workers=8) as ex:
        for n, ((lo, hi), want_pos) in enumerate(zip(ranges, ex.map(_encode_positive_chunk, ranges))):
            pos = np.arange(lo, hi, dtype=np.uint64).astype(np.uint32).view(np.float32)
            vals = np.concatenate([pos, -pos])
            want = np.concatenate([want_pos, want_pos | np.uint8(0x80)])
            n_t = (vals.size + per - 1) // per
            pad = np.full(n_t * per, 448.0, np.float32)
            pad[:vals.size] = vals
            tiles = np.concatenate([np.full((n_t, 1), 448.0, np.float32), pad.reshape(n_t, per)], 1)
            q, d = moe.fp8_quant_1x128(to_dev(tiles))
            got = q.cpu().numpy()[:, 1:].reshape(-1)[:vals.size]
            torch.cuda.synchronize()
            assert np.all(d.cpu().numpy() == 1.0)
            bad += int(np.count_nonzero(got != want))
            if n % 8 == 0:
                print(f"chunk {n}: patterns {lo:#010x}..{hi - 1:#010x}, mismatches so far {bad}",
                      flush=True)
    assert bad == 0


def test_quant_1x128_f32_random_tiles():
    moe = _moe()
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((300, 512)) * np.exp(rng.uniform(-20, 20, (300, 1)))).astype(np.float32)
    log("fp8_quant_1x128 f32 random")
    q, d = moe.fp8_quant_1x128(to_dev(x))
    torch.cuda.synchronize()
    wq, wd = quant.quant_1x128(x.astype(np.float64))
    assert np.array_equal(q.cpu().numpy(), wq) and np.array_equal(d.cpu().numpy(), wd)


@pytest.mark.parametrize("tiles", [1, 3, 4, 5, 7, 9])
def test_quant_1x128_runs_and_row_stride(tiles):
    """Rows of 1-9 tiles (the quantiser takes runs of four tiles of a row, so
    every remainder of a run occurs) read from a wider tensor (row stride
    larger than the row), 37 rows."""
    moe = _moe()
    rng = np.random.default_rng(40 + tiles)
    cols = 128 * tiles
    full = (rng.standard_normal((37, cols + 136)) *
            np.exp(rng.uniform(-8, 8, (37, 1)))).astype(np.float32)
    full[5, :] = 0.0                                       # zero tiles
    full[9, 128 * (tiles - 1) + 3] = 3e4                   # outlier in the last tile
    bits = synth.f32_to_bf16_bits(full)
    x = bf16_to_dev(bits)[:, 8:8 + cols]                   # stride cols + 136, offset 16 bytes
    log(f"fp8_quant_1x128 bf16 tiles={tiles} ld={x.stride(0)}")
    q, d = moe.fp8_quant_1x128(x)
    torch.cuda.synchronize()
    wq, wd = quant.quant_1x128(synth.as_f64(bits[:, 8:8 + cols]))
    assert np.array_equal(q.cpu().numpy(), wq)
    assert np.array_equal(d.cpu().numpy(), wd)


@pytest.mark.parametrize("interleave", [False, True])
def test_quant_128x128_bit_exact(interleave):
    moe = _moe()
    w = synth.WORKLOADS["tiny"]
    bits = synth.generate(w.w1_spec(), w.seed)          # [17, 256, 256]
    bits[3, 130, 200] = synth.f32_to_bf16_bits(np.array([7.0], np.float32))[0]   # outlier block
    bits[4, :128, :128] = 0                                                       # zero block
    log(f"fp8_quant_128x128 interleave={interleave}")
    q, d = moe.fp8_quant_128x128(bf16_to_dev(bits), interleave_gate_up=interleave)
    torch.cuda.synchronize()
    wq, wd = quant.quant_128x128(synth.as_f64(bits))
    if interleave:                    # row blocks (gate j, up j) -> (2j, 2j+1)
        nb = bits.shape[1] // 128
        order = np.array([j // 2 if j % 2 == 0 else nb // 2 + j // 2 for j in range(nb)])
        wq = wq.reshape(w.G, nb, 128, -1)[:, order].reshape(wq.shape)
        wd = wd[:, order]
    assert np.array_equal(q.cpu().numpy(), wq) and np.array_equal(d.cpu().numpy(), wd)


# --------------------------------------------------------------------------- routing


@pytest.mark.parametrize("T,N,k,ties", [(1000, 16, 2, False), (777, 256, 8, False),
                                        (500, 256, 8, True), (64, 1000, 32, False),
                                        (300, 32, 32, False), (129, 48, 1, True),
                                        (200, 1024, 32, True)])   # the largest N and k
def test_topk_from_scores_bit_exact(T, N, k, ties):
    moe = _moe()
    rng = np.random.default_rng(T + N + k)
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, N).astype(np.float32)
    if ties:
        s = (np.round(s * 8) / 8).astype(np.float32)
        b[:] = 0
    log(f"moe_topk_from_scores T={T} N={N} k={k}")
    idx, gate = moe.moe_topk_from_scores(to_dev(s), to_dev(b), k)
    torch.cuda.synchronize()
    want = route.select_topk(s, b, k)
    assert np.array_equal(idx.cpu().numpy(), want)
    g = route.gates(s, want)
    np.testing.assert_allclose(gate.cpu().numpy(), g, rtol=2e-6, atol=1e-7)


def _route_check(x_bits, wr_bits, b, k, s_gpu, idx_gpu, gate_gpu, delta=3e-5):
    """Indices bit-exact to the selection rule on the GPU's own scores (every
    token); scores within 1e-5 of the float64 oracle; indices bit-exact on every
    token whose k-th/(k+1)-th key gap exceeds delta (three times the score
    tolerance), a valid top-k of the float64 keys on the others."""
    # same-score check: on every token the selection is bit-exact to the
    # oracle's selection rule applied to the GPU's own float32 scores
    assert np.array_equal(idx_gpu, route.select_topk(s_gpu, b, k))
    np.testing.assert_allclose(gate_gpu, route.gates(s_gpu, idx_gpu), rtol=2e-6, atol=1e-7)
    s64 = route.router_scores(synth.as_f64(x_bits), synth.as_f64(wr_bits))
    err = np.max(np.abs(s_gpu - s64))
    print(f"max |score - oracle| = {err:.3e}")
    assert err < 1e-5
    margin = route.topk_margin(s64, b, k)
    idx_o = route.select_topk(s64.astype(np.float32), b, k)
    clear = margin > delta
    assert clear.mean() > 0.97
    assert np.array_equal(idx_gpu[clear], idx_o[clear])
    # low-margin tokens: the GPU's set is still a valid top-k of the float64 keys
    key = s64 + b.astype(np.float64)[None, :]
    for t in np.nonzero(~clear)[0]:
        kth = -np.sort(-key[t])[k - 1]
        assert np.all(key[t, idx_gpu[t]] >= kth - 2 * delta)
    g = route.gates(s64.astype(np.float32), idx_gpu)
    np.testing.assert_allclose(gate_gpu, g, rtol=1e-5, atol=1e-6)
    return int((~clear).sum())


@pytest.mark.parametrize("name,T", [("tiny", None), ("routing", 2048), ("prefill", 1000),
                                    ("skew", 512)])
def test_route_topk(name, T):
    moe = _moe()
    w = synth.WORKLOADS[name]
    T = w.T if T is None else T
    xb = synth.generate(w.x_spec(), w.seed, rows=np.arange(T))
    wrb = w.router_weight()
    b = w.bias()
    log(f"moe_route_topk {name} T={T}")
    idx, gate, s = moe.moe_route_topk(bf16_to_dev(xb), bf16_to_dev(wrb), to_dev(b), w.k)
    torch.cuda.synchronize()
    _route_check(xb, wrb, b, w.k, s.cpu().numpy(), idx.cpu().numpy(), gate.cpu().numpy())
    # scores buffer is optional
    idx2, gate2, _ = moe.moe_route_topk(bf16_to_dev(xb), bf16_to_dev(wrb), to_dev(b), w.k,
                                        scores=False)
    assert torch.equal(idx, idx2) and torch.equal(gate, gate2)


def test_route_topk_ragged_small():
    """T not a multiple of the 128-token tile, N = k (all chosen), N = 16, N
    not a multiple of 64 (partly empty expert bands), H of one 128 block."""
    moe = _moe()
    rng = np.random.default_rng(5)
    for T, H, N, k in [(33, 128, 16, 16), (70, 384, 32, 3), (1, 256, 16, 1), (129, 640, 80, 6),
                       (300, 1024, 208, 8)]:
        x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        wr = synth.f32_to_bf16_bits((rng.standard_normal((N, H)) * 0.05).astype(np.float32))
        b = rng.uniform(-0.1, 0.1, N).astype(np.float32)
        log(f"moe_route_topk ragged T={T} H={H} N={N} k={k}")
        idx, gate, s = moe.moe_route_topk(bf16_to_dev(x), bf16_to_dev(wr), to_dev(b), k)
        torch.cuda.synchronize()
        _route_check(x, wr, b, k, s.cpu().numpy(), idx.cpu().numpy(), gate.cpu().numpy())


@pytest.mark.parametrize("case", ["tiny", "decode", "prefill-1000", "ragged", "ragged-h128",
                                  "ragged-h640", "skew-300"])
def test_route_topk_quant_x(case):
    """The router that also quantises x: its codes and scales equal the
    oracle's 1x128 quantisation bit for bit (adversarial rows appended:
    zero tiles, -0, overflowing 448 / amax, subnormals, an outlier), and its
    routing equals moe_route_topk's bit for bit (same kernel arithmetic).
    Shapes span 1-56 blocks of H per row, slices of one to several blocks,
    token tiles with a ragged last tile, and 16-256 experts."""
    moe = _moe()
    rng = np.random.default_rng(11)
    if case.startswith("ragged"):
        T, H, N, k = {"ragged": (133, 384, 32, 3), "ragged-h128": (33, 128, 16, 16),
                      "ragged-h640": (129, 640, 80, 6)}[case]
        xb = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        wrb = synth.f32_to_bf16_bits((rng.standard_normal((N, H)) * 0.05).astype(np.float32))
        b = rng.uniform(-0.1, 0.1, N).astype(np.float32)
    else:
        name, _, rows = case.partition("-")
        w = synth.WORKLOADS[name]
        T = int(rows) if rows else w.T
        xb = synth.generate(w.x_spec(), w.seed, rows=np.arange(T))
        wrb, b, k, H = w.router_weight(), w.bias(), w.k, w.H
    xb = np.concatenate([xb, synth.f32_to_bf16_bits(_adversarial_rows(H))])
    log(f"moe_route_topk_quant_x {case} T={xb.shape[0]} H={H} N={wrb.shape[0]}")
    x, wr, bd = bf16_to_dev(xb), bf16_to_dev(wrb), to_dev(b)
    idx, gate, s, q, d = moe.moe_route_topk_quant_x(x, wr, bd, k)
    idx0, gate0, s0 = moe.moe_route_topk(x, wr, bd, k)
    torch.cuda.synchronize()
    wq, wd = quant.quant_1x128(synth.as_f64(xb))
    assert np.array_equal(q.cpu().numpy(), wq)
    assert np.array_equal(d.cpu().numpy(), wd)
    assert torch.equal(idx, idx0) and torch.equal(gate, gate0) and torch.equal(s, s0)


def test_route_topk_quant_x_full_prefill():
    """At the prefill batch's full size (T = 8192, H 7168, 256 experts), in
    the layer's launch configuration: codes and scales equal
    fp8_quant_1x128's bit for bit on every token, and the oracle's on a
    sample of 256 tokens; routing equals moe_route_topk's."""
    moe = _moe()
    w = synth.WORKLOADS["prefill"]
    x = device_tensor(w.x_spec(), w.seed)
    wr, bd = bf16_to_dev(w.router_weight()), to_dev(w.bias())
    log(f"moe_route_topk_quant_x prefill T={w.T}")
    idx, gate, s, q, d = moe.moe_route_topk_quant_x(x, wr, bd, w.k)
    q1, d1 = moe.fp8_quant_1x128(x)
    idx0, gate0, s0 = moe.moe_route_topk(x, wr, bd, w.k)
    torch.cuda.synchronize()
    assert torch.equal(q, q1) and torch.equal(d, d1)
    assert torch.equal(idx, idx0) and torch.equal(gate, gate0) and torch.equal(s, s0)
    rows = np.unique(np.concatenate([[0, w.T - 1], np.random.default_rng(3).integers(0, w.T, 254)]))
    xb = synth.generate(w.x_spec(), w.seed, rows=rows)
    wq, wd = quant.quant_1x128(synth.as_f64(xb))
    assert np.array_equal(q.cpu().numpy()[rows], wq)
    assert np.array_equal(d.cpu().numpy()[rows], wd)


def test_route_topk_full_routing_workload_sampled():
    """The routing workload at its full size (T = 16384, H 7168, 256 experts,
    top-8), in the launch configuration the layer uses; the oracle recomputes
    a seeded sample of 384 tokens (first, last and random rows)."""
    moe = _moe()
    w = synth.WORKLOADS["routing"]
    x = device_tensor(w.x_spec(), w.seed)
    wrb = w.router_weight()
    b = w.bias()
    log(f"moe_route_topk routing full T={w.T}")
    idx, gate, s = moe.moe_route_topk(x, bf16_to_dev(wrb), to_dev(b), w.k)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, w.T - 1], rng.choice(w.T, 381, replace=False)]))
    xb = synth.generate(w.x_spec(), w.seed, rows=rows)
    _route_check(xb, wrb, b, w.k, s.cpu().numpy()[rows], idx.cpu().numpy()[rows],
                 gate.cpu().numpy()[rows])


# --------------------------------------------------------------------------- FP8 router


FP8_ROUTER_REL = 1e-4   # |logit - exact block-scaled sum| / sum|q_x q_W d_x d_W|, as for the GEMM


def _route_fp8_check(xb, wrb, b, k, xq, xd, wq, wd, s_gpu, idx_gpu, gate_gpu, idx_bf16,
                     G=1, M=1):
    """The opt-in FP8 router against the oracle's FP8 router: operand codes
    and scales bit-exact to the oracle's quantisers; selection bit-exact to
    the rule on the GPU's own scores; scores within the MFMA band of the
    float64 block-scaled product; index sets equal to the oracle's wherever
    the key gap exceeds twice that band.  Returns the fraction of tokens
    routed to the same set as the bf16 router."""
    xq_o, xd_o = quant.quant_1x128(synth.as_f64(xb))
    wq_o, wd_o = quant.quant_128x128(synth.as_f64(wrb))
    assert np.array_equal(xq, xq_o) and np.array_equal(xd, xd_o)
    assert np.array_equal(wq, wq_o) and np.array_equal(wd, wd_o)
    assert np.array_equal(idx_gpu, route.select_topk_grouped(s_gpu, b, k, G, M))
    np.testing.assert_allclose(gate_gpu, route.gates(s_gpu, idx_gpu), rtol=2e-6, atol=1e-7)
    s64 = route.sigmoid(route.router_logits_fp8(xq_o, xd_o, wq_o, wd_o))
    mag = route.router_logits_fp8(xq_o & 0x7F, xd_o, wq_o & 0x7F, wd_o)
    tol = 0.25 * FP8_ROUTER_REL * mag + 2e-7          # sigmoid' <= 1/4, plus float32 rounding
    err = np.abs(s_gpu - s64)
    print(f"max |score - oracle| = {err.max():.3e} (bound {tol.max():.3e}, "
          f"max ratio {np.max(err / tol):.3f})")
    assert np.all(err <= tol)
    if G <= 1:
        margin = route.topk_margin(s64, b, k)
        clear = margin > 2 * (tol.max(axis=1) + 1e-7)
        want = route.select_topk(s64.astype(np.float32), b, k)
        print(f"tokens with a clear margin: {clear.mean():.3f}")
        assert np.array_equal(np.sort(idx_gpu[clear], 1), np.sort(want[clear], 1))
    agree = float(np.mean(np.all(np.sort(idx_gpu, 1) == np.sort(idx_bf16, 1), axis=1)))
    print(f"agreement with the bf16 router (same expert set): {agree:.4f}")
    return agree


def _run_route_fp8(moe, x_dev, wr_dev, b, k, G=1, M=1):
    xq, xd = moe.fp8_quant_1x128(x_dev)
    wq, wd = moe.fp8_quant_128x128(wr_dev)
    idx, gate, s = moe.moe_route_topk_fp8(xq, xd, wq[0], wd[0], to_dev(b), k, n_groups=G,
                                          topk_groups=M)
    idx_b, _, _ = moe.moe_route_topk(x_dev, wr_dev, to_dev(b), k, scores=False, n_groups=G,
                                     topk_groups=M)
    torch.cuda.synchronize()
    return (xq.cpu().numpy(), xd.cpu().numpy(), wq[0].cpu().numpy(), wd[0].cpu().numpy(),
            s.cpu().numpy(), idx.cpu().numpy(), gate.cpu().numpy(), idx_b.cpu().numpy())


@pytest.mark.parametrize("name,T,G,M", [("routing", 2048, 1, 1), ("prefill", 1000, 1, 1),
                                        ("skew", 512, 1, 1), ("routing", 777, 8, 4)])
def test_route_topk_fp8(name, T, G, M):
    moe = _moe()
    w = synth.WORKLOADS[name]
    xb = synth.generate(w.x_spec(), w.seed, rows=np.arange(T))
    wrb = w.router_weight()
    b = w.bias()
    log(f"moe_route_topk_fp8 {name} T={T} G={G} M={M}")
    r = _run_route_fp8(moe, bf16_to_dev(xb), bf16_to_dev(wrb), b, w.k, G, M)
    agree = _route_fp8_check(xb, wrb, b, w.k, *r, G=G, M=M)
    assert agree > 0.5


def test_route_topk_fp8_ragged_small():
    """T off the 128-token tile, one and two 128-expert blocks, one H block,
    k = 1 and k = 32 (the largest)."""
    moe = _moe()
    rng = np.random.default_rng(6)
    for T, H, N, k in [(33, 256, 128, 4), (129, 640, 256, 8), (300, 1024, 128, 8),
                       (1, 128, 128, 1), (70, 384, 128, 128 // 4)]:
        x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        wr = synth.f32_to_bf16_bits((rng.standard_normal((N, H)) * 0.05).astype(np.float32))
        b = rng.uniform(-0.1, 0.1, N).astype(np.float32)
        log(f"moe_route_topk_fp8 ragged T={T} H={H} N={N} k={k}")
        r = _run_route_fp8(moe, bf16_to_dev(x), bf16_to_dev(wr), b, k)
        _route_fp8_check(x, wr, b, k, *r)


def test_route_topk_fp8_full_routing_workload_sampled():
    """The routing workload at full size (T = 16384) through the FP8 router;
    the oracle checks a seeded sample of 256 tokens (first, last, random)."""
    moe = _moe()
    w = synth.WORKLOADS["routing"]
    x = device_tensor(w.x_spec(), w.seed)
    wrb = w.router_weight()
    b = w.bias()
    log(f"moe_route_topk_fp8 routing full T={w.T}")
    xq, xd, wq, wd, s, idx, gate, idx_b = _run_route_fp8(moe, x, bf16_to_dev(wrb), b, w.k)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 1, w.T - 1], rng.choice(w.T, 253, replace=False)]))
    xb = synth.generate(w.x_spec(), w.seed, rows=rows)
    _route_fp8_check(xb, wrb, b, w.k, xq[rows], xd[rows], wq, wd, s[rows], idx[rows], gate[rows],
                     idx_b[rows])
    agree = float(np.mean(np.all(np.sort(idx, 1) == np.sort(idx_b, 1), axis=1)))
    print(f"agreement with the bf16 router over all {w.T} tokens: {agree:.4f}")


@pytest.mark.parametrize("T,N,G,M,k,ties", [(1000, 256, 8, 4, 8, False), (777, 256, 8, 4, 8, True),
                                            (300, 64, 4, 2, 4, False), (200, 960, 60, 6, 12, True),
                                            (64, 16, 2, 1, 2, False), (50, 48, 3, 3, 3, True)])
def test_topk_from_scores_grouped_bit_exact(T, N, G, M, k, ties):
    """Group-limited selection against the oracle's, bit-exact, with and
    without exact ties in the scores (group ties included)."""
    moe = _moe()
    rng = np.random.default_rng(T + N + G)
    s = rng.uniform(0, 1, (T, N)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, N).astype(np.float32)
    if ties:
        s = (np.round(s * 8) / 8).astype(np.float32)
        b[:] = 0
    log(f"moe_topk_from_scores grouped T={T} N={N} G={G} M={M} k={k}")
    idx, gate = moe.moe_topk_from_scores(to_dev(s), to_dev(b), k, n_groups=G, topk_groups=M)
    torch.cuda.synchronize()
    want = route.select_topk_grouped(s, b, k, G, M)
    assert np.array_equal(idx.cpu().numpy(), want)
    np.testing.assert_allclose(gate.cpu().numpy(), route.gates(s, want), rtol=2e-6, atol=1e-7)


def test_route_topk_grouped_v3_shape():
    """The fused router with 8 groups of 32 experts, 4 groups eligible, at the
    DeepSeek-V3 shape: bit-exact to the oracle's group-limited rule on the
    GPU's own scores, every token within 4 groups, and different from the
    plain top-k on some tokens."""
    moe = _moe()
    w = synth.WORKLOADS["prefill"]
    T = 2048
    xb = synth.generate(w.x_spec(), w.seed, rows=np.arange(T))
    wrb = w.router_weight()
    b = w.bias()
    log(f"moe_route_topk grouped T={T}")
    idx, gate, s = moe.moe_route_topk(bf16_to_dev(xb), bf16_to_dev(wrb), to_dev(b), w.k,
                                      n_groups=8, topk_groups=4)
    torch.cuda.synchronize()
    s_gpu, idx_gpu = s.cpu().numpy(), idx.cpu().numpy()
    want = route.select_topk_grouped(s_gpu, b, w.k, 8, 4)
    assert np.array_equal(idx_gpu, want)
    np.testing.assert_allclose(gate.cpu().numpy(), route.gates(s_gpu, want), rtol=2e-6, atol=1e-7)
    assert max(len(set((r // 32).tolist())) for r in idx_gpu) <= 4
    assert np.any(np.sort(idx_gpu, 1) != np.sort(route.select_topk(s_gpu, b, w.k), 1))
    s64 = route.router_scores(synth.as_f64(xb), synth.as_f64(wrb))
    assert np.max(np.abs(s_gpu - s64)) < 1e-5


# --------------------------------------------------------------------------- permutation


@pytest.mark.parametrize("T,N,k,shared", [(1, 16, 1, True), (255, 16, 2, True),
                                          (256, 256, 8, True), (257, 256, 8, False),
                                          (4097, 1000, 8, True), (3000, 64, 32, True),
                                          (16384, 256, 8, True),
                                          (600, 1024, 32, True)])   # the largest N and k
def test_permute_bit_exact(T, N, k, shared):
    moe = _moe()
    rng = np.random.default_rng(T * 7 + N)
    n_use = N - 5 if N >= 64 else N              # leave some experts empty
    allowed = rng.permutation(N)[:n_use]
    idx = allowed[np.argsort(rng.uniform(size=(T, n_use)), axis=1)[:, :k]].astype(np.int32)
    log(f"moe_permute T={T} N={N} k={k} shared={shared}")
    c, o, r, t = moe.moe_permute(to_dev(idx), N, shared)
    torch.cuda.synchronize()
    wc, wo, wr, wt = opermute.permute(idx, N, shared)
    assert np.array_equal(c.cpu().numpy(), wc)
    assert np.array_equal(o.cpu().numpy(), wo)
    assert np.array_equal(r.cpu().numpy(), wr)
    assert np.array_equal(t.cpu().numpy(), wt)


# --------------------------------------------------------------------------- grouped GEMM


def _ragged_offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def _int_codes(rng, shape, lim=4):
    return e4m3.encode(rng.integers(-lim, lim + 1, shape).astype(np.float64))


@pytest.mark.parametrize("K,n_out,sizes,gather", [
    (128, 256, [1, 200, 0, 77], True),          # one K block: the prologue alone
    (256, 256, [0, 1, 127, 128, 129, 300, 0], False),
    (512, 256, [129, 40], False),               # four K blocks: one copy per wave group
    (384, 384, [3, 140, 0, 64], True),
    (256, 384, [20, 64, 192, 100, 33], True),   # tails of 20, 64 and 33 rows: narrow tiles
    (7168, 512, [5, 0, 200], True),
    (2048, 7168, [130, 3], False),
    (16384, 256, [3, 130], True),               # the largest K: 128 K blocks
    (1152, 512, [255, 256, 257, 600, 0, 31], True),   # 256-row tiles: evenly split groups
    # the last group spread over the XCD runs in 8 column parts (at least 8
    # other groups and 8 column tiles): one column tile per part, parts of
    # one and two, and 7 column tiles (no spread); empty groups at the part
    # boundaries
    (256, 2048, [40, 0, 0, 130, 7, 0, 256, 1, 600], True),
    (256, 2304, [3, 300, 0, 0, 0, 64, 129, 0, 17, 250, 0, 9, 0, 0, 511, 2, 700], False),
    (128, 1792, [10, 0, 257, 33, 0, 0, 128, 1, 90, 513], True),
])
def test_gemm_integer_operands_bit_exact(K, n_out, sizes, gather):
    """Integer-valued codes with power-of-two scales: every partial sum is an
    exact integer, so the result is exact for any summation order."""
    moe = _moe()
    rng = np.random.default_rng(K + n_out)
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    a_rows = R + 13
    aq = _int_codes(rng, (a_rows, K))
    ad = np.full((a_rows, K // 128), 2.0 ** -3, np.float32)
    bq = _int_codes(rng, (G, n_out, K))
    bd = np.full((G, n_out // 128, K // 128), 2.0 ** -5, np.float32)
    rix = rng.integers(0, a_rows, R).astype(np.int32) if gather else None
    src = rix if gather else np.arange(R)
    want = np.zeros((R, n_out))
    for g in range(G):
        rr = np.arange(off[g], off[g + 1])
        if rr.size:
            want[rr] = ffn.block_scaled_gemm(aq[src[rr]], ad[src[rr]], bq[g], bd[g])
    # the bf16 epilogue on both row tiles where the columns allow 256-row tiles
    runs = [(moe.MOE_EPI_F32, None)] + [(moe.MOE_EPI_BF16, t) for t in
                                        ((128, 256) if n_out % 256 == 0 else (None,))]
    for epi, tile_rows in runs:
        log(f"moe_grouped_gemm_fp8 integer K={K} n_out={n_out} sizes={sizes} epi={epi} tile_rows={tile_rows}")
        out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                          to_dev(off), R, epi,
                                          a_row_index=to_dev(rix) if gather else None,
                                          tile_rows=tile_rows)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        ref = want if epi == moe.MOE_EPI_F32 else ffn.bf16_round(want)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("K,n_out,tile_rows", [(256, 384, None), (7168, 384, None),
                                               (256, 512, 256), (2048, 512, 256)])
def test_gemm_bf16_row_scale_bit_exact(K, n_out, tile_rows):
    """The bf16 epilogue's per-row multiplier: out = bf16(fl32(C * row_scale))
    with C exact (integer operands, power-of-two scales), so the result is
    bit-exact: the float32 product, then round to nearest even bf16.  With
    128-row tiles K = 256 runs the single-group K loop, K = 7168 the
    ping-pong; the others run the 256-row kernel."""
    moe = _moe()
    rng = np.random.default_rng(K + 5)
    sizes = [70, 0, 200, 1]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    aq = _int_codes(rng, (R + 9, K))
    ad = np.full((R + 9, K // 128), 2.0 ** -3, np.float32)
    bq = _int_codes(rng, (G, n_out, K))
    bd = np.full((G, n_out // 128, K // 128), 2.0 ** -5, np.float32)
    rix = rng.integers(0, R + 9, R).astype(np.int32)
    rs = rng.uniform(0.1, 2.0, R).astype(np.float32)
    c = np.zeros((R, n_out))
    for g in range(G):
        rr = np.arange(off[g], off[g + 1])
        if rr.size:
            c[rr] = ffn.block_scaled_gemm(aq[rix[rr]], ad[rix[rr]], bq[g], bd[g])
    want = ffn.bf16_round((c.astype(np.float32) * rs[:, None]).astype(np.float64))
    log(f"moe_grouped_gemm_fp8 bf16 row_scale K={K} n_out={n_out} tile_rows={tile_rows}")
    out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                      to_dev(off), R, moe.MOE_EPI_BF16, a_row_index=to_dev(rix),
                                      row_scale=to_dev(rs), tile_rows=tile_rows)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), want)


def test_strided_rows_bit_exact():
    """Row strides larger than the row: the quantiser reads x as a column
    slice of a wider bf16 array (ld > cols), and the GEMM reads A as a column
    slice (lda > K) and writes into a column slice of a wider output
    (ldo > n_out); all bit-exact against the oracle on the same values."""
    moe = _moe()
    rng = np.random.default_rng(77)
    rows, cols = 300, 512
    wide = (rng.standard_normal((rows, cols + 384)) * np.exp(rng.uniform(-3, 3, (rows, 1))))
    wide_b = synth.f32_to_bf16_bits(wide.astype(np.float32))
    wide_dev = bf16_to_dev(wide_b)
    log("fp8_quant_1x128 strided rows")
    q, d = moe.fp8_quant_1x128(wide_dev[:, 128:128 + cols])
    torch.cuda.synchronize()
    wq, wd = quant.quant_1x128(synth.as_f64(wide_b[:, 128:128 + cols]))
    assert np.array_equal(q.cpu().numpy(), wq) and np.array_equal(d.cpu().numpy(), wd)

    K, n_out = 256, 384
    sizes = [100, 3, 150]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    a_wide = _int_codes(rng, (R, K + 256))
    aq = a_wide[:, 128:128 + K]
    ad = np.full((R, K // 128), 2.0 ** -3, np.float32)
    bq = _int_codes(rng, (G, n_out, K))
    bd = np.full((G, n_out // 128, K // 128), 2.0 ** -5, np.float32)
    want = np.zeros((R, n_out))
    for g in range(G):
        rr = np.arange(off[g], off[g + 1])
        want[rr] = ffn.block_scaled_gemm(aq[rr], ad[rr], bq[g], bd[g])
    out_wide = torch.zeros(R, n_out + 128, dtype=torch.bfloat16, device="cuda")
    log("moe_grouped_gemm_fp8 strided A and output")
    moe.moe_grouped_gemm_fp8(to_dev(a_wide)[:, 128:128 + K], to_dev(ad), to_dev(bq), to_dev(bd),
                             to_dev(off), R, moe.MOE_EPI_BF16, out=out_wide[:, 64:64 + n_out])
    torch.cuda.synchronize()
    got = out_wide.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:, 64:64 + n_out], ffn.bf16_round(want))
    assert not got[:, :64].any() and not got[:, 64 + n_out:].any()   # nothing outside the slice


def test_strided_rows_256_row_tiles():
    """The 256-row kernel with row strides larger than the row: A read as a
    column slice (lda > K), the bf16 output written into a column slice of a
    wider array (ldo > n_out, bit-exact against the oracle), and the SwiGLU
    codes into a column slice of a wider byte array (identical to the
    128-row kernel's); nothing outside either slice is written."""
    moe = _moe()
    rng = np.random.default_rng(78)
    K, n_out = 384, 512
    sizes = [300, 3, 0, 257]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    a_wide = _int_codes(rng, (R, K + 256))
    aq = a_wide[:, 128:128 + K]
    ad = np.full((R, K // 128), 2.0 ** -3, np.float32)
    bq = _int_codes(rng, (G, n_out, K))
    bd = np.full((G, n_out // 128, K // 128), 2.0 ** -5, np.float32)
    want = np.zeros((R, n_out))
    for g in range(G):
        rr = np.arange(off[g], off[g + 1])
        if rr.size:
            want[rr] = ffn.block_scaled_gemm(aq[rr], ad[rr], bq[g], bd[g])
    out_wide = torch.zeros(R, n_out + 128, dtype=torch.bfloat16, device="cuda")
    log("moe_grouped_gemm_fp8_tiles bf16 strided A and output, 256-row tiles")
    moe.moe_grouped_gemm_fp8(to_dev(a_wide)[:, 128:128 + K], to_dev(ad), to_dev(bq), to_dev(bd),
                             to_dev(off), R, moe.MOE_EPI_BF16, out=out_wide[:, 64:64 + n_out], tile_rows=256)
    torch.cuda.synchronize()
    got = out_wide.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:, 64:64 + n_out], ffn.bf16_round(want))
    assert not got[:, :64].any() and not got[:, 64 + n_out:].any()
    # SwiGLU codes into a slice of a wider byte array, on both row tiles
    xb = synth.f32_to_bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    xq, xd = moe.fp8_quant_1x128(bf16_to_dev(xb))
    w1 = synth.f32_to_bf16_bits((rng.standard_normal((G, n_out, K)) * 0.05).astype(np.float32))
    w1q, w1d = moe.fp8_quant_128x128(bf16_to_dev(w1), interleave_gate_up=True)
    got_h = {}
    for t in (128, 256):
        hq_wide = torch.zeros(R, n_out // 2 + 64, dtype=torch.uint8, device="cuda")
        hd = torch.zeros(R, n_out // 256, dtype=torch.float32, device="cuda")
        log(f"moe_grouped_gemm_fp8_tiles swiglu strided output tile_rows={t}")
        moe.moe_grouped_gemm_fp8(xq, xd, w1q, w1d, to_dev(off), R, moe.MOE_EPI_SWIGLU_FP8,
                                 out=hq_wide[:, 32:32 + n_out // 2], out_d=hd, tile_rows=t)
        torch.cuda.synchronize()
        got_h[t] = (hq_wide.cpu().numpy(), hd.cpu().numpy())
    np.testing.assert_array_equal(got_h[256][0], got_h[128][0])
    np.testing.assert_array_equal(got_h[256][1].view(np.uint32), got_h[128][1].view(np.uint32))
    assert not got_h[256][0][:, :32].any() and not got_h[256][0][:, 32 + n_out // 2:].any()
    assert np.count_nonzero(got_h[256][0][:, 32:32 + n_out // 2]) > R * n_out // 8


def test_gemm_many_groups_bit_exact():
    """1025 groups (the most the tile scan takes, three per thread), most of
    them empty, the others of 1 to 140 rows and a few split over two or three
    256-row tiles, integer operands: bit-exact with the float32 epilogue and
    with the bf16 one on both row tiles."""
    moe = _moe()
    rng = np.random.default_rng(1025)
    G, K, n_out = 1025, 256, 256
    sizes = np.zeros(G, np.int64)
    live = rng.choice(G, 40, replace=False)
    sizes[live] = rng.integers(1, 141, live.size)
    sizes[live[:3]] = [300, 513, 257]       # split over several 256-row tiles
    sizes[G - 1] = 129                      # the last group: a one-row tail
    off = _ragged_offsets(sizes)
    R = int(off[-1])
    aq = _int_codes(rng, (R, K))
    ad = np.full((R, K // 128), 2.0 ** -2, np.float32)
    bq = np.zeros((G, n_out, K), np.uint8)
    bd = np.full((G, n_out // 128, K // 128), 2.0 ** -4, np.float32)
    for g in np.nonzero(sizes)[0]:
        bq[g] = _int_codes(rng, (n_out, K))
    want = np.zeros((R, n_out))
    for g in np.nonzero(sizes)[0]:
        rr = np.arange(off[g], off[g + 1])
        want[rr] = ffn.block_scaled_gemm(aq[rr], ad[rr], bq[g], bd[g])
    for epi, tile_rows in ((moe.MOE_EPI_F32, None), (moe.MOE_EPI_BF16, 128), (moe.MOE_EPI_BF16, 256)):
        log(f"moe_grouped_gemm_fp8 1025 groups epi={epi} tile_rows={tile_rows}")
        out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                          to_dev(off), R, epi, tile_rows=tile_rows)
        torch.cuda.synchronize()
        ref = want if epi == moe.MOE_EPI_F32 else ffn.bf16_round(want)
        assert np.array_equal(out.float().cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("n_out,K", [(6912, 128), (7040, 128), (7040, 384)])
def test_gemm_paired_column_tiles_bit_exact(n_out, K):
    """A grid large enough (about 75 k rows, 27 or 28 column tiles) that the
    bf16 and float32 epilogues compute two column tiles per workgroup; an odd
    count of column tiles (the last pair holds one) and a 128-wide last tile.
    With the bf16 epilogue the second tile's first stage is requested before
    the first tile's epilogue (one K block: the only stage; three: the first
    wait also counts the epilogue's stores).  Integer operands, so every
    output is exact: sampled rows (every group's first and last rows and
    ragged tails, and random ones) bit-exact."""
    moe = _moe()
    rng = np.random.default_rng(n_out + K)
    sizes = [40000, 17, 35000]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    aq = _int_codes(rng, (R, K))
    ad = np.full((R, K // 128), 2.0 ** -3, np.float32)
    bq = _int_codes(rng, (G, n_out, K))
    bd = np.full((G, n_out // 128, K // 128), 2.0 ** -5, np.float32)
    rows = np.unique(np.concatenate([off[:-1], off[1:] - 1, [39999 - 63, 39999 - 64],
                                     rng.integers(0, R, 200)]))
    rows_dev = torch.from_numpy(rows.astype(np.int64)).cuda()
    want = np.zeros((rows.size, n_out))
    for g in range(G):
        sel = (rows >= off[g]) & (rows < off[g + 1])
        if sel.any():
            want[sel] = ffn.block_scaled_gemm(aq[rows[sel]], ad[rows[sel]], bq[g], bd[g])
    for epi in (moe.MOE_EPI_F32, moe.MOE_EPI_BF16):
        log(f"moe_grouped_gemm_fp8 paired columns n_out={n_out} epi={epi}")
        out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                          to_dev(off), R, epi)
        got = out.index_select(0, rows_dev).float().cpu().numpy().astype(np.float64)
        del out
        torch.cuda.synchronize()
        ref = want if epi == moe.MOE_EPI_F32 else ffn.bf16_round(want)
        assert np.array_equal(got, ref)


def _random_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)   # no NaN codes


def test_gemm_random_operands_f32():
    moe = _moe()
    rng = np.random.default_rng(11)
    sizes = [17, 0, 260, 128, 1]
    off = _ragged_offsets(sizes)
    R, G, K, n_out = int(off[-1]), len(sizes), 1024, 512
    aq = _random_codes(rng, (R, K))
    ad = rng.uniform(1e-3, 1e-2, (R, K // 128)).astype(np.float32)
    bq = _random_codes(rng, (G, n_out, K))
    bd = rng.uniform(1e-3, 1e-2, (G, n_out // 128, K // 128)).astype(np.float32)
    log("moe_grouped_gemm_fp8 random f32")
    out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                      to_dev(off), R, moe.MOE_EPI_F32)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for g in range(G):
        rr = slice(off[g], off[g + 1])
        if off[g + 1] > off[g]:
            want = ffn.block_scaled_gemm(aq[rr], ad[rr], bq[g], bd[g])
            scale = np.abs(ffn.block_scaled_gemm(aq[rr] & 0x7F, ad[rr], bq[g] & 0x7F, bd[g]))
            worst = max(worst, float(np.max(np.abs(got[rr] - want) / scale)))
    # The MFMA's own 128-deep FP8 dot product is not a round-to-nearest float32
    # sum: on full-range random codes it sits ~1e-5 of sum|a*b| away from the
    # exact block sum.  An indexing or scaling mistake would be O(1).
    print(f"max |C - exact| / sum|a*b| = {worst:.3e}")
    assert worst <= 1e-4


@pytest.mark.parametrize("K", [2048, 7168])
def test_gemm_single_group_against_library_matmul(K):
    """A single group holding every row is an ordinary GEMM: compared with
    torch's float32 matmul (rocBLAS / hipBLASLt, an independent library) on
    the dequantised operands, within the FP8 MFMA's block-sum band
    (2^-13 of sum|a*b| per 128-deep block) plus the library's own float32
    rounding.  K = 2048 runs the single-group K loop, K = 7168 the
    ping-pong."""
    moe = _moe()
    rng = np.random.default_rng(K)
    M, N = 1000, 512
    aq = _random_codes(rng, (M, K))
    ad = rng.uniform(1e-3, 1e-2, (M, K // 128)).astype(np.float32)
    bq = _random_codes(rng, (1, N, K))
    bd = rng.uniform(1e-3, 1e-2, (1, N // 128, K // 128)).astype(np.float32)
    off = np.array([0, M], np.int32)
    log(f"moe_grouped_gemm_fp8 single group vs torch.matmul K={K}")
    out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                      to_dev(off), M, moe.MOE_EPI_F32)
    table = torch.from_numpy(e4m3.TABLE.astype(np.float32)).cuda()
    a = table[to_dev(aq).long()] * to_dev(ad).repeat_interleave(128, dim=1)
    sb = to_dev(bd[0]).repeat_interleave(128, dim=0).repeat_interleave(128, dim=1)
    b = table[to_dev(bq[0]).long()] * sb
    ref = torch.matmul(a, b.t().contiguous())
    mag = torch.matmul(a.abs(), b.abs().t().contiguous())
    ratio = ((out - ref).abs() / mag).max().item()
    torch.cuda.synchronize()
    print(f"max |ours - library| / sum|a*b| = {ratio:.3e}")
    assert ratio <= 2e-4


def _swiglu_case(integer, tile_rows=None):
    moe = _moe()
    rng = np.random.default_rng(12)
    H, I = 512, 256
    sizes = [40, 0, 130, 7, 64, 20, 192, 257, 513]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    T = 50
    if integer:
        # integer codes, power-of-two scales: the GEMM result a is exact on both
        # sides, so only the epilogue's float32 SiLU and quantiser are compared
        xq = _int_codes(rng, (T, H), 2)
        xd = np.full((T, H // 128), 2.0 ** -4, np.float32)
        w1q_nat = _int_codes(rng, (G, 2 * I, H), 2)
        w1d_nat = np.full((G, 2 * I // 128, H // 128), 2.0 ** -6, np.float32)
        nb = 2 * I // 128
        order = np.array([j // 2 if j % 2 == 0 else nb // 2 + j // 2 for j in range(nb)])
        w1q_dev = to_dev(w1q_nat.reshape(G, nb, 128, H)[:, order].reshape(G, 2 * I, H))
        w1d_dev = to_dev(w1d_nat[:, order])
    else:
        xb = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        xq, xd = quant.quant_1x128(synth.as_f64(xb))
        w1 = synth.f32_to_bf16_bits((rng.standard_normal((G, 2 * I, H)) * 0.02).astype(np.float32))
        w1q_nat, w1d_nat = quant.quant_128x128(synth.as_f64(w1))
        w1q_dev, w1d_dev = moe.fp8_quant_128x128(bf16_to_dev(w1), interleave_gate_up=True)
    tok = rng.integers(0, T, R).astype(np.int32)
    log(f"moe_grouped_gemm_fp8 swiglu integer={integer} tile_rows={tile_rows}")
    hq, hd = moe.moe_grouped_gemm_fp8(to_dev(xq), to_dev(xd), w1q_dev, w1d_dev, to_dev(off), R,
                                      moe.MOE_EPI_SWIGLU_FP8, a_row_index=to_dev(tok),
                                      tile_rows=tile_rows)
    torch.cuda.synchronize()
    return hq.cpu().numpy(), hd.cpu().numpy(), xq, xd, w1q_nat, w1d_nat, tok, off, I


@pytest.mark.parametrize("tile_rows", [128, 256])
@pytest.mark.parametrize("integer", [True, False])
def test_gemm_swiglu_epilogue(integer, tile_rows):
    """Integer operands: a is exact on both sides, so codes must match except
    within 2e-6 of a rounding tie and the scales to 1e-6.  Random operands: a
    carries the MFMA block-sum error, so h is checked against the oracle with
    the per-element band propagated from that bound (check_h): scales and
    dequantised values inside it, differing codes only at rounding midpoints
    inside it and roundings of values inside it, and at most flip_cap of them."""
    hq, hd, xq, xd, w1q_nat, w1d_nat, tok, off, I = _swiglu_case(integer, tile_rows)
    n_diff, n_all = 0, 0
    for g in range(len(off) - 1):
        rr = np.arange(off[g], off[g + 1])
        if not rr.size:
            continue
        res = ffn.expert_ffn(xq[tok[rr]], xd[tok[rr]], w1q_nat[g], w1d_nat[g],
                             np.zeros((128, I), np.uint8), np.ones((1, I // 128), np.float32), "Q")
        h = res["h"]
        amax = np.abs(h).reshape(rr.size, I // 128, 128).max(-1)
        if integer:
            np.testing.assert_allclose(hd[rr], res["hd"], rtol=1e-6)
            n_diff += codes_agree_up_to_ties(hq[rr], res["hq"], h * np.repeat(448.0 / amax, 128, 1),
                                             rel=2e-6)
        else:
            band = swiglu_band(xq[tok[rr]], xd[tok[rr]], w1q_nat[g], w1d_nat[g], h, res["a"])
            n_diff += check_h(hq[rr], hd[rr], res, band)
        n_all += h.size
    print(f"h codes differing: {n_diff} of {n_all}")
    if integer:
        assert n_diff <= 1e-4 * n_all
    else:
        assert n_diff <= flip_cap(n_all)


@pytest.mark.parametrize("K", [128, 256, 384, 1152, 2176])
def test_gemm_swiglu_tile_sizes_agree_bit_exact(K):
    """The 256-row and the 128-row SwiGLU kernels form every output from the
    same sequence of per-block MFMA products and fused multiply-adds, then the
    same float32 epilogue, so their codes and scales must be identical bit for
    bit.  Group sizes straddle both tile heights (empty, 1, 255-257, 511-513,
    rows past a 64-row band), and K covers 1, 2 and 3 K blocks (the prologue
    and the loop's tail) and 9 and 17 (past one and two 8-block scale
    windows); the A rows are gathered through a random index."""
    moe = _moe()
    rng = np.random.default_rng(1000 + K)
    I = 256
    sizes = [1, 0, 255, 256, 257, 300, 17, 511, 512, 513, 64, 65, 129, 0, 3]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    T = 700
    xb = synth.f32_to_bf16_bits(rng.standard_normal((T, K)).astype(np.float32))
    xq, xd = moe.fp8_quant_1x128(bf16_to_dev(xb))
    w1 = synth.f32_to_bf16_bits((rng.standard_normal((G, 2 * I, K)) * 0.03).astype(np.float32))
    w1q, w1d = moe.fp8_quant_128x128(bf16_to_dev(w1), interleave_gate_up=True)
    tok = to_dev(rng.integers(0, T, R).astype(np.int32))
    got = {}
    for t in (128, 256, 0):
        log(f"moe_grouped_gemm_fp8_tiles swiglu K={K} tile_rows={t}")
        hq, hd = moe.moe_grouped_gemm_fp8(xq, xd, w1q, w1d, to_dev(off), R, moe.MOE_EPI_SWIGLU_FP8,
                                          a_row_index=tok, tile_rows=t)
        torch.cuda.synchronize()
        got[t] = (hq.cpu().numpy(), hd.cpu().numpy())
    for t in (256, 0):
        np.testing.assert_array_equal(got[t][0], got[128][0])
        np.testing.assert_array_equal(got[t][1].view(np.uint32), got[128][1].view(np.uint32))
    assert np.count_nonzero(got[128][0]) > R * I // 4      # the outputs carry data


@pytest.mark.parametrize("K", [128, 384, 2048, 2176])
def test_gemm_bf16_tile_sizes_agree_bit_exact(K):
    """The 256-row and 128-row kernels with the bf16 epilogue: the same
    per-block products and fused multiply-adds per output, so identical bf16
    outputs, on random operands, ragged groups straddling both tile heights
    and 1 to 17 K blocks (the 128-row kernel runs its single-group loop up to
    16 K blocks and the ping-pong beyond)."""
    moe = _moe()
    rng = np.random.default_rng(2000 + K)
    n_out = 768
    sizes = [1, 0, 255, 256, 257, 300, 17, 511, 512, 513, 64, 65, 129, 0, 3]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    xb = synth.f32_to_bf16_bits(rng.standard_normal((R, K)).astype(np.float32))
    aq, ad = moe.fp8_quant_1x128(bf16_to_dev(xb))
    w = synth.f32_to_bf16_bits((rng.standard_normal((G, n_out, K)) * 0.03).astype(np.float32))
    bq, bd = moe.fp8_quant_128x128(bf16_to_dev(w))
    got = {}
    for t in (128, 256, 0):
        log(f"moe_grouped_gemm_fp8_tiles bf16 K={K} tile_rows={t}")
        out, _ = moe.moe_grouped_gemm_fp8(aq, ad, bq, bd, to_dev(off), R, moe.MOE_EPI_BF16, tile_rows=t)
        torch.cuda.synchronize()
        got[t] = out.view(torch.int16).cpu().numpy()
    for t in (256, 0):
        np.testing.assert_array_equal(got[t], got[128])
    assert np.count_nonzero(got[128]) > R * n_out // 2


def _gpu_silu_rel_bound(g):
    """Relative error bound of the epilogue's float32 SwiGLU against the
    oracle's correctly rounded float32 chain on the same accumulators: the
    hardware exp of -g * log2(e) (argument rounding |g| 2^-24, result 1 ulp),
    the hardware reciprocal (1 ulp) and the two products (1/2 ulp each)."""
    return (np.abs(g) + 16.0) * 2.0 ** -24


def test_gemm_swiglu_epilogue_matches_its_own_accumulators():
    """The SwiGLU epilogue against the oracle's "Q" SwiGLU and 1x128
    requantisation applied to the GEMM's own float32 accumulators (the float32
    epilogue runs the same K loop, so its output is bit for bit what the
    SwiGLU epilogue sees).  This separates the epilogue from the MFMA: scales
    within the hardware exp / reciprocal bound, and codes identical except
    where the oracle's scaled value lies within that bound of a rounding
    midpoint."""
    from oracle import e4m3
    moe = _moe()
    rng = np.random.default_rng(21)
    H, I = 1024, 256
    sizes = [40, 0, 130, 7, 64, 300, 192]
    off = _ragged_offsets(sizes)
    R, G = int(off[-1]), len(sizes)
    T = 300
    xb = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    xq, xd = quant.quant_1x128(synth.as_f64(xb))
    w1 = synth.f32_to_bf16_bits((rng.standard_normal((G, 2 * I, H)) * 0.05).astype(np.float32))
    w1q_dev, w1d_dev = moe.fp8_quant_128x128(bf16_to_dev(w1), interleave_gate_up=True)
    tok = rng.integers(0, T, R).astype(np.int32)
    args = (to_dev(xq), to_dev(xd), w1q_dev, w1d_dev, to_dev(off), R)
    log("moe_grouped_gemm_fp8 swiglu vs own float32 accumulators")
    hq, hd = moe.moe_grouped_gemm_fp8(*args, moe.MOE_EPI_SWIGLU_FP8, a_row_index=to_dev(tok))
    a, _ = moe.moe_grouped_gemm_fp8(*args, moe.MOE_EPI_F32, a_row_index=to_dev(tok))
    torch.cuda.synchronize()
    hq, hd = hq.cpu().numpy(), hd.cpu().numpy().astype(np.float64)
    a = a.cpu().numpy().astype(np.float64).reshape(R, I // 128, 2, 128)
    gate = a[:, :, 0, :].reshape(R, I)                 # interleaved: gate block j, then up block j
    up = a[:, :, 1, :].reshape(R, I)
    h = ffn.fl32(ffn.silu32(gate) * up)
    want_q, want_d = quant.quant_1x128(h)
    rel = _gpu_silu_rel_bound(gate)
    rel_t = rel.reshape(R, I // 128, 128).max(-1)
    assert np.all(np.abs(hd - want_d) <= (rel_t + 2.0 ** -23) * want_d)
    diff = hq != want_q
    n = int(diff.sum())
    if n:
        m = np.repeat(448.0 / np.abs(h).reshape(R, I // 128, 128).max(-1), 128, 1)
        scaled = np.abs(h[diff]) * m[diff]
        pos = e4m3.POS_VALUES
        mids = (pos[:-1] + pos[1:]) / 2
        i = np.clip(np.searchsorted(mids, scaled), 1, mids.size - 1)
        dist = np.minimum(np.abs(scaled - mids[i - 1]), np.abs(scaled - mids[i]))
        tol = (rel[diff] + np.repeat(rel_t, 128, 1)[diff] + 2.0 ** -22) * scaled
        assert np.all(dist <= tol), "a code differs away from a rounding midpoint"
    print(f"codes differing from the oracle on the GEMM's own accumulators: {n} of {hq.size}")
    assert n <= 1e-4 * hq.size


# --------------------------------------------------------------------------- combine, bias


@pytest.mark.parametrize("T,H,k,shared", [(64, 256, 2, True), (300, 7168, 8, True),
                                          (5, 4096, 1, False)])
def test_combine(T, H, k, shared):
    moe = _moe()
    rng = np.random.default_rng(T + H)
    R = T * k + (T if shared else 0)
    spec = synth.Spec(synth.T_ROWS, (R, H), synth.NORMAL, 0.05)
    rows_b = synth.generate(spec, 1)
    gate = rng.uniform(0.01, 1, (T, k)).astype(np.float32)
    gate /= gate.sum(1, keepdims=True)
    row_of = rng.permutation(T * k).reshape(T, k).astype(np.int32)
    log(f"moe_combine T={T} H={H} k={k}")
    y = moe.moe_combine(bf16_to_dev(rows_b), to_dev(gate), to_dev(row_of),
                        T * k if shared else -1)
    torch.cuda.synchronize()
    got = bf16_values(y)
    want = ffn.combine(synth.as_f64(rows_b), gate.astype(np.float64), row_of,
                       T * k if shared else -1, "Q")
    ulp = np.abs(want) * 2.0 ** -7 + 1e-30
    diff = np.abs(got - want)
    assert np.all(diff <= ulp)
    assert np.mean(diff > 0) < 1e-3


def test_combine_with_residual():
    moe = _moe()
    rng = np.random.default_rng(9)
    T, H, k = 16, 256, 2
    rows = synth.f32_to_bf16_bits(rng.standard_normal((T * k + T, H)).astype(np.float32))
    res = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    gate = np.full((T, k), 0.5, np.float32)
    row_of = np.arange(T * k).reshape(T, k).astype(np.int32)
    y = moe.moe_combine(bf16_to_dev(rows), to_dev(gate), to_dev(row_of), T * k,
                        residual=bf16_to_dev(res))
    torch.cuda.synchronize()
    r = synth.as_f64(rows)
    acc = ffn.fl32(synth.as_f64(res) + r[T * k:])
    for j in range(k):
        acc = ffn.fl32(acc + 0.5 * r[row_of[:, j]])
    assert np.array_equal(bf16_values(y), ffn.bf16_round(acc))


def test_bias_update_bit_exact():
    moe = _moe()
    rng = np.random.default_rng(13)
    for N, T, k, gamma in [(16, 64, 2, 1e-3), (256, 8192, 8, 1e-3), (256, 512, 8, 0.0),
                           (100, 7, 3, 0.01)]:
        b = rng.uniform(-0.05, 0.05, N).astype(np.float32)
        c = rng.integers(0, 2 * T * k // N + 2, N).astype(np.int32)
        c[:3] = T * k // N if (T * k) % N == 0 else c[:3]
        bt = to_dev(b.copy())
        log(f"moe_bias_update N={N}")
        moe.moe_bias_update(bt, to_dev(c), T, k, gamma)
        torch.cuda.synchronize()
        assert np.array_equal(bt.cpu().numpy(), obias.bias_update(b, c, T, k, gamma))


def test_mfma_block_sum_precision_probe():
    """Characterises the FP8 MFMA's internal 128-deep sum: one product of
    448 * 448 = 200704 plus 127 products of 2^e (e from 8 down to -9).  A float32
    round-to-nearest sum of these is exact for every e here.  On gfx950 the
    hardware sums each group of 8 consecutive products on a fixed-point grid
    2^-13 below the group's largest product exponent (here 2^(16-13) = 8), so
    the 7 small products that share a group with the large one are dropped
    once 2^e < 8, while the other 120 stay exact.  This test pins that
    behaviour (it is the reason the layer's h codes can differ from an exact
    oracle at rounding ties)."""
    moe = _moe()
    K, n_out = 128, 256
    es = list(range(8, -10, -1))
    rows = len(es)
    aq = np.zeros((rows, K), np.uint8)
    for i, e in enumerate(es):
        aq[i, 0] = 0x7E
        aq[i, 1:] = e4m3.encode(2.0 ** e)
    bq = np.full((1, n_out, K), e4m3.encode(1.0), np.uint8)
    bq[0, :, 0] = 0x7E
    ad = np.ones((rows, 1), np.float32)
    bd = np.ones((1, 2, 1), np.float32)
    off = np.array([0, rows], np.int32)
    log("mfma precision probe")
    out, _ = moe.moe_grouped_gemm_fp8(to_dev(aq), to_dev(ad), to_dev(bq), to_dev(bd),
                                      to_dev(off), rows, moe.MOE_EPI_F32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[:, 0].astype(np.float64)
    for i, e in enumerate(es):
        exact = 200704.0 + 127 * 2.0 ** e
        lost = (exact - got[i]) / 2.0 ** e
        print(f"small products 2^{e:+d}: exact {exact:.6f} mfma {got[i]:.6f} lost {lost:g}")
        assert lost == (0 if 2.0 ** e >= 8 else 7)


# --------------------------------------------------------------------------- balance statistic


def test_seq_balance_loss_against_oracle():
    """Router output of the prefill workload's first 3000 tokens, cut into
    ragged sequences (one empty): the per-sequence statistic within 1e-6 of
    the float64 oracle, and bit-identical when run twice."""
    moe = _moe()
    w = synth.WORKLOADS["prefill"]
    T = 3000
    xb = synth.generate(w.x_spec(), w.seed, rows=np.arange(T))
    log("moe_seq_balance_loss")
    idx, gate, _ = moe.moe_route_topk(bf16_to_dev(xb), bf16_to_dev(w.router_weight()),
                                      to_dev(w.bias()), w.k)
    off = np.array([0, 1, 1000, 1000, 2047, 3000], np.int32)
    loss = moe.moe_seq_balance_loss(idx, gate, to_dev(off), w.N)
    loss2 = moe.moe_seq_balance_loss(idx, gate, to_dev(off), w.N)
    torch.cuda.synchronize()
    want = obalance.seq_balance_loss(idx.cpu().numpy(), gate.cpu().numpy(), off, w.N)
    got = loss.cpu().numpy()
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=0)
    assert got[2] == 0.0
    assert np.array_equal(got, loss2.cpu().numpy())


# --------------------------------------------------------------------------- diagnostics


def test_mfma_rate_probe_runs():
    """The FP8 MFMA rate probe (a diagnostic the benchmark times): finite,
    positive sums from finite codes, identical on a second call."""
    moe = _moe()
    log("moe_probe_fp8_mfma")
    sink, flops = moe.moe_probe_fp8_mfma(8, 3)
    again, _ = moe.moe_probe_fp8_mfma(8, 3)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 3 * 16 * 65536
    s = sink.cpu().numpy()
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    assert np.array_equal(s, again.cpu().numpy())
