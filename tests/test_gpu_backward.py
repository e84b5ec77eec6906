"""GPU parity of the FP8 backward GEMMs (Dgrad, Wgrad) and their operand
kernels against the CPU oracle (``oracle.backward``).  Codes, scales and the
padded offsets must match bit for bit; products within the FP8 MFMA band.

The band: one 16x16x128 FP8 MFMA sums each group of 8 products on a grid
2^-13 below the group's largest product, so its error is at most
2^-13 * sum|products|; the per-tile scaling and the float accumulation over
at most 128 token or channel tiles add at most 128 * 2^-23 = 2^-16 of it."""
import numpy as np
import pytest

import synth
from helpers import bf16_to_dev, device_tensor, log, to_dev
from oracle import backward, e4m3, quant

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

MFMA_REL = 2.0 ** -13 + 2.0 ** -16


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a device"
    import fp8_block_scaled_sigmoid_amd as moe
    moe.lib()
    return moe


def _moe():
    import fp8_block_scaled_sigmoid_amd as moe
    return moe


def _codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    return np.where((c & 0x7F) == 0x7F, c & 0xF0, c).astype(np.uint8)


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def _bf16(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_transpose_bit_exact():
    moe = _moe()
    rng = np.random.default_rng(1)
    wq = _codes(rng, (3, 256, 384))
    wd = rng.uniform(1e-4, 1e-2, (3, 2, 3)).astype(np.float32)
    log("fp8_transpose_128x128 3x256x384")
    tq, td = moe.fp8_transpose_128x128(to_dev(wq), to_dev(wd))
    torch.cuda.synchronize()
    oq, od = backward.transpose_blocks(wq, wd)
    assert np.array_equal(tq.cpu().numpy(), oq)
    assert np.array_equal(td.cpu().numpy(), od)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_tokens_bit_exact(dtype):
    moe = _moe()
    rng = np.random.default_rng(2)
    sizes = [0, 1, 127, 128, 129, 300, 0, 315]
    off = _offsets(sizes)
    R, C = int(off[-1]), 192
    x = rng.standard_normal((R, C)) * np.exp2(rng.integers(-6, 6, (1, C)))
    x[5, 7] = 0.0
    x[200:328, 3] = 0.0                                   # an all-zero tile (group 5, channel 3)
    x[310, :] *= 80.0                                     # an outlier token
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x.astype(np.float32))
        xv, xd_dev = synth.as_f64(bits), bf16_to_dev(bits)
    else:
        xv = x.astype(np.float32).astype(np.float64)
        xd_dev = to_dev(x.astype(np.float32))
    log(f"fp8_quant_tokens_128 {dtype} R={R} C={C} G={len(sizes)}")
    xt_q, xt_d, pad = moe.fp8_quant_tokens_128(xd_dev, to_dev(off))
    torch.cuda.synchronize()
    oq, od, opad = backward.quant_tokens(xv, off)
    pad = pad.cpu().numpy()
    assert np.array_equal(pad, opad)
    P = int(opad[-1])
    assert np.array_equal(xt_q.cpu().numpy()[:, :P], oq)
    assert np.array_equal(xt_d.cpu().numpy()[:, :P // 128], od)


def _check_product(got, want, mag, what):
    err = np.abs(got - want)
    ratio = np.max(err / (mag + 1e-30))
    print(f"{what}: max |got - oracle| / sum|products| = {ratio:.3e}")
    assert np.all(err <= MFMA_REL * mag + 1e-30)


@pytest.mark.parametrize("epilogue", ["f32", "bf16"])
def test_dgrad_against_oracle(epilogue):
    moe = _moe()
    rng = np.random.default_rng(3)
    sizes = [17, 0, 260, 128, 1]
    off = _offsets(sizes)
    R, N, K, G = int(off[-1]), 512, 384, len(sizes)
    dy = _bf16(rng, (R, N), 0.01)
    w = rng.standard_normal((G, N, K)) * np.exp2(rng.integers(-9, -4, (G, 1, 1)))
    wq, wd = quant.quant_128x128(w)
    log(f"moe_grouped_dgrad_fp8 {epilogue} R={R} N={N} K={K}")
    tq, td = moe.fp8_transpose_128x128(to_dev(wq), to_dev(wd))
    ep = moe.MOE_EPI_F32 if epilogue == "f32" else moe.MOE_EPI_BF16
    dx = moe.moe_grouped_dgrad_fp8(bf16_to_dev(dy), tq, td, to_dev(off), epilogue=ep)
    torch.cuda.synchronize()
    got = dx.float().cpu().numpy().astype(np.float64)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            continue
        want, dyq, dyd = backward.dgrad(synth.as_f64(dy[r0:r1]), wq[g], wd[g])
        mag = (np.abs(quant.dequant_1x128(dyq, dyd)) @ np.abs(quant.dequant_128x128(wq[g], wd[g])))
        if epilogue == "f32":
            _check_product(got[r0:r1], want, mag, f"dgrad group {g}")
        else:
            # bf16 output: one rounding (relative 2^-8) on top of the MFMA band
            err = np.abs(got[r0:r1] - want)
            assert np.all(err <= MFMA_REL * mag + 2.0 ** -8 * np.abs(want) + 1e-30)


def test_wgrad_against_oracle():
    moe = _moe()
    rng = np.random.default_rng(4)
    sizes = [17, 0, 260, 128, 1, 300]
    off = _offsets(sizes)
    R, N, K, G = int(off[-1]), 256, 384, len(sizes)
    dy = _bf16(rng, (R, N), 0.01)
    x = _bf16(rng, (R, K), 1.0)
    log(f"moe_grouped_wgrad_fp8 R={R} N={N} K={K} G={G}")
    a_q, a_d, pad = moe.fp8_quant_tokens_128(bf16_to_dev(dy), to_dev(off))
    b_q, b_d, _ = moe.fp8_quant_tokens_128(bf16_to_dev(x), to_dev(off))
    out = moe.moe_grouped_wgrad_fp8(a_q, a_d, b_q, b_d, pad)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    want, (aq, ad), (bq, bd), opad = backward.wgrad(synth.as_f64(dy), synth.as_f64(x), off)
    P = int(opad[-1])
    assert np.array_equal(a_q.cpu().numpy()[:, :P], aq)
    assert np.array_equal(b_q.cpu().numpy()[:, :P], bq)
    av, bv = np.abs(backward.dequant_tokens(aq, ad)), np.abs(backward.dequant_tokens(bq, bd))
    for g in range(G):
        sl = slice(int(opad[g]), int(opad[g + 1]))
        if sl.stop == sl.start:
            assert np.all(got[g] == 0.0)
            continue
        _check_product(got[g], want[g], av[:, sl] @ bv[:, sl].T, f"wgrad group {g}")


def test_wgrad_half_tile_and_single_group():
    """K not a multiple of the 256-column tile (half tiles), one group."""
    moe = _moe()
    rng = np.random.default_rng(5)
    off = _offsets([200])
    dy = _bf16(rng, (200, 128), 0.1)
    x = _bf16(rng, (200, 128), 1.0)
    log("moe_grouped_wgrad_fp8 half tile")
    a_q, a_d, pad = moe.fp8_quant_tokens_128(bf16_to_dev(dy), to_dev(off))
    b_q, b_d, _ = moe.fp8_quant_tokens_128(bf16_to_dev(x), to_dev(off))
    out = moe.moe_grouped_wgrad_fp8(a_q, a_d, b_q, b_d, pad)
    torch.cuda.synchronize()
    want, (aq, ad), (bq, bd), opad = backward.wgrad(synth.as_f64(dy), synth.as_f64(x), off)
    mag = np.abs(backward.dequant_tokens(aq, ad)) @ np.abs(backward.dequant_tokens(bq, bd)).T
    _check_product(out.cpu().numpy()[0].astype(np.float64), want[0], mag, "wgrad half tile")


def test_backward_v3_shape_sampled():
    """The second expert GEMM's backward at the V3 shape for the decode-size
    batch (512 tokens x 9 rows each: 256 routed experts top-8 plus the shared
    one, hidden 7168, intermediate 2048; W2 from the decode workload's seeded
    generator, built on the device), groups from a seeded multinomial: Dgrad
    dH = dOut W2 on sampled rows of five experts, Wgrad dW2 = dOut^T h on
    sampled channels of every expert, against the oracle."""
    moe = _moe()
    rng = np.random.default_rng(6)
    wl = synth.WORKLOADS["decode"]
    T, H, I, N = wl.T, wl.H, wl.I, wl.N
    sizes = np.concatenate([rng.multinomial(T * 8, np.full(N, 1.0 / N)), [T]])
    off = _offsets(sizes)
    R, G = int(off[-1]), N + 1
    dout = _bf16(rng, (R, H), 1e-3)
    h = _bf16(rng, (R, I), 1.0)
    spec = wl.w2_spec()
    log(f"backward V3 shape R={R} H={H} I={I} G={G}")
    w2q, w2d = moe.fp8_quant_128x128(device_tensor(spec, wl.seed))
    tq, td = moe.fp8_transpose_128x128(w2q, w2d)
    dh = moe.moe_grouped_dgrad_fp8(bf16_to_dev(dout), tq, td, to_dev(off), epilogue=moe.MOE_EPI_F32)
    a_q, a_d, pad = moe.fp8_quant_tokens_128(bf16_to_dev(dout), to_dev(off))
    b_q, b_d, _ = moe.fp8_quant_tokens_128(bf16_to_dev(h), to_dev(off))
    dw2 = moe.moe_grouped_wgrad_fp8(a_q, a_d, b_q, b_d, pad)
    torch.cuda.synchronize()
    # Dgrad: 3 sampled rows of each of 5 experts (first, middle, last row);
    # the oracle quantises those experts' W2 from the host generator
    dh_h = dh.cpu().numpy().astype(np.float64)
    for g in [0, 77, 128, 255, 256]:
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 == r0:
            continue
        wg = synth.as_f64(synth.generate(spec, wl.seed, rows=np.arange(g * H, (g + 1) * H)))
        wq_o, wd_o = quant.quant_128x128(wg)
        assert np.array_equal(w2q[g].cpu().numpy(), wq_o)
        rows = np.unique([r0, r1 - 1, (r0 + r1) // 2])
        want, dyq, dyd = backward.dgrad(synth.as_f64(dout[rows]), wq_o, wd_o)
        mag = np.abs(quant.dequant_1x128(dyq, dyd)) @ np.abs(quant.dequant_128x128(wq_o, wd_o))
        _check_product(dh_h[rows], want, mag, f"V3 dgrad group {g}")
    # Wgrad: 24 output channels x 40 input channels, every expert (a tile's
    # scale depends on its own channel only, so quantising the sampled
    # channels alone gives the same codes)
    cn = np.sort(rng.choice(H, 24, replace=False))
    ck = np.sort(rng.choice(I, 40, replace=False))
    want, (aq, ad), (bq, bd), opad = backward.wgrad(synth.as_f64(dout[:, cn]), synth.as_f64(h[:, ck]), off)
    assert np.array_equal(pad.cpu().numpy(), opad)
    got = dw2[:, to_dev(cn.astype(np.int64))][:, :, to_dev(ck.astype(np.int64))].cpu().numpy().astype(np.float64)
    av, bv = np.abs(backward.dequant_tokens(aq, ad)), np.abs(backward.dequant_tokens(bq, bd))
    worst = 0.0
    for g in range(G):
        sl = slice(int(opad[g]), int(opad[g + 1]))
        mag = av[:, sl] @ bv[:, sl].T
        err = np.abs(got[g] - want[g])
        assert np.all(err <= MFMA_REL * mag + 1e-30)
        worst = max(worst, float(np.max(err / (mag + 1e-30))))
    print(f"V3 wgrad sampled: max |got - oracle| / sum|products| = {worst:.3e}")
