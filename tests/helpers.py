"""Shared helpers of the GPU tests: moving generator output to the device and
comparing HIP results with the oracle."""
import sys

import numpy as np

import synth


def log(msg):
    """Name the case before each GPU step, flushed, so a lost box still leaves
    a trace of what ran."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def bf16_to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_from_dev(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t):
    """device bf16 tensor -> float64 numpy values"""
    return synth.as_f64(bf16_from_dev(t))


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def device_tensor(spec, seed, dtype="bf16"):
    """Generate the whole tensor on the device with the shared definition."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = torch.empty(spec.shape, dtype=tdt, device="cuda")
    synth.device_generate(spec, seed, t)
    return t


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


def max_rel(a, b):
    """max |a - b| / max |b| over the whole array (normwise max)."""
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def near_tie(scaled, rel=2e-5):
    """True where an oracle value (already multiplied by its tile multiplier)
    lies so close to an E4M3 rounding boundary that a float32 evaluation with a
    different rounding order may land on either neighbour."""
    from oracle import e4m3
    a = np.abs(np.asarray(scaled, np.float64))
    pos = e4m3.POS_VALUES
    mids = (pos[:-1] + pos[1:]) / 2
    i = np.clip(np.searchsorted(mids, a), 1, mids.size - 1)
    d = np.minimum(np.abs(a - mids[i - 1]), np.abs(a - mids[i]))
    return d <= rel * np.maximum(a, 2.0 ** -9)


def codes_agree_up_to_ties(got, want, scaled_oracle, rel=2e-5):
    """E4M3 codes must be equal except where the oracle value lies within
    `rel` (relative) of a rounding tie; there the two codes must be
    neighbours.  Returns the number of differing codes."""
    got = np.asarray(got).astype(np.int64)
    want = np.asarray(want).astype(np.int64)
    diff = got != want
    if not diff.any():
        return 0
    tie = near_tie(scaled_oracle, rel)
    bad = diff & ~tie
    assert not bad.any(), f"{bad.sum()} codes differ away from a rounding tie"
    from oracle import e4m3
    vg = e4m3.decode(got[diff].astype(np.uint8))
    vw = e4m3.decode(want[diff].astype(np.uint8))
    ok = np.abs(vg - vw) <= np.maximum(np.abs(vw), np.abs(vg)) * 0.125 + 2.0 ** -9
    assert ok.all(), "codes at a tie differ by more than one step"
    return int(diff.sum())


# The FP8 MFMA block-sum bound (per output): gfx950's v_mfma_f32_16x16x128_f8f6f4
# sums each group of 8 products on a grid 2^-13 below the group's largest
# (test_mfma_block_sum_precision_probe), so one 128-deep block loses at most
# about 2^-13 of its absolute sum; accumulated over K blocks, and measured
# against an independent float32 library matmul at 1.9e-5 and 3.7e-5 of
# sum |a b|, the bar used throughout is
MFMA_REL = 1e-4          # |error| <= MFMA_REL * sum_kb |block product| d_A d_B
# Measured share of h codes that land on the neighbouring E4M3 value of the
# oracle's (each a value within the MFMA band of a rounding midpoint): 0.1-0.2 %
# at the prefill and decode shapes.  The bar allows 3x the upper figure.
H_FLIP_MAX_FRAC = 6e-3


def abs_codes(q):
    """E4M3 codes of |value| (the sign bit cleared)."""
    return np.asarray(q, np.uint8) & np.uint8(0x7F)


def swiglu_band(xq, xd, w1q, w1d, h_ref, a_ref):
    """Per-element bound on |h_gpu - h_oracle| from the MFMA block-sum bound,
    propagated through h = SiLU(g) * u:  |dh| <= |u| |SiLU'(g)| |dg| +
    |SiLU(g)| |du|, with |dg|, |du| <= MFMA_REL * (the same block-scaled GEMM on
    |codes|), plus a few float32 ulps of the SwiGLU arithmetic itself."""
    from oracle import ffn
    mag = ffn.block_scaled_gemm(abs_codes(xq), xd, abs_codes(w1q), w1d)
    I = h_ref.shape[1]
    g, u = a_ref[:, :I], a_ref[:, I:]
    sg = 1.0 / (1.0 + np.exp(-g))
    dsilu = np.abs(sg * (1.0 + g * (1.0 - sg)))         # |d SiLU / dg| <= 1.1
    band = MFMA_REL * (np.abs(u) * dsilu * mag[:, :I] + np.abs(g * sg) * mag[:, I:])
    return band + 8 * 2.0 ** -24 * np.abs(h_ref)


def flip_cap(n_codes, max_frac=H_FLIP_MAX_FRAC):
    """Largest allowed count of differing h codes among n_codes: the 1e-9
    upper quantile of a Poisson count whose mean is max_frac * n_codes (3x
    the measured flip rate), so a small sample is not failed by one or two
    legitimate flips while a large one is held to about max_frac."""
    from scipy.stats import poisson
    return int(poisson.ppf(1.0 - 1e-9, max_frac * n_codes))


def check_h(hq, hd, res_q, band, max_frac=H_FLIP_MAX_FRAC, max_flips=None):
    """The GPU's re-quantised intermediate h against the oracle's "Q" expert
    result ``res_q`` (dict with h, hq, hd) given the per-element bound
    ``band`` on |h_gpu - h_oracle| (swiglu_band):
      * each tile's scale within the band of the tile's largest |h|;
      * every dequantised GPU value within half an E4M3 step of the oracle's
        h plus the band (scaled);
      * a code differs from the oracle's only where the oracle's scaled value
        lies within the band of a rounding midpoint, and then it is the
        rounding of a value inside the band;
      * at most flip_cap(codes, max_frac) codes differ (or ``max_flips``).
    Returns the number of differing codes."""
    from oracle import e4m3, quant
    h = res_q["h"]
    rows, I = h.shape
    hd_ref = np.asarray(res_q["hd"], np.float64)
    hd = np.asarray(hd, np.float64)
    amax = np.abs(h).reshape(rows, I // 128, 128).max(-1)
    band_t = band.reshape(rows, I // 128, 128).max(-1)
    # d = amax / 448 correctly rounded on both sides, amax moved by <= band
    assert np.all(np.abs(hd - hd_ref) <= (band_t / 448.0) * (1 + 2.0 ** -22) + 2.0 ** -23 * hd_ref), \
        "h scale outside the MFMA band"
    m_ref = np.repeat(np.where(amax > 0, 448.0 / np.maximum(amax, 1e-300), 0.0), 128, 1)
    dd = np.repeat(hd, 128, 1)
    hh = quant.dequant_1x128(hq, hd)
    rel_d = np.repeat(np.abs(hd - hd_ref) / np.maximum(hd_ref, 1e-300), 128, 1)
    half_step = 2.0 ** -4 * np.abs(h) + 2.0 ** -10 * dd
    assert np.all(np.abs(hh - h) <= half_step + band * (1 + 2.0 ** -3) + rel_d * np.abs(h)), \
        "dequantised h outside half an E4M3 step plus the MFMA band"
    diff = np.asarray(hq) != np.asarray(res_q["hq"])
    n = int(diff.sum())
    if n:
        scaled = np.abs(h[diff]) * m_ref[diff]
        tol = (band[diff] + rel_d[diff] * np.abs(h[diff])) * m_ref[diff] * (1 + 2.0 ** -10)
        pos = e4m3.POS_VALUES
        mids = (pos[:-1] + pos[1:]) / 2
        i = np.clip(np.searchsorted(mids, scaled), 1, mids.size - 1)
        dist = np.minimum(np.abs(scaled - mids[i - 1]), np.abs(scaled - mids[i]))
        assert np.all(dist <= tol + 2.0 ** -20), "an h code differs away from a rounding midpoint"
        # the GPU code is the rounding of some value within tol of the
        # oracle's scaled value: rounding is monotone, so it lies between the
        # roundings of the interval's ends (one step either way, or, for |h|
        # below the band, the subnormals on either side of zero)
        s = h[diff] * m_ref[diff]
        vg = e4m3.decode(np.asarray(hq)[diff])
        lo = e4m3.round_to_e4m3(s - tol)
        hi = e4m3.round_to_e4m3(s + tol)
        assert np.all((lo <= vg) & (vg <= hi)), "an h code is not a rounding of a value inside the band"
    cap = flip_cap(h.size, max_frac) if max_flips is None else max_flips
    assert n <= cap, f"{n} of {h.size} h codes differ (cap {cap}, rate bar {max_frac:.1e})"
    return n
