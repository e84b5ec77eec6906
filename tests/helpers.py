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


def check_h(hq, hd, h, max_frac=5e-2):
    """The re-quantised intermediate h of the FP8 GEMM path against the
    oracle's h (float64 [rows, I]).  The GPU's h carries the MFMA block-sum
    error (~1e-5 of sum|a*b|), so instead of exact codes: the scales within
    5e-4, every dequantised value within half an E4M3 step of h plus 1e-3 of
    its tile maximum, and at most `max_frac` of the codes different.  Returns
    the number of differing codes."""
    from oracle import quant
    rows, I = h.shape
    wq, wd = quant.quant_1x128(h)
    np.testing.assert_allclose(hd, wd, rtol=5e-4)
    amax = np.abs(h).reshape(rows, I // 128, 128).max(-1)
    hh = quant.dequant_1x128(hq, hd)
    dd = np.repeat(np.asarray(hd, np.float64), 128, 1)
    band = 2.0 ** -4 * np.abs(h) + 2.0 ** -10 * dd + 1e-3 * np.repeat(amax, 128, 1)
    assert np.all(np.abs(hh - h) <= band), "dequantised h outside the E4M3 + MFMA band"
    n = int(np.sum(np.asarray(hq) != wq))
    assert n <= max_frac * wq.size, f"{n} of {wq.size} h codes differ"
    return n
