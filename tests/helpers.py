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


def codes_agree_up_to_ties(got, want, scaled_oracle):
    """E4M3 codes must be equal except where the oracle value sits on a tie;
    there the two codes must be neighbours."""
    got = np.asarray(got).astype(np.int64)
    want = np.asarray(want).astype(np.int64)
    diff = got != want
    if not diff.any():
        return 0
    tie = near_tie(scaled_oracle)
    bad = diff & ~tie
    assert not bad.any(), f"{bad.sum()} codes differ away from a rounding tie"
    from oracle import e4m3
    vg = e4m3.decode(got[diff].astype(np.uint8))
    vw = e4m3.decode(want[diff].astype(np.uint8))
    ok = np.abs(vg - vw) <= np.maximum(np.abs(vw), np.abs(vg)) * 0.125 + 2.0 ** -9
    assert ok.all(), "codes at a tie differ by more than one step"
    return int(diff.sum())
