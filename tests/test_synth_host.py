"""Host side of the seeded input generator: determinism, slice access and the
shape of the distributions (the recipe each workload states)."""
import numpy as np

import synth


def test_mix64_reference_values():
    # SplitMix64 seeded with 0 yields these first outputs (published test values
    # of the generator: state += golden, then the output function)
    z = 0
    outs = []
    for _ in range(3):
        z = (z + synth.GOLDEN) & synth.MASK64
        outs.append(synth.mix64_int(z))
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_numpy_and_int_mix_agree():
    key = synth.stream_key(3, synth.T_W1)
    w0, w1 = synth.words(key, np.arange(5))
    for i in range(5):
        base = (key + (2 * i + 1) * synth.GOLDEN) & synth.MASK64
        assert int(w0[i]) == synth.mix64_int(base)
        assert int(w1[i]) == synth.mix64_int((base + synth.GOLDEN) & synth.MASK64)


def test_row_slices_equal_the_full_tensor():
    w = synth.WORKLOADS["tiny"]
    full = synth.generate(w.w1_spec(), 0)
    rows = np.array([0, 7, 300, 17 * 256 - 1])
    part = synth.generate(w.w1_spec(), 0, rows=rows)
    assert np.array_equal(part, full.reshape(-1, w.H)[rows])
    assert not np.array_equal(synth.generate(w.w1_spec(), 1, rows=rows), part)


def test_distributions():
    spec = synth.Spec(99, (200, 1024), synth.NORMAL, 0.5)
    v = synth.as_f64(synth.generate(spec, 0))
    assert abs(v.mean()) < 5e-3 and abs(v.std() - 0.5) < 5e-3
    assert np.abs(v).max() < 0.5 * 4.9
    spec = synth.Spec(98, (1000, 128), synth.UNIFORM, 0.1, dtype="f32")
    u = synth.generate(spec, 0)
    assert u.dtype == np.float32 and np.abs(u).max() < 0.1 and abs(u.std() - 0.1 / np.sqrt(3)) < 1e-3


def test_skew_recipe():
    w = synth.WORKLOADS["skew"]
    ch = w.outlier_channels()
    assert ch.size == 72 and 0 not in ch and np.unique(ch).size == 72
    rows = synth.as_f64(synth.generate(w.x_spec(), 0, rows=np.arange(64)))
    assert np.all(rows[:, 0] == 1.0)
    assert rows[:, ch].std() > 50 and rows[:, 1:].std() < 20
    o = w.zipf_offsets()
    p = np.exp(o) / w.N
    assert abs(p.sum() - 1) < 1e-12 and np.sort(p)[::-1][0] / np.sort(p)[::-1][1] > 2
