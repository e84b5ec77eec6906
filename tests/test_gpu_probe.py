"""The HBM rate probe (moe_probe_hbm), a diagnostic the benchmark's measured
peaks come from: the read modes must touch every byte once (their sink is
the XOR of every 32-bit word of the buffer) and the write modes must write
every 16-byte vector (words 2 and 3 of each carry the probe's pattern),
including a tail past the last whole 32 KiB chunk."""
import numpy as np
import pytest

from helpers import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _moe():
    import fp8_block_scaled_sigmoid_amd as moe
    return moe


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, 3 * 32768])
@pytest.mark.parametrize("mode", [0, 2])
def test_probe_read_modes_fold_every_word(mode, nbytes):
    moe = _moe()
    log(f"moe_probe_hbm read mode={mode} bytes={nbytes}")
    rng = np.random.default_rng(nbytes + mode)
    host = rng.integers(-2 ** 31, 2 ** 31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = moe.moe_probe_hbm(mode, buf)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48])
@pytest.mark.parametrize("mode", [1, 3])
def test_probe_write_modes_cover_every_vector(mode, nbytes):
    moe = _moe()
    log(f"moe_probe_hbm write mode={mode} bytes={nbytes}")
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    moe.moe_probe_hbm(mode, buf)
    torch.cuda.synchronize()
    v = buf.cpu().numpy().view(np.uint32).reshape(-1, 4)
    assert np.all(v[:, 2] == 0x5A5A5A5A) and np.all(v[:, 3] == 0x3C3C3C3C)
