"""The allocation-free permutation entry point (moe_permute_noalloc), called
through the C ABI, against moe_permute with a caller workspace on the same
inputs: counts, offsets and both row maps bit for bit, on two calls in a row
(the second smaller, so the scratch holds the first call's data), and sizes
beyond the scratch rejected before any launch."""
import ctypes

import numpy as np
import pytest

from helpers import log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _routing(T, N, k, seed):
    rng = np.random.default_rng(seed)
    return np.argsort(rng.uniform(size=(T, N)), 1)[:, :k].astype(np.int32)


def _call(lib, fn, idx, N, shared, ws=None):
    T, k = idx.shape
    R = T * k + (T if shared else 0)
    out = [torch.full((N,), -7, dtype=torch.int32, device="cuda"),
           torch.full((N + 2,), -7, dtype=torch.int32, device="cuda"),
           torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
           torch.full((max(R, 1),), -7, dtype=torch.int32, device="cuda")]
    torch.cuda.synchronize()
    d = to_dev(idx)
    P = ctypes.c_void_p
    args = [P(d.data_ptr()), T, N, k, 1 if shared else 0] + [P(t.data_ptr()) for t in out]
    if ws is not None:
        st = fn(*args, P(ws.data_ptr()), ctypes.c_size_t(ws.numel()), None)
    else:
        st = fn(*args, None)
    torch.cuda.synchronize()
    return st, [t.cpu().numpy() for t in out]


@pytest.fixture(scope="module")
def lib():
    import fp8_block_scaled_sigmoid_amd as moe
    L = moe.lib()
    P, I = ctypes.c_void_p, ctypes.c_int
    L.moe_permute.argtypes = [P, I, I, I, I, P, P, P, P, P, ctypes.c_size_t, P]
    L.moe_permute.restype = ctypes.c_int
    L.moe_permute_noalloc.argtypes = [P, I, I, I, I, P, P, P, P, P]
    L.moe_permute_noalloc.restype = ctypes.c_int
    L.moe_permute_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
    L.moe_permute_workspace_bytes.argtypes = [I, I, I]
    L.moe_permute_workspace_bytes.restype = ctypes.c_size_t
    return L


def test_no_alloc_permute_matches_the_workspace_entry_point(lib):
    # two calls in a row, the second smaller: the scratch still holds the
    # first call's block counts when the second runs
    for T, N, k, shared, seed in [(16384, 256, 8, True, 1), (700, 64, 4, False, 2), (5, 16, 2, True, 3)]:
        idx = _routing(T, N, k, seed)
        ws = torch.empty(int(lib.moe_permute_workspace_bytes(T, N, k)) + 16, dtype=torch.uint8,
                         device="cuda")
        log(f"moe_permute vs moe_permute_noalloc T={T} N={N} k={k} shared={shared}")
        st_ws, want = _call(lib, lib.moe_permute, idx, N, shared, ws)
        st_na, got = _call(lib, lib.moe_permute_noalloc, idx, N, shared)
        assert st_ws == 0 and st_na == 0
        for g, w_ in zip(got, want):
            assert np.array_equal(g, w_)
        assert want[0].sum() == T * k


def test_no_alloc_permute_rejects_sizes_beyond_its_scratch(lib):
    cap = int(lib.moe_permute_noalloc_max_scratch_bytes())
    assert cap == 1 << 20
    N, k = 1024, 8
    T = 65536 + 1                  # ceil(T / 256) * N * 4 bytes > 1 MiB
    assert lib.moe_permute_workspace_bytes(T, N, k) > cap
    idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    outs = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (N, N + 2, T * k, T * k + T)]
    P = ctypes.c_void_p
    st = lib.moe_permute_noalloc(P(idx.data_ptr()), T, N, k, 1, *[P(o.data_ptr()) for o in outs],
                                 None)
    assert st == 6                 # MOE_ERR_UNSUPPORTED, nothing enqueued
