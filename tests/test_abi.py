"""The C ABI of libmoe_fp8.so, checked on the CPU: the library loads, exports
every function include/moe_fp8.h declares, and rejects invalid arguments with
the documented status before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_fp8.h")
LIB = os.path.join(ROOT, "fp8_block_scaled_sigmoid_amd", "libmoe_fp8.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoe_fp8.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_layer_calls():
    names = declared_functions()
    for n in ["moe_route_topk", "moe_route_topk_quant_x", "moe_route_topk_fp8",
              "moe_route_workspace_bytes",
              "moe_topk_from_scores", "moe_permute",
              "moe_permute_workspace_bytes", "fp8_quant_1x128", "fp8_quant_128x128",
              "moe_grouped_gemm_fp8", "moe_grouped_gemm_fp8_tiles", "moe_combine", "moe_bias_update", "moe_status_str",
              "moe_last_hip_error", "fp8_transpose_128x128", "fp8_quant_tokens_128",
              "moe_grouped_wgrad_fp8"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in moe_fp8.h but not exported"


def test_status_strings(lib):
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [ctypes.c_int]
    assert lib.moe_status_str(0) == b"MOE_OK"
    for c in range(1, 8):
        assert lib.moe_status_str(c).startswith(b"MOE_ERR_")


def test_validation_before_any_launch(lib):
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.moe_permute.argtypes = [P, I, I, I, I, P, P, P, P, P, ctypes.c_size_t, P]
    # N out of range, k out of range -> shape error
    assert lib.moe_permute(None, 4, 0, 2, 1, None, None, None, None, None, 0, None) == 2
    assert lib.moe_permute(None, 4, 8, 33, 1, None, None, None, None, None, 0, None) == 2
    dummy = ctypes.c_void_p(16)
    # missing workspace
    assert lib.moe_permute(dummy, 4, 8, 2, 1, dummy, dummy, dummy, dummy, None, 0, None) == 4
    lib.fp8_quant_1x128.argtypes = [P, I, I, I, I, P, P, P]
    assert lib.fp8_quant_1x128(None, 0, 4, 100, 100, None, None, None) == 2     # cols % 128
    assert lib.fp8_quant_1x128(None, 0, 0, 128, 128, None, None, None) == 0     # empty: no-op
    assert lib.fp8_quant_1x128(None, 0, 4, 128, 128, None, None, None) == 1     # NULL
    assert lib.fp8_quant_1x128(ctypes.c_void_p(8), 0, 4, 128, 128, dummy, dummy, None) == 3
    lib.moe_route_topk.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, ctypes.c_size_t, P]
    R = lambda T, H, N, k, G=1, M=1, x=None, ws=None: lib.moe_route_topk(  # noqa: E731
        x, x, x, T, H, N, k, G, M, None, x, x, ws, 0, None)
    assert R(4, 256, 257, 8) == 2
    assert R(4, 256, 16, 17) == 2
    assert R(0, 256, 16, 2) == 0
    # group-limited arguments: G must divide N, M <= G, M | k, k / M <= N / G
    assert R(4, 256, 256, 8, 3, 1) == 2
    assert R(4, 256, 256, 8, 8, 9) == 2
    assert R(4, 256, 256, 8, 8, 3) == 2
    assert R(4, 256, 16, 8, 8, 2) == 2            # 4 per group > 2 experts per group
    assert R(4, 256, 256, 8, 128, 4) == 2         # more than 64 groups
    assert R(0, 256, 256, 8, 8, 4) == 0
    # missing workspace (checked before any device access)
    assert R(4, 256, 16, 2, x=dummy) == 4
    assert R(4, 256, 256, 8, 8, 4, x=dummy) == 4
    lib.moe_route_topk_quant_x.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, P, P,
                                           ctypes.c_size_t, P]
    RQ = lambda T, H, N, k, x=None, q=None, ws=None: lib.moe_route_topk_quant_x(  # noqa: E731
        x, x, x, T, H, N, k, 1, 1, None, x, x, q, q, ws, 0, None)
    assert RQ(4, 200, 16, 2) == 2                 # H % 128
    assert RQ(4, 256, 257, 8) == 2
    assert RQ(0, 256, 16, 2) == 0
    assert RQ(4, 256, 16, 2, x=dummy) == 1        # no x_q / x_d
    assert RQ(4, 256, 16, 2, x=dummy, q=dummy) == 4   # missing workspace
    lib.moe_route_topk_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P, P, P, P,
                                       ctypes.c_size_t, P]
    R8 = lambda T, H, N, k, G=1, M=1, x=None, ws=None: lib.moe_route_topk_fp8(  # noqa: E731
        x, x, x, x, x, T, H, N, k, G, M, None, x, x, ws, 0, None)
    assert R8(4, 256, 16, 2) == 2                 # N below one 128-row weight block
    assert R8(4, 256, 192, 8) == 2                # N % 128
    assert R8(4, 200, 256, 8) == 2                # H % 128
    assert R8(4, 256, 256, 8, 8, 3) == 2
    assert R8(0, 256, 256, 8) == 0
    assert R8(4, 256, 256, 8) == 1                # NULL operands
    assert R8(4, 256, 256, 8, x=dummy) == 4       # missing workspace
    lib.moe_topk_from_scores.argtypes = [P, P, I, I, I, I, I, P, P, P]
    assert lib.moe_topk_from_scores(None, None, 4, 256, 8, 8, 3, None, None, None) == 2
    assert lib.moe_topk_from_scores(None, None, 0, 256, 8, 8, 4, None, None, None) == 0
    lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_route_workspace_bytes.argtypes = [I, I, I]
    # 8192 tokens of H 7168: 64 token tiles, 4 slices of the 112 chunks
    assert lib.moe_route_workspace_bytes(8192, 7168, 256) == 4 * 8192 * 256 * 4
    # 64 tokens of H 256: one token tile, one slice per 128-wide block of H
    assert lib.moe_route_workspace_bytes(64, 256, 16) == 2 * 64 * 16 * 4
    assert lib.moe_route_workspace_bytes(0, 256, 16) == 0
    lib.moe_combine.argtypes = [P, P, P, I, I, I, I, P, P, P]
    assert lib.moe_combine(None, None, None, 0, 4, 12, 2, None, None, None) == 2   # H % 8
    lib.moe_bias_update.argtypes = [P, P, I, I, I, ctypes.c_float, P]
    assert lib.moe_bias_update(None, None, 4, 1, 1, 0.1, None) == 1
    lib.moe_seq_balance_loss.argtypes = [P, P, P, I, I, I, I, ctypes.c_float, P, P]
    assert lib.moe_seq_balance_loss(None, None, None, 2, 8, 2000, 2, 1e-4, None, None) == 2
    assert lib.moe_seq_balance_loss(None, None, None, 0, 8, 16, 2, 1e-4, None, None) == 0
    assert lib.moe_seq_balance_loss(None, None, dummy, 2, 8, 16, 2, 1e-4, dummy, None) == 1
    LL = ctypes.c_longlong
    lib.fp8_transpose_128x128.argtypes = [P, P, I, I, I, P, P, P]
    assert lib.fp8_transpose_128x128(None, None, 1, 100, 128, None, None, None) == 2
    assert lib.fp8_transpose_128x128(None, None, 0, 128, 128, None, None, None) == 0
    assert lib.fp8_transpose_128x128(None, None, 1, 128, 128, None, None, None) == 1
    assert lib.fp8_transpose_128x128(ctypes.c_void_p(8), dummy, 1, 128, 128, dummy, dummy, None) == 3
    lib.fp8_quant_tokens_128.argtypes = [P, I, I, I, LL, P, I, P, P, LL, P, P]
    assert lib.fp8_quant_tokens_128(None, 0, 300, 100, 100, None, 2, None, None, 640, None, None) == 2  # cols % 64
    assert lib.fp8_quant_tokens_128(None, 0, 300, 64, 64, None, 2, None, None, 512, None, None) == 2   # ldt too small
    assert lib.fp8_quant_tokens_128(None, 0, 300, 64, 64, None, 2, None, None, 640, None, None) == 1   # NULL offsets
    assert lib.fp8_quant_tokens_128(None, 2, 300, 64, 64, dummy, 2, None, None, 640, dummy, None) == 6  # dtype
    lib.moe_grouped_wgrad_fp8.argtypes = [P, P, LL, I, P, P, LL, I, P, I, P, P]
    assert lib.moe_grouped_wgrad_fp8(None, None, 256, 100, None, None, 256, 128, None, 2, None, None) == 2
    assert lib.moe_grouped_wgrad_fp8(None, None, 200, 128, None, None, 256, 128, None, 2, None, None) == 2
    assert lib.moe_grouped_wgrad_fp8(None, None, 256, 128, None, None, 256, 128, None, 2, None, None) == 1
    assert lib.moe_grouped_wgrad_fp8(None, None, 256, 0, None, None, 256, 128, None, 2, None, None) == 0
    # the MFMA rate probe: shape first, then the sink pointer
    lib.moe_probe_fp8_mfma.argtypes = [I, I, P, P]
    assert lib.moe_probe_fp8_mfma(0, 10, None, None) == 2
    assert lib.moe_probe_fp8_mfma(4, 0, None, None) == 2
    assert lib.moe_probe_fp8_mfma(4, 10, None, None) == 1
    # the HBM rate probe: mode and size, then pointers, then alignment
    lib.moe_probe_hbm.argtypes = [I, P, ctypes.c_size_t, P, P]
    assert lib.moe_probe_hbm(4, dummy, 1024, dummy, None) == 2
    assert lib.moe_probe_hbm(-1, dummy, 1024, dummy, None) == 2
    assert lib.moe_probe_hbm(2, dummy, 1024, None, None) == 1
    assert lib.moe_probe_hbm(0, dummy, 1000, dummy, None) == 2
    assert lib.moe_probe_hbm(0, None, 1024, dummy, None) == 1
    assert lib.moe_probe_hbm(0, dummy, 1024, None, None) == 1
    assert lib.moe_probe_hbm(1, ctypes.c_void_p(8), 1024, None, None) == 3
    assert lib.moe_probe_hbm(1, dummy, 0, None, None) == 0
    lib.moe_permute_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_permute_workspace_bytes.argtypes = [I, I, I]
    assert lib.moe_permute_workspace_bytes(513, 256, 8) == 3 * 256 * 4


class GemmArgs(ctypes.Structure):
    _fields_ = [("a_q", ctypes.c_void_p), ("a_d", ctypes.c_void_p), ("lda", ctypes.c_int),
                ("a_rows", ctypes.c_int), ("a_row_index", ctypes.c_void_p),
                ("b_q", ctypes.c_void_p), ("b_d", ctypes.c_void_p),
                ("group_offsets", ctypes.c_void_p), ("num_groups", ctypes.c_int),
                ("total_rows", ctypes.c_int), ("n_out", ctypes.c_int), ("k_dim", ctypes.c_int),
                ("epilogue", ctypes.c_int), ("out", ctypes.c_void_p), ("out_d", ctypes.c_void_p),
                ("ldo", ctypes.c_int), ("row_scale", ctypes.c_void_p)]


def test_gemm_validation(lib):
    lib.moe_grouped_gemm_fp8.argtypes = [ctypes.POINTER(GemmArgs), ctypes.c_void_p]
    assert lib.moe_grouped_gemm_fp8(None, None) == 1
    a = GemmArgs(16, 16, 256, 8, None, 16, 16, 16, 3, 8, 256, 256, 0, 16, None, 256, None)
    a.k_dim = 200
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 2   # K % 128
    a.k_dim, a.n_out = 256, 320
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 2   # n_out % 128
    a.n_out, a.epilogue, a.out_d = 384, 1, 16
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 2   # SwiGLU needs n_out % 256
    a.out_d = None
    a.n_out, a.epilogue = 256, 9
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 6
    a.epilogue, a.ldo = 0, (1 << 22) + 8
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 6   # bf16 row stride too long
    a.ldo = 256
    a.epilogue, a.total_rows = 0, 0
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 0   # nothing to do
    a.total_rows, a.epilogue, a.out_d = 8, 1, None
    assert lib.moe_grouped_gemm_fp8(ctypes.byref(a), None) == 1   # SwiGLU needs out_d


def test_gemm_tiles_validation(lib):
    f = lib.moe_grouped_gemm_fp8_tiles
    f.argtypes = [ctypes.POINTER(GemmArgs), ctypes.c_int, ctypes.c_void_p]
    assert f(None, 0, None) == 1
    a = GemmArgs(16, 16, 256, 8, None, 16, 16, 16, 3, 8, 256, 256, 0, 16, None, 256, None)
    for bad in (-1, 1, 64, 192, 512):
        assert f(ctypes.byref(a), bad, None) == 6, bad          # no such row tile
    a.epilogue = 2
    assert f(ctypes.byref(a), 256, None) == 6                   # 256 rows: not with float32 out
    a.epilogue, a.n_out = 0, 384
    assert f(ctypes.byref(a), 256, None) == 6                   # bf16 256 rows: n_out % 256
    a.n_out, a.ldo = 256, (1 << 21) + 8
    assert f(ctypes.byref(a), 256, None) == 6                   # bf16 256 rows: ldo <= 2^21
    a.ldo = 256
    a.epilogue, a.out_d = 1, None
    for t in (0, 128, 256):
        assert f(ctypes.byref(a), t, None) == 1, t              # the other checks still apply
    a.out_d, a.n_out = 16, 384
    assert f(ctypes.byref(a), 256, None) == 2                   # n_out % 256
    a.n_out, a.total_rows = 256, 0
    assert f(ctypes.byref(a), 256, None) == 0                   # nothing to do


def _layer_args(**kw):
    from fp8_block_scaled_sigmoid_amd import LayerArgs
    a = dict(x=16, w_router=16, w_router_q=None, w_router_d=None, bias=16, w1_q=16, w1_d=16,
             w2_q=16, w2_d=16, T=8, H=256, N=16, k=2, I=128, with_shared=1, n_groups=1,
             topk_groups=1, router_fp8=0, update_bias=1, gamma=1e-3, residual=None, y=16,
             scores=None, topk_idx=None, topk_gate=None, counts=None)
    a.update(kw)
    return LayerArgs(**a)


def test_layer_workspace_bytes(lib):
    lib.moe_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_layer_workspace_bytes.argtypes = [ctypes.c_int] * 6
    T, H, N, k, I = 300, 512, 32, 4, 256
    R = T * k + T
    got = lib.moe_layer_workspace_bytes(T, H, N, k, I, 1)
    parts = (3 * T * k * 4 + N * 4 + (N + 2) * 4 + R * 4 + T * H + T * (H // 128) * 4 + R * I
             + R * (I // 128) * 4 + R * H * 2)
    assert parts <= got <= parts + 15 * 256 + 4 * T * N * 64
    assert got % 256 == 0
    assert lib.moe_layer_workspace_bytes(T, H, N, k, I, 0) < got          # no shared rows
    assert lib.moe_layer_workspace_bytes(T, 500, N, k, I, 1) == 0         # H % 128
    assert lib.moe_layer_workspace_bytes(T, H, N, k, 100, 1) == 0         # I % 128
    assert lib.moe_layer_workspace_bytes(0, H, N, k, I, 1) > 0            # counts, offsets


def test_layer_validation_before_any_launch(lib):
    P = ctypes.c_void_p
    from fp8_block_scaled_sigmoid_amd import LayerArgs
    lib.moe_layer_forward.argtypes = [ctypes.POINTER(LayerArgs), P, ctypes.c_size_t, P]
    lib.moe_layer_forward.restype = ctypes.c_int
    lib.moe_layer_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_layer_workspace_bytes.argtypes = [ctypes.c_int] * 6
    need = lib.moe_layer_workspace_bytes(8, 256, 16, 2, 128, 1)
    ws = P(4096)

    def call(a, ws=ws, n=need):
        return lib.moe_layer_forward(ctypes.byref(a), ws, n, None)

    assert lib.moe_layer_forward(None, ws, need, None) == 1             # MOE_ERR_NULL
    assert call(_layer_args(H=200)) == 2                                  # MOE_ERR_SHAPE
    assert call(_layer_args(I=100)) == 2
    assert call(_layer_args(N=8)) == 2
    assert call(_layer_args(k=17)) == 2                                   # k > N
    assert call(_layer_args(router_fp8=1, w_router_q=16, w_router_d=16)) == 2   # N < 128
    assert call(_layer_args(n_groups=3)) == 2                             # N % groups
    assert call(_layer_args(n_groups=4, topk_groups=2, k=3)) == 2         # k % topk_groups
    assert call(_layer_args(T=1 << 20, H=2048)) == 6                      # MOE_ERR_UNSUPPORTED
    assert call(_layer_args(bias=None)) == 1
    assert call(_layer_args(w_router=None)) == 1
    assert call(_layer_args(router_fp8=1, N=128)) == 1                    # no FP8 router weight
    assert call(_layer_args(y=None)) == 1
    assert call(_layer_args(), ws=None) == 4                              # MOE_ERR_WORKSPACE
    assert call(_layer_args(), n=need - 1) == 4
    assert call(_layer_args(), ws=P(4096 + 16)) == 3                      # MOE_ERR_ALIGN
    assert call(_layer_args(x=24)) == 3
    assert call(_layer_args(w1_q=8)) == 3
