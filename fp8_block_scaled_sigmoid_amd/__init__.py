"""Python binding of libmoe_fp8.so: the DeepSeekMoE forward layer on MI355X.

Argument marshalling only.  Every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/moe_fp8.h``; PyTorch is used for device
memory and the current stream, nothing else.  There is no fallback: if the
library is missing or the device is not gfx950 the calls raise.

The functions carry the C entry points' names.  ``MoELayer`` chains them into
the forward pass (router + biased top-k, permutation, 1x128 activation
quantisation, the two grouped FP8 GEMMs, combine, bias update);
``moe_layer_forward`` runs the same steps in one library call.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")

MOE_BF16, MOE_F32 = 0, 1
MOE_EPI_BF16, MOE_EPI_SWIGLU_FP8, MOE_EPI_F32 = 0, 1, 2

STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN",
          4: "MOE_ERR_WORKSPACE", 5: "MOE_ERR_DEVICE", 6: "MOE_ERR_UNSUPPORTED",
          7: "MOE_ERR_HIP"}


class MoeError(RuntimeError):
    def __init__(self, fn, code, hip=0):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}"
                         + (f" (hipError {hip})" if code == 7 else ""))
        self.code = code


class GemmArgs(ctypes.Structure):
    _fields_ = [("a_q", ctypes.c_void_p), ("a_d", ctypes.c_void_p), ("lda", ctypes.c_int),
                ("a_rows", ctypes.c_int), ("a_row_index", ctypes.c_void_p),
                ("b_q", ctypes.c_void_p), ("b_d", ctypes.c_void_p),
                ("group_offsets", ctypes.c_void_p), ("num_groups", ctypes.c_int),
                ("total_rows", ctypes.c_int), ("n_out", ctypes.c_int), ("k_dim", ctypes.c_int),
                ("epilogue", ctypes.c_int), ("out", ctypes.c_void_p), ("out_d", ctypes.c_void_p),
                ("ldo", ctypes.c_int), ("row_scale", ctypes.c_void_p)]


class LayerArgs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("w_router", ctypes.c_void_p),
                ("w_router_q", ctypes.c_void_p), ("w_router_d", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("w1_q", ctypes.c_void_p), ("w1_d", ctypes.c_void_p),
                ("w2_q", ctypes.c_void_p), ("w2_d", ctypes.c_void_p),
                ("T", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int), ("k", ctypes.c_int),
                ("I", ctypes.c_int), ("with_shared", ctypes.c_int), ("n_groups", ctypes.c_int),
                ("topk_groups", ctypes.c_int), ("router_fp8", ctypes.c_int),
                ("update_bias", ctypes.c_int), ("gamma", ctypes.c_float),
                ("residual", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("scores", ctypes.c_void_p), ("topk_idx", ctypes.c_void_p),
                ("topk_gate", ctypes.c_void_p), ("counts", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong


def lib():
    """Load libmoe_fp8.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "moe_route_topk": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, ctypes.c_size_t, _P],
            "moe_route_topk_quant_x": [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P],
            "moe_route_topk_fp8": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                   ctypes.c_size_t, _P],
            "moe_topk_from_scores": [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P],
            "moe_permute": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
            "fp8_quant_1x128": [_P, _I, _I, _I, _I, _P, _P, _P],
            "fp8_quant_128x128": [_P, _I, _I, _I, _I, _P, _P, _P],
            "moe_grouped_gemm_fp8": [ctypes.POINTER(GemmArgs), _P],
            "moe_grouped_gemm_fp8_tiles": [ctypes.POINTER(GemmArgs), _I, _P],
            "moe_combine": [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P],
            "moe_bias_update": [_P, _P, _I, _I, _I, ctypes.c_float, _P],
            "moe_seq_balance_loss": [_P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P],
            "fp8_transpose_128x128": [_P, _P, _I, _I, _I, _P, _P, _P],
            "fp8_quant_tokens_128": [_P, _I, _I, _I, _LL, _P, _I, _P, _P, _LL, _P, _P],
            "moe_grouped_wgrad_fp8": [_P, _P, _LL, _I, _P, _P, _LL, _I, _P, _I, _P, _P],
            "moe_probe_fp8_mfma": [_I, _I, _P, _P],
            "moe_probe_hbm": [_I, _P, ctypes.c_size_t, _P, _P],
            "moe_permute_noalloc": [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P],
            "moe_layer_forward": [ctypes.POINTER(LayerArgs), _P, ctypes.c_size_t, _P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.moe_permute_workspace_bytes.argtypes = [_I, _I, _I]
        L.moe_permute_workspace_bytes.restype = ctypes.c_size_t
        L.moe_route_workspace_bytes.argtypes = [_I, _I, _I]
        L.moe_route_workspace_bytes.restype = ctypes.c_size_t
        L.moe_permute_noalloc_max_scratch_bytes.argtypes = []
        L.moe_permute_noalloc_max_scratch_bytes.restype = ctypes.c_size_t
        L.moe_layer_workspace_bytes.argtypes = [_I, _I, _I, _I, _I, _I]
        L.moe_layer_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_str.argtypes = [_I]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_hip_error.argtypes = []
        L.moe_last_hip_error.restype = ctypes.c_int
        _lib = L
    return _lib


def _check(name, rc):
    if rc != 0:
        raise MoeError(name, rc, lib().moe_last_hip_error() if rc == 7 else 0)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name):
    if not (t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise ValueError(f"{name}: need a contiguous {dtype} device tensor, got "
                         f"{t.dtype} on {t.device} (contiguous={t.is_contiguous()})")
    return t


# ---------------------------------------------------------------------------
# the C entry points


def moe_route_workspace_bytes(T, H, N):
    return int(lib().moe_route_workspace_bytes(T, H, N))


def moe_route_topk(x, w_router, bias, k, scores=True, idx=None, gate=None, ws=None,
                   n_groups=1, topk_groups=1, stream=None):
    """Sigmoid router + biased top-k.  x [T,H] bf16, w_router [N,H] bf16,
    bias [N] float32.  Returns (idx int32 [T,k], gate float32 [T,k],
    scores float32 [T,N] or None).  ws: optional uint8 device scratch of
    moe_route_workspace_bytes(T, H, N) bytes.  n_groups > 1 turns on the
    group-limited selection (the best topk_groups groups are eligible)."""
    T, H = x.shape
    N = w_router.shape[0]
    _dev(x, torch.bfloat16, "x"), _dev(w_router, torch.bfloat16, "w_router")
    _dev(bias, torch.float32, "bias")
    if scores is True:
        scores = torch.empty(T, N, dtype=torch.float32, device=x.device)
    elif scores is False:
        scores = None
    idx = torch.empty(T, k, dtype=torch.int32, device=x.device) if idx is None else idx
    gate = torch.empty(T, k, dtype=torch.float32, device=x.device) if gate is None else gate
    if ws is None:
        ws = torch.empty(max(moe_route_workspace_bytes(T, H, N), 16), dtype=torch.uint8,
                         device=x.device)
    _check("moe_route_topk", lib().moe_route_topk(_ptr(x), _ptr(w_router), _ptr(bias), T, H, N, k,
                                                  n_groups, topk_groups, _ptr(scores), _ptr(idx),
                                                  _ptr(gate), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, gate, scores


def moe_route_topk_quant_x(x, w_router, bias, k, x_q=None, x_d=None, scores=True, idx=None,
                           gate=None, ws=None, n_groups=1, topk_groups=1, stream=None):
    """moe_route_topk that also writes the 1x128 FP8 quantisation of x (the
    codes and scales fp8_quant_1x128 gives) from the same read of x.
    Returns (idx, gate, scores, x_q uint8 [T,H], x_d float32 [T,H/128])."""
    T, H = x.shape
    N = w_router.shape[0]
    _dev(x, torch.bfloat16, "x"), _dev(w_router, torch.bfloat16, "w_router")
    _dev(bias, torch.float32, "bias")
    if scores is True:
        scores = torch.empty(T, N, dtype=torch.float32, device=x.device)
    elif scores is False:
        scores = None
    idx = torch.empty(T, k, dtype=torch.int32, device=x.device) if idx is None else idx
    gate = torch.empty(T, k, dtype=torch.float32, device=x.device) if gate is None else gate
    x_q = torch.empty(T, H, dtype=torch.uint8, device=x.device) if x_q is None else x_q
    x_d = torch.empty(T, H // 128, dtype=torch.float32, device=x.device) if x_d is None else x_d
    _dev(x_q, torch.uint8, "x_q"), _dev(x_d, torch.float32, "x_d")
    if ws is None:
        ws = torch.empty(max(moe_route_workspace_bytes(T, H, N), 16), dtype=torch.uint8,
                         device=x.device)
    _check("moe_route_topk_quant_x",
           lib().moe_route_topk_quant_x(_ptr(x), _ptr(w_router), _ptr(bias), T, H, N, k, n_groups,
                                        topk_groups, _ptr(scores), _ptr(idx), _ptr(gate),
                                        _ptr(x_q), _ptr(x_d), _ptr(ws), ws.numel(),
                                        _stream(stream)))
    return idx, gate, scores, x_q, x_d


def moe_route_topk_fp8(x_q, x_d, w_router_q, w_router_d, bias, k, scores=True, idx=None,
                       gate=None, ws=None, n_groups=1, topk_groups=1, stream=None):
    """Opt-in FP8 router + biased top-k.  x_q uint8 [T,H] with x_d float32
    [T,H/128] (fp8_quant_1x128), w_router_q uint8 [N,H] with w_router_d float32
    [N/128,H/128] (fp8_quant_128x128), bias [N] float32.  Same outputs and
    workspace as moe_route_topk."""
    T, H = x_q.shape
    N = w_router_q.shape[-2]
    _dev(x_q, torch.uint8, "x_q"), _dev(x_d, torch.float32, "x_d")
    _dev(w_router_q, torch.uint8, "w_router_q"), _dev(w_router_d, torch.float32, "w_router_d")
    _dev(bias, torch.float32, "bias")
    if scores is True:
        scores = torch.empty(T, N, dtype=torch.float32, device=x_q.device)
    elif scores is False:
        scores = None
    idx = torch.empty(T, k, dtype=torch.int32, device=x_q.device) if idx is None else idx
    gate = torch.empty(T, k, dtype=torch.float32, device=x_q.device) if gate is None else gate
    if ws is None:
        ws = torch.empty(max(moe_route_workspace_bytes(T, H, N), 16), dtype=torch.uint8,
                         device=x_q.device)
    _check("moe_route_topk_fp8",
           lib().moe_route_topk_fp8(_ptr(x_q), _ptr(x_d), _ptr(w_router_q), _ptr(w_router_d),
                                    _ptr(bias), T, H, N, k, n_groups, topk_groups, _ptr(scores),
                                    _ptr(idx), _ptr(gate), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return idx, gate, scores


def moe_topk_from_scores(scores, bias, k, idx=None, gate=None, n_groups=1, topk_groups=1,
                         stream=None):
    T, N = scores.shape
    _dev(scores, torch.float32, "scores"), _dev(bias, torch.float32, "bias")
    idx = torch.empty(T, k, dtype=torch.int32, device=scores.device) if idx is None else idx
    gate = torch.empty(T, k, dtype=torch.float32, device=scores.device) if gate is None else gate
    _check("moe_topk_from_scores", lib().moe_topk_from_scores(
        _ptr(scores), _ptr(bias), T, N, k, n_groups, topk_groups, _ptr(idx), _ptr(gate),
        _stream(stream)))
    return idx, gate


def moe_permute_workspace_bytes(T, N, k):
    return int(lib().moe_permute_workspace_bytes(T, N, k))


def moe_permute(idx, N, with_shared=True, out=None, ws=None, stream=None):
    """idx int32 [T,k] -> (counts [N], offsets [N+2], row_of [T,k],
    token_of [T*k (+T)]), all int32."""
    T, k = idx.shape
    _dev(idx, torch.int32, "idx")
    dev = idx.device
    if out is None:
        R = T * k + (T if with_shared else 0)
        out = (torch.empty(N, dtype=torch.int32, device=dev),
               torch.empty(N + 2, dtype=torch.int32, device=dev),
               torch.empty(T, k, dtype=torch.int32, device=dev),
               torch.empty(R, dtype=torch.int32, device=dev))
    counts, offsets, row_of, token_of = out
    nbytes = moe_permute_workspace_bytes(T, N, k)
    if ws is None:
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _check("moe_permute", lib().moe_permute(_ptr(idx), T, N, k, 1 if with_shared else 0,
                                            _ptr(counts), _ptr(offsets), _ptr(row_of),
                                            _ptr(token_of), _ptr(ws), ws.numel(),
                                            _stream(stream)))
    return counts, offsets, row_of, token_of


def moe_permute_noalloc_max_scratch_bytes():
    return int(lib().moe_permute_noalloc_max_scratch_bytes())


def moe_permute_noalloc(idx, N, with_shared, out, stream=None):
    """moe_permute without a workspace (the library's own device scratch, for
    callers that cannot allocate): writes into the caller's ``out`` tensors
    (counts [N], offsets [N+2], row_of [T,k], token_of [T*k (+T)], int32)."""
    T, k = idx.shape
    _dev(idx, torch.int32, "idx")
    counts, offsets, row_of, token_of = out
    _check("moe_permute_noalloc", lib().moe_permute_noalloc(
        _ptr(idx), T, N, k, 1 if with_shared else 0, _ptr(counts), _ptr(offsets), _ptr(row_of),
        _ptr(token_of), _stream(stream)))
    return counts, offsets, row_of, token_of


def fp8_quant_1x128(x, q=None, d=None, stream=None):
    """x [rows, cols] bf16 or float32 -> (q uint8 [rows, cols], d float32 [rows, cols/128])."""
    rows, cols = x.shape
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[x.dtype]
    if x.stride(1) != 1:
        raise ValueError("x: rows must be contiguous")
    q = torch.empty(rows, cols, dtype=torch.uint8, device=x.device) if q is None else q
    d = torch.empty(rows, cols // 128, dtype=torch.float32, device=x.device) if d is None else d
    _check("fp8_quant_1x128", lib().fp8_quant_1x128(_ptr(x), dt, rows, cols, x.stride(0), _ptr(q),
                                                    _ptr(d), _stream(stream)))
    return q, d


def fp8_quant_128x128(w, interleave_gate_up=False, q=None, d=None, stream=None):
    """w [batch, rows, cols] bf16 -> (q uint8 like w, d float32 [batch, rows/128, cols/128])."""
    if w.dim() == 2:
        w = w.unsqueeze(0)
    B, rows, cols = w.shape
    _dev(w, torch.bfloat16, "w")
    q = torch.empty(B, rows, cols, dtype=torch.uint8, device=w.device) if q is None else q
    d = torch.empty(B, rows // 128, cols // 128, dtype=torch.float32, device=w.device) \
        if d is None else d
    _check("fp8_quant_128x128", lib().fp8_quant_128x128(_ptr(w), B, rows, cols,
                                                        1 if interleave_gate_up else 0, _ptr(q),
                                                        _ptr(d), _stream(stream)))
    return q, d


def moe_grouped_gemm_fp8(a_q, a_d, b_q, b_d, group_offsets, total_rows, epilogue,
                         a_row_index=None, out=None, out_d=None, row_scale=None, stream=None,
                         tile_rows=None):
    """Grouped block-scaled FP8 GEMM (see include/moe_fp8.h).  b_q [G, n_out, K].
    tile_rows None calls moe_grouped_gemm_fp8 (the library picks the row tile);
    0, 128 or 256 calls moe_grouped_gemm_fp8_tiles with it."""
    G, n_out, K = b_q.shape
    dev = a_q.device
    if out is None:
        if epilogue == MOE_EPI_SWIGLU_FP8:
            out = torch.empty(total_rows, n_out // 2, dtype=torch.uint8, device=dev)
            out_d = torch.empty(total_rows, n_out // 256, dtype=torch.float32, device=dev)
        elif epilogue == MOE_EPI_BF16:
            out = torch.empty(total_rows, n_out, dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty(total_rows, n_out, dtype=torch.float32, device=dev)
    args = GemmArgs(a_q.data_ptr(), a_d.data_ptr(), a_q.stride(0), a_q.shape[0],
                    a_row_index.data_ptr() if a_row_index is not None else None,
                    b_q.data_ptr(), b_d.data_ptr(), group_offsets.data_ptr(), G, total_rows,
                    n_out, K, epilogue, out.data_ptr(),
                    out_d.data_ptr() if out_d is not None else None, out.stride(0),
                    row_scale.data_ptr() if row_scale is not None else None)
    if tile_rows is None:
        _check("moe_grouped_gemm_fp8", lib().moe_grouped_gemm_fp8(ctypes.byref(args), _stream(stream)))
    else:
        _check("moe_grouped_gemm_fp8_tiles",
               lib().moe_grouped_gemm_fp8_tiles(ctypes.byref(args), int(tile_rows), _stream(stream)))
    return out, out_d


def fp8_transpose_128x128(w_q, w_d, wt_q=None, wt_d=None, stream=None):
    """Exact transpose of 128x128 block-quantised weights: w_q uint8
    [B, rows, cols], w_d float32 [B, rows/128, cols/128] -> (wt_q [B, cols,
    rows], wt_d [B, cols/128, rows/128]).  The B operand of Dgrad."""
    if w_q.dim() == 2:
        w_q, w_d = w_q.unsqueeze(0), w_d.unsqueeze(0)
    B, rows, cols = w_q.shape
    _dev(w_q, torch.uint8, "w_q"), _dev(w_d, torch.float32, "w_d")
    dev = w_q.device
    wt_q = torch.empty(B, cols, rows, dtype=torch.uint8, device=dev) if wt_q is None else wt_q
    wt_d = torch.empty(B, cols // 128, rows // 128, dtype=torch.float32, device=dev) \
        if wt_d is None else wt_d
    _check("fp8_transpose_128x128", lib().fp8_transpose_128x128(
        _ptr(w_q), _ptr(w_d), B, rows, cols, _ptr(wt_q), _ptr(wt_d), _stream(stream)))
    return wt_q, wt_d


def tokens_padded_width(rows, num_groups):
    """Row stride (bytes) that holds any token-tile layout of `rows` tokens in
    `num_groups` groups: a multiple of 128, at least rows + 127 * num_groups."""
    return (rows + 127 * num_groups + 127) // 128 * 128


def fp8_quant_tokens_128(x, group_offsets, ldt=None, xt_q=None, xt_d=None, pad_offsets=None,
                         stream=None):
    """Token-tile quantiser (Wgrad operands).  x [rows, cols] bf16 or float32
    in expert-grouped row order, group_offsets int32 [G+1] -> (xt_q uint8
    [cols, ldt], xt_d float32 [cols, ldt/128], pad_offsets int32 [G+1])."""
    rows, cols = x.shape
    G = group_offsets.numel() - 1
    dt = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[x.dtype]
    if x.stride(1) != 1:
        raise ValueError("x: rows must be contiguous")
    _dev(group_offsets, torch.int32, "group_offsets")
    ldt = tokens_padded_width(rows, G) if ldt is None else ldt
    dev = x.device
    xt_q = torch.empty(cols, ldt, dtype=torch.uint8, device=dev) if xt_q is None else xt_q
    xt_d = torch.empty(cols, ldt // 128, dtype=torch.float32, device=dev) if xt_d is None else xt_d
    pad_offsets = torch.empty(G + 1, dtype=torch.int32, device=dev) if pad_offsets is None \
        else pad_offsets
    _check("fp8_quant_tokens_128", lib().fp8_quant_tokens_128(
        _ptr(x), dt, rows, cols, x.stride(0), _ptr(group_offsets), G, _ptr(xt_q), _ptr(xt_d),
        ldt, _ptr(pad_offsets), _stream(stream)))
    return xt_q, xt_d, pad_offsets


def moe_grouped_wgrad_fp8(a_q, a_d, b_q, b_d, pad_offsets, out=None, stream=None):
    """Wgrad grouped GEMM: out[g] = dY_g^T X_g (float32 [G, N, K]) from the
    token-tile operands a (dY^T, [N, lda]) and b (X^T, [K, ldb])."""
    N, lda = a_q.shape
    K, ldb = b_q.shape
    G = pad_offsets.numel() - 1
    for t, dt, n in ((a_q, torch.uint8, "a_q"), (a_d, torch.float32, "a_d"),
                     (b_q, torch.uint8, "b_q"), (b_d, torch.float32, "b_d"),
                     (pad_offsets, torch.int32, "pad_offsets")):
        _dev(t, dt, n)
    out = torch.empty(G, N, K, dtype=torch.float32, device=a_q.device) if out is None else out
    _check("moe_grouped_wgrad_fp8", lib().moe_grouped_wgrad_fp8(
        _ptr(a_q), _ptr(a_d), lda, N, _ptr(b_q), _ptr(b_d), ldb, K, _ptr(pad_offsets), G,
        _ptr(out), _stream(stream)))
    return out


def moe_grouped_dgrad_fp8(dy, wt_q, wt_d, group_offsets, epilogue=MOE_EPI_BF16, dy_q=None,
                          dy_d=None, out=None, stream=None):
    """Dgrad: dX = dY W per group.  dy [R, N] bf16 or float32 (grouped rows),
    wt_q/wt_d the transposed weights from fp8_transpose_128x128 ([G, K, N]).
    dY is quantised 1x128 (fp8_quant_1x128), then the grouped FP8 GEMM runs
    with the bf16 or float32 epilogue.  Returns dX [R, K]."""
    dy_q, dy_d = fp8_quant_1x128(dy, q=dy_q, d=dy_d, stream=stream)
    out, _ = moe_grouped_gemm_fp8(dy_q, dy_d, wt_q, wt_d, group_offsets, dy.shape[0], epilogue,
                                  out=out, stream=stream)
    return out


def moe_combine(out_rows, gate, row_of, shared_row0, residual=None, y=None, stream=None):
    T, k = row_of.shape
    H = out_rows.shape[1]
    y = torch.empty(T, H, dtype=torch.bfloat16, device=out_rows.device) if y is None else y
    _check("moe_combine", lib().moe_combine(_ptr(out_rows), _ptr(gate), _ptr(row_of), shared_row0,
                                            T, H, k, _ptr(residual), _ptr(y), _stream(stream)))
    return y


def moe_bias_update(bias, counts, T, k, gamma, stream=None):
    N = bias.shape[0]
    _check("moe_bias_update", lib().moe_bias_update(_ptr(bias), _ptr(counts), N, T, k,
                                                    float(gamma), _stream(stream)))
    return bias


def moe_seq_balance_loss(idx, gate, seq_offsets, n_experts, alpha=1e-4, loss=None, stream=None):
    """Sequence-wise balance statistic per sequence: idx int32 [T,k], gate
    float32 [T,k], seq_offsets int32 [S+1] (device) -> loss float32 [S]."""
    T, k = idx.shape
    _dev(idx, torch.int32, "idx"), _dev(gate, torch.float32, "gate")
    _dev(seq_offsets, torch.int32, "seq_offsets")
    S = seq_offsets.numel() - 1
    loss = torch.empty(max(S, 0), dtype=torch.float32, device=idx.device) if loss is None else loss
    _check("moe_seq_balance_loss", lib().moe_seq_balance_loss(
        _ptr(idx), _ptr(gate), _ptr(seq_offsets), S, T, n_experts, k, alpha, _ptr(loss),
        _stream(stream)))
    return loss


def moe_probe_fp8_mfma(blocks, iters, sink=None, stream=None):
    """Enqueue the FP8 MFMA rate probe (a diagnostic, not a layer step):
    blocks * 4 waves, each issuing iters * 16 16x16x128 FP8 MFMAs.  Returns
    (sink, flops)."""
    if sink is None:
        sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    _check("moe_probe_fp8_mfma", lib().moe_probe_fp8_mfma(blocks, iters, _ptr(sink),
                                                          _stream(stream)))
    return sink, float(blocks) * 4 * iters * 16 * 65536


def moe_probe_hbm(mode, buf, sink=None, stream=None):
    """Enqueue the HBM rate probe (a diagnostic, not a layer step): modes 0
    and 2 read every byte of the device tensor ``buf`` (non-temporal, eight
    loads in flight per lane; ordinary, four), modes 1 and 3 write them
    (non-temporal; ordinary stores).  Returns the sink (read modes) or None."""
    if mode in (0, 2) and sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check("moe_probe_hbm", lib().moe_probe_hbm(mode, _ptr(buf), buf.numel() * buf.element_size(),
                                                _ptr(sink), _stream(stream)))
    return sink


def moe_layer_workspace_bytes(T, H, N, k, I, with_shared=True):
    return int(lib().moe_layer_workspace_bytes(T, H, N, k, I, 1 if with_shared else 0))


def moe_layer_forward(w, x, k, gamma=1e-3, n_groups=1, topk_groups=1, router_fp8=False,
                      update_bias=True, residual=None, y=None, scores=None, idx=None, gate=None,
                      counts=None, ws=None, stream=None):
    """The whole forward pass in one library call (moe_layer_forward): w a
    MoEWeights, x [T,H] bf16.  Returns y [T,H] bf16.  scores / idx / gate /
    counts: optional device outputs.  ws: optional uint8 device workspace of
    moe_layer_workspace_bytes(...) bytes (allocated here when None)."""
    T, H = x.shape
    _dev(x, torch.bfloat16, "x"), _dev(w.bias, torch.float32, "bias")
    with_shared = w.G == w.N + 1
    if router_fp8 and w.w_router_q is None:
        raise ValueError("router_fp8 needs MoEWeights(..., router_fp8=True)")
    y = torch.empty(T, H, dtype=torch.bfloat16, device=x.device) if y is None else y
    if ws is None:
        ws = torch.empty(max(moe_layer_workspace_bytes(T, H, w.N, k, w.I, with_shared), 256),
                         dtype=torch.uint8, device=x.device)
    a = LayerArgs(x.data_ptr(), w.w_router.data_ptr(),
                  w.w_router_q.data_ptr() if w.w_router_q is not None else None,
                  w.w_router_d.data_ptr() if w.w_router_d is not None else None,
                  w.bias.data_ptr(), w.w1q.data_ptr(), w.w1d.data_ptr(), w.w2q.data_ptr(),
                  w.w2d.data_ptr(), T, H, w.N, k, w.I, 1 if with_shared else 0, n_groups,
                  topk_groups, 1 if router_fp8 else 0, 1 if update_bias else 0, float(gamma),
                  residual.data_ptr() if residual is not None else None, y.data_ptr(),
                  *[t.data_ptr() if t is not None else None for t in (scores, idx, gate, counts)])
    _check("moe_layer_forward", lib().moe_layer_forward(ctypes.byref(a), _ptr(ws), ws.numel(),
                                                        _stream(stream)))
    return y


# ---------------------------------------------------------------------------
# the layer


class MoEWeights:
    """Device weights of one layer: router [N,H] bf16, bias [N] float32, and
    FP8 experts quantised 128x128 from bf16 W1 [G,2I,H] (gate rows, then up
    rows) and W2 [G,H,I]; expert G-1 = N is the shared expert.  router_fp8
    also keeps the router quantised 128x128 for the opt-in FP8 router."""

    def __init__(self, w_router, bias, w1_bf16=None, w2_bf16=None, w1q=None, w1d=None,
                 w2q=None, w2d=None, router_fp8=False):
        self.w_router = w_router
        self.bias = bias
        self.w_router_q = self.w_router_d = None
        if router_fp8:   # the opt-in FP8 router: Wr quantised 128x128 as well
            q, d = fp8_quant_128x128(w_router)
            self.w_router_q, self.w_router_d = q[0], d[0]
        if w1_bf16 is not None:
            w1q, w1d = fp8_quant_128x128(w1_bf16, interleave_gate_up=True)
        if w2_bf16 is not None:
            w2q, w2d = fp8_quant_128x128(w2_bf16)
        self.w1q, self.w1d, self.w2q, self.w2d = w1q, w1d, w2q, w2d
        self.N, self.H = w_router.shape
        self.G = w1q.shape[0]
        self.I = w1q.shape[1] // 2


class MoELayer:
    """Buffers for a batch of T tokens and the forward pass over them.  All
    buffers are allocated once here; ``forward`` only enqueues kernels."""

    def __init__(self, weights, T, k, gamma=1e-3, device="cuda", n_groups=1, topk_groups=1,
                 router_fp8=False):
        w = weights
        self.w, self.T, self.k, self.gamma = w, T, k, gamma
        self.n_groups, self.topk_groups = n_groups, topk_groups
        if router_fp8 and w.w_router_q is None:
            raise ValueError("router_fp8 needs MoEWeights(..., router_fp8=True)")
        self.router_fp8 = router_fp8
        N, H, I = w.N, w.H, w.I
        self.with_shared = w.G == N + 1
        R = T * k + (T if self.with_shared else 0)
        self.R = R
        e = dict(device=device)
        self.scores = torch.empty(T, N, dtype=torch.float32, **e)
        self.idx = torch.empty(T, k, dtype=torch.int32, **e)
        self.gate = torch.empty(T, k, dtype=torch.float32, **e)
        self.counts = torch.empty(N, dtype=torch.int32, **e)
        self.offsets = torch.empty(N + 2, dtype=torch.int32, **e)
        self.row_of = torch.empty(T, k, dtype=torch.int32, **e)
        self.token_of = torch.empty(R, dtype=torch.int32, **e)
        self.ws = torch.empty(max(moe_permute_workspace_bytes(T, N, k), 16), dtype=torch.uint8, **e)
        self.route_ws = torch.empty(max(moe_route_workspace_bytes(T, H, N), 16), dtype=torch.uint8,
                                    **e)
        self.xq = torch.empty(T, H, dtype=torch.uint8, **e)
        self.xd = torch.empty(T, H // 128, dtype=torch.float32, **e)
        self.hq = torch.empty(R, I, dtype=torch.uint8, **e)
        self.hd = torch.empty(R, I // 128, dtype=torch.float32, **e)
        self.out_rows = torch.empty(R, H, dtype=torch.bfloat16, **e)
        self.y = torch.empty(T, H, dtype=torch.bfloat16, **e)

    # the individual steps, so that callers can time or replace one of them
    def route(self, x, stream=None):
        """Routing from x with the bf16 router, which also writes the 1x128
        quantisation of x into self.xq / self.xd from the same read of x; or,
        with the FP8 router, from the quantised x already there (quant_x runs
        first)."""
        if self.router_fp8:
            moe_route_topk_fp8(self.xq, self.xd, self.w.w_router_q, self.w.w_router_d,
                               self.w.bias, self.k, scores=self.scores, idx=self.idx,
                               gate=self.gate, ws=self.route_ws, n_groups=self.n_groups,
                               topk_groups=self.topk_groups, stream=stream)
            return
        moe_route_topk_quant_x(x, self.w.w_router, self.w.bias, self.k, x_q=self.xq, x_d=self.xd,
                               scores=self.scores, idx=self.idx, gate=self.gate,
                               ws=self.route_ws, n_groups=self.n_groups,
                               topk_groups=self.topk_groups, stream=stream)

    def permute(self, stream=None):
        moe_permute(self.idx, self.w.N, self.with_shared,
                    out=(self.counts, self.offsets, self.row_of, self.token_of), ws=self.ws,
                    stream=stream)

    def quant_x(self, x, stream=None):
        fp8_quant_1x128(x, q=self.xq, d=self.xd, stream=stream)

    def gemm1(self, stream=None):
        moe_grouped_gemm_fp8(self.xq, self.xd, self.w.w1q, self.w.w1d, self.offsets, self.R,
                             MOE_EPI_SWIGLU_FP8,
                             a_row_index=self.token_of, out=self.hq, out_d=self.hd, stream=stream)

    def gemm2(self, stream=None):
        moe_grouped_gemm_fp8(self.hq, self.hd, self.w.w2q, self.w.w2d, self.offsets, self.R,
                             MOE_EPI_BF16, out=self.out_rows, stream=stream)

    def combine(self, stream=None):
        moe_combine(self.out_rows, self.gate, self.row_of,
                    self.T * self.k if self.with_shared else -1, y=self.y, stream=stream)

    def bias_update(self, stream=None):
        moe_bias_update(self.w.bias, self.counts, self.T, self.k, self.gamma, stream=stream)

    def forward(self, x, update_bias=True, stream=None):
        """One forward pass of the layer over x [T,H] bf16; returns y [T,H]
        bf16 (a buffer of this object).  With update_bias the per-expert bias
        is updated from this batch's counts at the end."""
        if self.router_fp8:
            self.quant_x(x, stream)
        self.route(x, stream)
        self.permute(stream)
        self.gemm1(stream)
        self.gemm2(stream)
        self.combine(stream)
        if update_bias:
            self.bias_update(stream)
        return self.y
