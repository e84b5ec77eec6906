"""Seeded synthetic inputs for the DeepSeekMoE layer (host side).

This module produces input tensors only; it holds none of the layer's
arithmetic.  Both the CPU oracle and the GPU path are fed from it.  Large
tensors (hundreds of millions of weights) are generated on the device by
``synth/synth.hip``, which implements the same counter-based definition, so
that the host can regenerate any slice (one expert's weights, a few token rows)
bit-identically without materialising the whole tensor.

Definition (identical on host and device):
  * mix64: the SplitMix64 output function (Steele, Lea and Flood, "Fast
    splittable pseudorandom number generators", OOPSLA 2014):
        z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
        z *= 0x94D049BB133111EB; z ^= z >> 31            (all mod 2^64)
  * stream key of a tensor: key = mix64(seed * GOLDEN + tensor_id), with
    GOLDEN = 0x9E3779B97F4A7C15.
  * element i (flat row-major index in the logical tensor) draws two words
        w_j = mix64(key + (2 i + j + 1) * GOLDEN),   j = 0, 1
  * "normal": the eight 16-bit fields u_0..u_7 of (w_0, w_1) give the
    Irwin-Hall integer z = 2 * sum(u) - 8 * 65535 (|z| < 2^20, exact in
    float32); value = fl32(fl32(z) * c_col), c_col = fl32(std * col_mult /
    sd_z) with sd_z = sqrt(32 (65536^2 - 1) / 12).  Tails stop at 4.9 sd.
  * "uniform" on (-w, w): u = w_0 >> 40 (24 bits); value =
    fl32(fl32(2u + 1 - 2^24) * fl32(w * col_mult / 2^24)).
  * bf16 tensors round that float32 value to nearest even.
Each value is one exact integer conversion and one float32 multiply, so host
(NumPy) and device (HIP) agree bit for bit.
"""
import math
import os
import ctypes

import numpy as np

GOLDEN = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1
SD_Z = math.sqrt(32.0 * (65536.0 ** 2 - 1.0) / 12.0)

NORMAL = 0
UNIFORM = 1

# tensor ids
T_X, T_WR, T_BIAS, T_W1, T_W2, T_PERM, T_OUTLIER, T_SCORES, T_ROWS, T_GATES = range(1, 11)
# upstream gradients of the backward workload: d(layer output rows), d(GEMM1
# output), and the SwiGLU output h
T_DOUT, T_DA, T_H = range(11, 14)


def mix64_int(z):
    z &= MASK64
    z ^= z >> 30
    z = (z * M1) & MASK64
    z ^= z >> 27
    z = (z * M2) & MASK64
    z ^= z >> 31
    return z


def stream_key(seed, tensor_id):
    return mix64_int((int(seed) * GOLDEN + int(tensor_id)) & MASK64)


def _mix64_np(z):
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(M1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(M2)
    z = z ^ (z >> np.uint64(31))
    return z


def words(key, flat_index):
    """The two 64-bit words of each element index (uint64 arrays)."""
    i = np.asarray(flat_index, dtype=np.uint64)
    base = np.uint64(key) + (np.uint64(2) * i + np.uint64(1)) * np.uint64(GOLDEN)
    with np.errstate(over="ignore"):
        w0 = _mix64_np(base)
        w1 = _mix64_np(base + np.uint64(GOLDEN))
    return w0, w1


def normal_coef(std, col_mult=1.0):
    return np.float32(std * col_mult / SD_Z)


def uniform_coef(width, col_mult=1.0):
    return np.float32(width * col_mult / float(1 << 24))


def _values(key, flat_index, dist, coef):
    """float32 values; coef is a float32 scalar or an array broadcastable to
    flat_index (per-element multiplier)."""
    w0, w1 = words(key, flat_index)
    coef = np.asarray(coef, dtype=np.float32)
    if dist == NORMAL:
        m = np.uint64(0xFFFF)
        s = np.zeros(np.shape(w0), dtype=np.int64)
        for w in (w0, w1):
            for sh in (0, 16, 32, 48):
                s += ((w >> np.uint64(sh)) & m).astype(np.int64)
        z = (2 * s - 8 * 65535).astype(np.float32)          # exact
        return (z * coef).astype(np.float32)
    if dist == UNIFORM:
        u = (w0 >> np.uint64(40)).astype(np.int64)
        z = (2 * u + 1 - (1 << 24)).astype(np.float32)      # exact
        return (z * coef).astype(np.float32)
    raise ValueError(dist)


def f32_to_bf16_bits(f):
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Spec:
    """How one tensor is drawn: distribution, std or half-width, and optional
    per-column multipliers / constant columns (applied along the last axis)."""

    def __init__(self, tensor_id, shape, dist, param, col_mult=None, const_cols=None,
                 seed_offset=0, dtype="bf16"):
        self.tensor_id = tensor_id
        self.shape = tuple(int(s) for s in shape)
        self.dist = dist
        self.param = float(param)
        self.col_mult = col_mult          # float64 [cols] or None
        self.const_cols = const_cols      # dict col -> float (bf16-exact) or None
        self.seed_offset = seed_offset
        self.dtype = dtype

    def coef_cols(self):
        cols = self.shape[-1]
        mult = np.ones(cols) if self.col_mult is None else np.asarray(self.col_mult, np.float64)
        f = normal_coef if self.dist == NORMAL else uniform_coef
        return np.array([f(self.param, m) for m in mult], dtype=np.float32)


def generate(spec, seed, rows=None):
    """Host generation.  Returns float32 (dtype 'f32') or bf16 bit patterns
    (uint16) of the tensor, or of the given leading-flattened rows only
    (``rows`` indexes the tensor viewed as [-1, cols])."""
    key = stream_key(seed + spec.seed_offset, spec.tensor_id)
    cols = spec.shape[-1]
    nrows_total = int(np.prod(spec.shape[:-1])) if len(spec.shape) > 1 else 1
    row_ids = np.arange(nrows_total, dtype=np.int64) if rows is None \
        else np.asarray(rows, dtype=np.int64)
    coef = spec.coef_cols()
    out = np.empty((row_ids.size, cols), dtype=np.float32)
    chunk = max(1, (1 << 22) // cols)
    for r0 in range(0, row_ids.size, chunk):
        rr = row_ids[r0:r0 + chunk]
        flat = rr[:, None] * cols + np.arange(cols, dtype=np.int64)[None, :]
        out[r0:r0 + chunk] = _values(key, flat, spec.dist, coef[None, :])
    if spec.const_cols:
        for c, v in spec.const_cols.items():
            out[:, c] = np.float32(v)
    shape = spec.shape if rows is None else (row_ids.size, cols)
    out = out.reshape(shape)
    if spec.dtype == "bf16":
        return f32_to_bf16_bits(out)
    return out


def as_f64(bf16_bits):
    """bf16 bit patterns -> float64 values."""
    return bf16_bits_to_f32(bf16_bits).astype(np.float64)


# ---------------------------------------------------------------------------
# workloads


def _hash_order(seed, tensor_id, n):
    """A seeded permutation of range(n): indices sorted by their hash."""
    key = stream_key(seed, tensor_id)
    w0, _ = words(key, np.arange(n))
    return np.argsort(w0, kind="stable")


class Workload:
    """Shapes and input recipe of one layer configuration."""

    def __init__(self, name, T, H, N, k, I, x_std, wr_dist, wr_param, bias_half,
                 w_std, gamma=1e-3, seed=0, skew=False, batches=1, with_experts=True):
        self.name, self.T, self.H, self.N, self.k, self.I = name, T, H, N, k, I
        self.x_std, self.wr_dist, self.wr_param = x_std, wr_dist, wr_param
        self.bias_half, self.w_std, self.gamma, self.seed = bias_half, w_std, gamma, seed
        self.skew, self.batches, self.with_experts = skew, batches, with_experts
        self.G = N + 1
        self.R = T * k + T

    # -- skewed-load extras: outlier channels and a Zipf per-expert offset
    def outlier_channels(self):
        if not self.skew:
            return np.zeros(0, dtype=np.int64)
        n_out = int(round(0.01 * self.H))
        order = _hash_order(self.seed, T_OUTLIER, self.H - 1) + 1   # never channel 0
        return np.sort(order[:n_out])

    def zipf_offsets(self):
        """o_i = ln(N p_pi(i)), p_r proportional to r^-1.2 (r = 1..N)."""
        r = np.arange(1, self.N + 1, dtype=np.float64)
        p = r ** -1.2
        p /= p.sum()
        perm = _hash_order(self.seed, T_PERM, self.N)
        return np.log(self.N * p[perm])

    def x_spec(self, batch=0):
        col_mult, const = None, None
        if self.skew:
            col_mult = np.ones(self.H)
            col_mult[self.outlier_channels()] = 100.0
            const = {0: 1.0}
        return Spec(T_X, (self.T, self.H), NORMAL, self.x_std, col_mult, const,
                    seed_offset=batch)

    def wr_spec(self):
        col_mult = None
        if self.skew:
            col_mult = np.ones(self.H)
            col_mult[self.outlier_channels()] = 0.01
        return Spec(T_WR, (self.N, self.H), self.wr_dist, self.wr_param, col_mult)

    def w1_spec(self):
        return Spec(T_W1, (self.G, 2 * self.I, self.H), NORMAL, self.w_std)

    def w2_spec(self):
        return Spec(T_W2, (self.G, self.H, self.I), NORMAL, self.w_std)

    def router_weight(self):
        """bf16 bits [N, H] (small enough to build on the host)."""
        w = generate(self.wr_spec(), self.seed)
        if self.skew:
            off = f32_to_bf16_bits(self.zipf_offsets().astype(np.float32))
            w[:, 0] = off
        return w

    def bias(self):
        if self.bias_half == 0.0:
            return np.zeros(self.N, dtype=np.float32)
        return generate(Spec(T_BIAS, (self.N,), UNIFORM, self.bias_half, dtype="f32"),
                        self.seed)

    def flops_per_token(self):
        return 2 * self.H * self.N + (self.k + 1) * 3 * 2 * self.H * self.I

    def gemm_flops(self):
        return 2.0 * self.R * 3 * self.H * self.I


WORKLOADS = {
    "tiny": Workload("tiny", T=64, H=256, N=16, k=2, I=128, x_std=1.0,
                     wr_dist=NORMAL, wr_param=0.02, bias_half=0.1, w_std=0.02),
    "routing": Workload("routing", T=16384, H=7168, N=256, k=8, I=2048, x_std=1.0,
                        wr_dist=NORMAL, wr_param=0.02, bias_half=0.05, w_std=0.006,
                        with_experts=False),
    # the V3-shaped layers start from a zero bias, as a fresh layer does: a
    # bias of +-0.05 moves the keys near the top of the sigmoid (where
    # s (1 - s) is about 0.03) by more than a logit standard deviation and
    # spreads the rows per expert from 1 to about 700 at T = 8192, where the
    # prefill batch is meant to load the experts roughly evenly
    "decode": Workload("decode", T=512, H=7168, N=256, k=8, I=2048, x_std=1.0,
                       wr_dist=NORMAL, wr_param=0.02, bias_half=0.0, w_std=0.006),
    "prefill": Workload("prefill", T=8192, H=7168, N=256, k=8, I=2048, x_std=1.0,
                        wr_dist=UNIFORM, wr_param=0.02 * math.sqrt(3.0),
                        bias_half=0.0, w_std=0.006),
    "skew": Workload("skew", T=32768, H=7168, N=256, k=8, I=2048, x_std=1.0,
                     wr_dist=NORMAL, wr_param=0.02, bias_half=0.0, w_std=0.006,
                     skew=True, batches=10),
}


# ---------------------------------------------------------------------------
# device generation (synth/libsynth.so, built by __graft_entry__.build)

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError("synth/libsynth.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.synth_fill.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def device_generate(spec, seed, out, stream=0, row0=0):
    """Fill the torch device tensor ``out`` (bf16 or float32, contiguous,
    holding rows [row0, row0 + out.numel() / cols) of the tensor viewed as
    [-1, cols]) on the device.  Constant columns are written afterwards by
    the caller-visible copy below."""
    import torch
    cols = spec.shape[-1]
    n = out.numel()
    assert n % cols == 0 and out.is_contiguous()
    coef = torch.from_numpy(spec.coef_cols()).to(out.device)
    key = stream_key(seed + spec.seed_offset, spec.tensor_id)
    is_bf16 = 1 if out.dtype == torch.bfloat16 else 0
    rc = _lib().synth_fill(ctypes.c_void_p(out.data_ptr()), n // cols, cols,
                           row0, ctypes.c_uint64(key), spec.dist,
                           ctypes.c_void_p(coef.data_ptr()), is_bf16,
                           ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill failed: {rc}")
    if spec.const_cols:
        v = out.view(-1, cols)
        for c, val in spec.const_cols.items():
            v[:, c] = val
    return out
