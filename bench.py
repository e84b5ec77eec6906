"""Benchmark of the DeepSeekMoE forward layer (FP8 block-scaled, sigmoid router)
on one MI355X.

A step is one forward pass of the whole layer over one batch: router + biased
top-k, permutation, 1x128 activation quantisation, grouped FP8 GEMM 1 with the
SwiGLU + re-quantisation epilogue, grouped FP8 GEMM 2, combine, bias update.
Weights are quantised 128x128 once before timing (a per-weight-update cost,
reported separately).  Inputs are seeded synthetic tensors generated on the
device, resident in HBM before the timed region.

Prints ONE JSON line.  Default workload: the DeepSeek-V3-shaped layer at
prefill size (T = 8192, H 7168, 256 routed experts top-8 + 1 shared, I 2048).
Other workloads: decode (T = 512), skew (T = 32768, ten batches cycled, load
max/mean reported), tiny, routing (T = 16384: router, top-k, permutation and
bias update only), and backward (the FP8 Dgrad and Wgrad GEMMs of both expert
GEMMs at the prefill shape, on synthetic upstream gradients).  The timed
region is K steps with an event pair around every launch on the launch stream;
per-kernel times are the means of those, and each step's time runs from its
first launch to its last (the median is reported beside the mean).  A second
pass of K steps, each after a write of --flush-mb MiB that evicts the caches,
gives the flushed median, K replays of one step captured in a HIP graph the
graph step time, and K calls of moe_layer_forward (the same kernels behind one
library call) the native-call step time.  Measured peaks are reported beside the published ones:
a 2 GiB device copy and the library's FP8 MFMA rate probe.
--router-fp8 swaps in the opt-in FP8 router (x quantised before routing); the
routing workload also times the other router on the same batch and reports
how many tokens both send to the same expert set.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
# rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the GEMM1 kernel at this
# workload; its bytes count only while the kernel source is unchanged
COUNTERS = os.path.join(ROOT, "profiles", "layer_prefill_T8192_hbm_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "fp8_block_scaled_sigmoid_amd", "csrc", f)
                  for f in ("gemm_fp8.hip", "common.h")]


def kernel_source_hash():
    """Hash of the GEMM kernel's source with comments and blank space removed
    (a comment edit does not change the kernel the counters measured)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per GEMM1 launch from the committed counter summary, or None
    if there is none for this workload or the kernel changed since."""
    if workload != "prefill" or not os.path.exists(COUNTERS):
        return None
    vals = {}
    for line in open(COUNTERS):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch_calibrated"])
    except (KeyError, ValueError):
        return None


def measured_peaks(moe, torch, st):
    """What the device reaches in practice, beside the published peaks: a
    plain 2 GiB device-to-device copy (read + write bytes per second), the
    library's HBM probe reading 2 GiB and writing 2 GiB (16-byte accesses;
    the faster of two read modes and of two write modes), and the FP8 MFMA rate probe (back-to-back
    16x16x128 FP8 MFMAs, four waves per SIMD, no memory traffic)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(5):
        dst.copy_(src)
    e1.record(st)
    torch.cuda.synchronize()
    copy_ms = e0.elapsed_time(e1) / 5
    stream_ms = {}
    for mode, name in ((0, "read_nt8"), (1, "write_nt"), (2, "read_plain4"), (3, "write_plain")):
        moe.moe_probe_hbm(mode, src, stream=st)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(5):
            moe.moe_probe_hbm(mode, src, stream=st)
        e1.record(st)
        torch.cuda.synchronize()
        stream_ms[name] = e0.elapsed_time(e1) / 5
    del src, dst
    blocks, iters = 256 * 4, 4000
    sink, _ = moe.moe_probe_fp8_mfma(blocks, 8)
    torch.cuda.synchronize()
    e0.record(st)
    _, flops = moe.moe_probe_fp8_mfma(blocks, iters, sink=sink)
    e1.record(st)
    torch.cuda.synchronize()
    mfma_ms = e0.elapsed_time(e1)
    return {"copy_bytes_read": n, "copy_bytes_written": n, "copy_ms": round(copy_ms, 4),
            "copy_GBps_read_plus_write": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
            "read_GBps": round(n / (min(stream_ms["read_nt8"], stream_ms["read_plain4"]) * 1e-3) / 1e9, 1),
            "write_GBps": round(n / (min(stream_ms["write_nt"], stream_ms["write_plain"]) * 1e-3) / 1e9, 1),
            "probe_GBps": {k: round(n / (v * 1e-3) / 1e9, 1) for k, v in stream_ms.items()},
            "fp8_mfma_probe_ms": round(mfma_ms, 4),
            "fp8_mfma_TFLOPs": round(flops / (mfma_ms * 1e-3) / 1e12, 1)}


def attainable_GBps(read_bytes, write_bytes, peaks):
    """The measured rate for a step's own mix of reads and writes: its reads
    at the measured read-only rate and its writes at the measured write-only
    rate, one after the other ((r + w) / (r / R + w / W)); a plain copy, which
    overlaps the two, is reported beside it."""
    t = read_bytes / peaks["read_GBps"] + write_bytes / peaks["write_GBps"]
    return (read_bytes + write_bytes) / t if t > 0 else 0.0


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill",
                    choices=["prefill", "decode", "skew", "routing", "tiny", "backward"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--router-fp8", action="store_true",
                    help="the opt-in FP8 router (x quantised 1x128 first, Wr 128x128) in place "
                         "of the bf16 one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also report the 2 GiB device copy under its own key (the reference "
                         "for the HBM byte counters; the copy itself always runs, as one of "
                         "the measured peaks)")
    ap.add_argument("--no-sub-workloads", action="store_true",
                    help="skip the decode and skew sub-results of the default prefill run")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="size of the write that precedes every step of the flushed pass")
    return ap.parse_args()


def cpu_baseline(w, sample_tokens=None):
    """The oracle, untuned, on a bounded sample of the same workload.

    Sample: the first `sample_tokens` tokens of the batch (default: up to
    8192).  Routing, the activation quantisation, the permutation, the combine
    and the bias update run on the whole sample; the expert FFN runs on every
    sample row of the shared expert and of the two routed experts with the
    most sample rows, and its per-row time is scaled to the sample's T*(k+1)
    rows (the per-row cost of the FFN does not depend on which expert the row
    belongs to).  Result: tokens per second of the whole layer on the host."""
    import synth
    from oracle import bias as obias, ffn, permute as operm, quant, route
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    S = min(w.T, 8192) if sample_tokens is None else min(sample_tokens, w.T)
    x = synth.as_f64(synth.generate(w.x_spec(), w.seed, rows=np.arange(S)))
    wr = synth.as_f64(w.router_weight())
    b = w.bias()
    t0 = time.perf_counter()
    s64, s32, idx, gate = route.route(x, wr, b, w.k)
    xq, xd = quant.quant_1x128(x)
    counts, offsets, row_of, token_of = operm.permute(idx, w.N, True)
    t_route = time.perf_counter() - t0
    top = np.argsort(-counts, kind="stable")[:2]
    experts = [w.N] + [int(e) for e in top]
    rows_done, t_ffn = 0, 0.0
    out = np.zeros((S * w.k + S, w.H))
    for g in experts:
        H, I = w.H, w.I
        w1 = synth.as_f64(synth.generate(w.w1_spec(), w.seed, rows=np.arange(g * 2 * I, (g + 1) * 2 * I)))
        w2 = synth.as_f64(synth.generate(w.w2_spec(), w.seed, rows=np.arange(g * H, (g + 1) * H)))
        w1q, w1d = quant.quant_128x128(w1)
        w2q, w2d = quant.quant_128x128(w2)
        del w1, w2
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        toks = token_of[r0:r1]
        t1 = time.perf_counter()
        res = ffn.expert_ffn(xq[toks], xd[toks], w1q, w1d, w2q, w2d, "D")
        t_ffn += time.perf_counter() - t1
        out[r0:r1] = res["out"]
        rows_done += r1 - r0
    t2 = time.perf_counter()
    ffn.combine(out, gate, row_of, S * w.k, "D")
    obias.bias_update(b, counts, S, w.k, w.gamma)
    t_tail = time.perf_counter() - t2
    t_total = t_route + t_tail + t_ffn / rows_done * (S * (w.k + 1))
    return {"value": S / t_total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"{S} tokens of the {w.name} batch: routing, quantisation, permutation, "
                       f"combine and bias update on all {S}; expert FFN timed on {rows_done} rows "
                       f"(shared expert + 2 most-loaded routed experts) and scaled per row to "
                       f"{S * (w.k + 1)} rows"),
            "measured_s": round(t_route + t_ffn + t_tail, 3)}


def cpu_baseline_routing(w):
    """The oracle's routing path (router, biased top-k, gates, counts and
    permutation, bias update) on the whole routing batch, on the host."""
    import synth
    from oracle import bias as obias, permute as operm, route
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    x = synth.as_f64(synth.generate(w.x_spec(), w.seed))
    wr = synth.as_f64(w.router_weight())
    b = w.bias()
    t0 = time.perf_counter()
    s64, s32, idx, gate = route.route(x, wr, b, w.k)
    counts, offsets, row_of, token_of = operm.permute(idx, w.N, False)
    obias.bias_update(b, counts, w.T, w.k, w.gamma)
    dt = time.perf_counter() - t0
    return {"value": w.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"all {w.T} tokens of the {w.name} batch (router, top-k, gates, counts, "
                      f"permutation, bias update)", "measured_s": round(dt, 3)}


def route_rw_of(T, H, N, k, fp8):
    """Algorithmic HBM bytes (read, written) of the routing step: x and Wr
    read once (bf16, or for the FP8 router x bf16 read by the quantiser, its
    codes and scales written and read back, Wr codes and scales read), bias
    read, scores and (index, gate) pairs written."""
    wr = T * N * 4 + T * k * 8
    if not fp8:
        return T * H * 2 + N * H * 2 + N * 4, wr
    xq = T * H + T * (H // 128) * 4
    return T * H * 2 + xq + N * H + (N // 128) * (H // 128) * 4 + N * 4, wr + xq


def route_bytes_of(T, H, N, k, fp8):
    return sum(route_rw_of(T, H, N, k, fp8))


def bench_routing(args, w, moe, torch, gen, wr, bias, st):
    """The routing-only workload: a step is the router with biased top-k and
    gates, the counts and permutation maps, and the bias update."""
    dev = wr.device
    T, H, N, k = w.T, w.H, w.N, w.k
    x = gen(w.x_spec())
    e = dict(device=dev)
    scores = torch.empty(T, N, dtype=torch.float32, **e)
    idx = torch.empty(T, k, dtype=torch.int32, **e)
    gate = torch.empty(T, k, dtype=torch.float32, **e)
    rws = torch.empty(max(moe.moe_route_workspace_bytes(T, H, N), 16), dtype=torch.uint8, **e)
    maps = (torch.empty(N, dtype=torch.int32, **e), torch.empty(N + 2, dtype=torch.int32, **e),
            torch.empty(T, k, dtype=torch.int32, **e), torch.empty(T * k, dtype=torch.int32, **e))
    pws = torch.empty(max(moe.moe_permute_workspace_bytes(T, N, k), 16), dtype=torch.uint8, **e)
    xq = torch.empty(T, H, dtype=torch.uint8, **e)
    xd = torch.empty(T, H // 128, dtype=torch.float32, **e)
    wq, wd = moe.fp8_quant_128x128(wr)          # per weight update, outside the timed region
    wq, wd = wq[0], wd[0]

    def route_bf16(out_idx):
        moe.moe_route_topk(x, wr, bias, k, scores=scores, idx=out_idx, gate=gate, ws=rws)

    def route_fp8(out_idx):
        moe.fp8_quant_1x128(x, q=xq, d=xd)
        moe.moe_route_topk_fp8(xq, xd, wq, wd, bias, k, scores=scores, idx=out_idx, gate=gate,
                               ws=rws)

    main_route, other_route = (route_fp8, route_bf16) if args.router_fp8 else \
        (route_bf16, route_fp8)
    names = ["route", "permute", "bias"]
    fns = [lambda: main_route(idx),
           lambda: moe.moe_permute(idx, N, False, out=maps, ws=pws),
           lambda: moe.moe_bias_update(bias, maps[0], T, k, w.gamma)]

    def step(evs=None):
        for i, f in enumerate(fns):
            if evs is not None:
                evs[i][0].record(st)
            f()
            if evs is not None:
                evs[i][1].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in names] for _ in range(args.steps)]
    e0.record(st)
    for i in range(args.steps):
        step(evs[i])
    e1.record(st)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    kern = {n: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1])
                              for i in range(args.steps)]))
            for j, n in enumerate(names)}
    step_ms = [evs[i][0][0].elapsed_time(evs[i][-1][1]) for i in range(args.steps)]
    route_bytes = route_bytes_of(T, H, N, k, args.router_fp8)
    gbs = route_bytes / (kern["route"] * 1e-3) / 1e9
    # the other router on the same batch and bias (after the timed region):
    # its time, and the fraction of tokens that both send to the same experts
    idx_other = torch.empty_like(idx)
    other_route(idx_other)
    e0.record(st)
    for _ in range(args.steps):
        other_route(idx_other)
    e1.record(st)
    torch.cuda.synchronize()
    main_route(idx)
    same = (idx.sort(dim=1).values == idx_other.sort(dim=1).values).all(dim=1)
    agree = float(same.float().mean().item())
    other_ms = e0.elapsed_time(e1) / args.steps
    peaks = measured_peaks(moe, torch, st)
    res = {
        "metric": "MoE routing tokens/s (sigmoid router + biased top-k + permutation + bias "
                  "update) at V3 shape, 1 GPU",
        "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8_e4m3 router" if args.router_fp8 else "bf16") + " (fp32 accumulate)",
        "data": "synthetic (seeded counter-based generator, generated on the device)",
        "config": {"workload": f"{w.name}: T={T} tokens, hidden {H}, {N} experts top-{k}, "
                               f"bias U(-0.05, 0.05), gamma {w.gamma}",
                   "T": T, "H": H, "N": N, "k": k,
                   "router": "fp8" if args.router_fp8 else "bf16"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": ("fp8_quant_1x128 + route_partial_fp8_kernel + route_finish_kernel"
                                if args.router_fp8 else
                                "route_partial_kernel + route_finish_kernel"),
                     "kernel_avg_ms": round(kern["route"], 4),
                     "algorithmic_bytes_per_launch": route_bytes},
        "kernel_ms": {n: round(v, 4) for n, v in kern.items()},
        "step_ms_median": round(float(np.median(step_ms)), 4),
        "route_frac_measured_read_write_mix": round(
            gbs / attainable_GBps(*route_rw_of(T, H, N, k, args.router_fp8), peaks), 4),
        "measured_peaks": peaks,
        "other_router": {"router": "bf16" if args.router_fp8 else "fp8",
                         "route_ms": round(other_ms, 4),
                         "same_expert_set_fraction": round(agree, 4)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_routing(w)
    print(json.dumps(res))


def bench_backward(args, w, moe, torch, gen, lay, st):
    """The FP8 backward GEMMs of the expert layer at the prefill shape.  A step:
      Dgrad2  dH = dOut W2           (dOut quantised 1x128; W2 transposed once)
      Wgrad2  dW2_g = dOut_g^T h_g   (128-token tiles of dOut and h)
      Dgrad1  dU = dA W1             (dA: gradient at the GEMM1 output)
      Wgrad1  dW1_g = dA_g^T x_g     (128-token tiles of dA and the gathered x)
    with every quantisation in the step.  The upstream gradients dOut and dA
    and the SwiGLU output h are seeded synthetic tensors; the expert groups are
    those of the forward routing of the workload's batch.  Weight gradients are
    float32, input gradients bf16."""
    import synth
    dev = lay.y.device
    x = gen(w.x_spec())
    lay.route(x)
    lay.permute()
    torch.cuda.synchronize()
    T, H, I, G, R = w.T, w.H, w.I, w.G, lay.R
    off = lay.offsets[:G + 1].contiguous()
    x_rows = x.index_select(0, lay.token_of.long())                  # the gathered GEMM1 input
    dout = gen(synth.Spec(synth.T_DOUT, (R, H), synth.NORMAL, 1e-3))
    d_a = gen(synth.Spec(synth.T_DA, (R, 2 * I), synth.NORMAL, 1e-3))
    h = gen(synth.Spec(synth.T_H, (R, I), synth.NORMAL, 1.0))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    w1t = moe.fp8_transpose_128x128(lay.w.w1q, lay.w.w1d)
    w2t = moe.fp8_transpose_128x128(lay.w.w2q, lay.w.w2d)
    e1.record(st)
    torch.cuda.synchronize()
    t_transpose = e0.elapsed_time(e1)
    e = dict(device=dev)
    ldt = moe.tokens_padded_width(R, G)
    dq = (torch.empty(R, H, dtype=torch.uint8, **e), torch.empty(R, H // 128, dtype=torch.float32, **e))
    aq = (torch.empty(R, 2 * I, dtype=torch.uint8, **e),
          torch.empty(R, 2 * I // 128, dtype=torch.float32, **e))
    d_h = torch.empty(R, I, dtype=torch.bfloat16, **e)
    d_u = torch.empty(R, H, dtype=torch.bfloat16, **e)

    def tok(C):
        return (torch.empty(C, ldt, dtype=torch.uint8, **e),
                torch.empty(C, ldt // 128, dtype=torch.float32, **e),
                torch.empty(G + 1, dtype=torch.int32, **e))
    t_dout, t_h, t_da, t_x = tok(H), tok(I), tok(2 * I), tok(H)
    dw2 = torch.empty(G, H, I, dtype=torch.float32, **e)
    dw1 = torch.empty(G, 2 * I, H, dtype=torch.float32, **e)
    E_BF16 = moe.MOE_EPI_BF16

    def tq(src, dst):
        moe.fp8_quant_tokens_128(src, off, ldt=ldt, xt_q=dst[0], xt_d=dst[1], pad_offsets=dst[2])

    names = ["quant_dout", "dgrad2", "tok_dout", "tok_h", "wgrad2",
             "quant_da", "dgrad1", "tok_da", "tok_x", "wgrad1"]
    fns = [lambda: moe.fp8_quant_1x128(dout, q=dq[0], d=dq[1]),
           lambda: moe.moe_grouped_gemm_fp8(dq[0], dq[1], w2t[0], w2t[1], off, R, E_BF16, out=d_h),
           lambda: tq(dout, t_dout), lambda: tq(h, t_h),
           lambda: moe.moe_grouped_wgrad_fp8(t_dout[0], t_dout[1], t_h[0], t_h[1], t_dout[2], out=dw2),
           lambda: moe.fp8_quant_1x128(d_a, q=aq[0], d=aq[1]),
           lambda: moe.moe_grouped_gemm_fp8(aq[0], aq[1], w1t[0], w1t[1], off, R, E_BF16, out=d_u),
           lambda: tq(d_a, t_da), lambda: tq(x_rows, t_x),
           lambda: moe.moe_grouped_wgrad_fp8(t_da[0], t_da[1], t_x[0], t_x[1], t_da[2], out=dw1)]

    def step(evs=None):
        for i, f in enumerate(fns):
            if evs is not None:
                evs[i][0].record(st)
            f()
            if evs is not None:
                evs[i][1].record(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in names] for _ in range(args.steps)]
    e0.record(st)
    for i in range(args.steps):
        step(evs[i])
    e1.record(st)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    kern = {n: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1])
                              for i in range(args.steps)]))
            for j, n in enumerate(names)}
    rpad = int(t_dout[2][-1].item())
    nb = rpad // 128
    # algorithmic work of each GEMM: operands read once, output written once
    work = {
        "dgrad2": (2.0 * R * H * I,
                   R * H + R * (H // 128) * 4 + G * H * I + G * (H // 128) * (I // 128) * 4 + R * I * 2),
        "wgrad2": (2.0 * R * H * I, (H + I) * (rpad + nb * 4) + G * H * I * 4),
        "dgrad1": (2.0 * R * 2 * I * H,
                   R * 2 * I + R * (2 * I // 128) * 4 + G * 2 * I * H
                   + G * (2 * I // 128) * (H // 128) * 4 + R * H * 2),
        "wgrad1": (2.0 * R * 2 * I * H, (2 * I + H) * (rpad + nb * 4) + G * 2 * I * H * 4),
    }
    gemm_flops = sum(f for f, _ in work.values())
    gemm_ms = sum(kern[n] for n in work)
    dom = max(work, key=lambda n: kern[n])
    fl, by = work[dom]
    t_dom = kern[dom] * 1e-3
    if by / (HBM_PEAK_GBS * 1e9) >= fl / (FP8_PEAK_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": round(by / t_dom / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(by / t_dom / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(fl / t_dom / 1e12, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(fl / t_dom / 1e12 / FP8_PEAK_TFLOPS, 4)}
    kname = {"wgrad1": "wgrad_kernel (dW1)", "wgrad2": "wgrad_kernel (dW2)",
             "dgrad1": "grouped_gemm256_kernel<BF16> (dX, Dgrad of W1)",
             "dgrad2": "grouped_gemm256_kernel<BF16> (dH, Dgrad of W2)"}[dom]
    roof.update({"traffic": None, "kernel": kname, "kernel_avg_ms": round(kern[dom], 4),
                 "algorithmic_bytes_per_launch": by, "algorithmic_flops_per_launch": fl,
                 "mfma_tflops": round(fl / t_dom / 1e12, 2),
                 "hbm_gbs": round(by / t_dom / 1e9, 1)})
    res = {
        "metric": "MoE layer FP8 backward GEMMs tokens/s (Dgrad + Wgrad of both expert GEMMs) "
                  "at V3 shape, 1 GPU",
        "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded upstream gradients and h generated on the device; expert "
                "groups from the forward routing of the prefill batch)",
        "config": {"workload": f"backward of the prefill layer's expert GEMMs: T={T} tokens, "
                               f"{R} expert rows, hidden {H}, {w.N} routed experts top-{w.k} + 1 "
                               f"shared, SwiGLU intermediate {I}",
                   "T": T, "R": R, "H": H, "I": I, "G": G, "padded_token_columns": rpad},
        "roofline": roof,
        "gemm_tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 2),
        "gemm_frac_fp8_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4),
        "kernel_ms": {n: round(v, 4) for n, v in kern.items()},
        "per_gemm": {n: {"ms": round(kern[n], 4),
                         "TFLOPs": round(f / (kern[n] * 1e-3) / 1e12, 2),
                         "GBps": round(b / (kern[n] * 1e-3) / 1e9, 1)} for n, (f, b) in work.items()},
        "weight_transpose_ms": round(t_transpose, 3),
    }
    peaks = measured_peaks(moe, torch, st)
    res["measured_peaks"] = peaks
    res["gemm_frac_measured_mfma_peak"] = round(
        gemm_flops / (gemm_ms * 1e-3) / 1e12 / peaks["fp8_mfma_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_backward(w, R)
    print(json.dumps(res))


def cpu_baseline_backward(w, R):
    """The oracle's four backward GEMMs with their quantisation on a sample of
    4096 expert rows in 16 groups of 256 (the mean routed-expert load), timed
    on the host and scaled per row to the step's R rows."""
    import synth
    from oracle import backward, quant
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    H, I, S = w.H, w.I, 4096
    off = np.arange(0, S + 1, 256)
    rows = np.arange(S)
    f64 = synth.as_f64
    dout = f64(synth.generate(synth.Spec(synth.T_DOUT, (R, H), synth.NORMAL, 1e-3), w.seed, rows=rows))
    d_a = f64(synth.generate(synth.Spec(synth.T_DA, (R, 2 * I), synth.NORMAL, 1e-3), w.seed, rows=rows))
    h = f64(synth.generate(synth.Spec(synth.T_H, (R, I), synth.NORMAL, 1.0), w.seed, rows=rows))
    x = f64(synth.generate(w.x_spec(), w.seed, rows=rows))
    w1q, w1d = quant.quant_128x128(f64(synth.generate(w.w1_spec(), w.seed, rows=np.arange(2 * I))))
    w2q, w2d = quant.quant_128x128(f64(synth.generate(w.w2_spec(), w.seed, rows=np.arange(H))))
    t0 = time.perf_counter()
    for g in range(off.size - 1):
        sl = slice(off[g], off[g + 1])
        backward.dgrad(dout[sl], w2q, w2d)
        backward.dgrad(d_a[sl], w1q, w1d)
    backward.wgrad(dout, h, off)
    backward.wgrad(d_a, x, off)
    dt = time.perf_counter() - t0
    return {"value": w.T / (dt / S * R), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{S} expert rows in 16 groups of 256: Dgrad and Wgrad of both expert "
                      f"GEMMs with their quantisers, scaled per row to {R} rows",
            "measured_s": round(dt, 3)}


def layer_step_fns(lay, xs, cur, router_fp8):
    """The launches of one layer step, in order, with their names."""
    names = ["route", "permute", "gemm1", "gemm2", "combine", "bias"]
    fns = [lambda: lay.route(xs[cur["i"] % len(xs)]), lay.permute, lay.gemm1, lay.gemm2,
           lay.combine, lay.bias_update]
    if router_fp8:    # the FP8 router reads the quantised x: quantise first
        names = ["quant_x"] + names
        fns = [lambda: lay.quant_x(xs[cur["i"] % len(xs)])] + fns
    return names, fns


def time_layer_steps(torch, st, names, fns, cur, steps, warmup):
    """W untimed steps, then K timed ones with an event pair around every
    launch on the launch stream and one pair around the whole region.
    Returns (ms per step, per-kernel mean ms, per-step ms, wall seconds, and
    the step function itself)."""
    def step(evs=None):
        for i, f in enumerate(fns):
            if evs is not None:
                evs[i][0].record(st)
            f()
            if evs is not None:
                evs[i][1].record(st)
        cur["i"] += 1

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in names] for _ in range(steps)]
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(steps):
        step(evs[i])
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    kern = {n: float(np.mean([evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(steps)]))
            for j, n in enumerate(names)}
    # each step's own time: from the first launch's start event to the last
    # launch's end event
    step_ms = [evs[i][0][0].elapsed_time(evs[i][-1][1]) for i in range(steps)]
    return ms_step, kern, step_ms, wall, step


def gemm_work(w, counts=None):
    """FLOPs of both expert GEMMs, and the algorithmic HBM bytes of one GEMM1
    launch (every W1 code and scale once, every token's x codes and scales
    once, the row map, the h codes and scales out) and of one GEMM2 launch
    (every W2 code and scale once, the h codes and scales, the expert rows
    out).  With the routed experts' row counts given, only the weights of the
    groups that hold rows count (the GEMMs never read the others); the shared
    expert always holds T rows."""
    R, G, T, H, I = w.R, w.G, w.T, w.H, w.I
    if counts is not None:
        G = int(np.count_nonzero(np.asarray(counts) > 0)) + 1
    g1_flops = 2.0 * R * H * 2 * I
    g2_flops = 2.0 * R * I * H
    g1_bytes = (G * 2 * I * H + G * (2 * I // 128) * (H // 128) * 4
                + T * H + T * (H // 128) * 4 + R * 4 + (G + 1) * 4
                + R * I + R * (I // 128) * 4)
    g2_bytes = (G * H * I + G * (H // 128) * (I // 128) * 4 + R * I + R * (I // 128) * 4
                + (G + 1) * 4 + R * H * 2)
    return g1_flops, g2_flops, g1_bytes, g2_bytes


def roofline_of(flops, nbytes, ms):
    """Achieved rate against the binding roof, the one with the longer
    minimum time (HBM 8 TB/s or FP8 MFMA 5 PFLOP/s)."""
    t = ms * 1e-3
    tf, gbs = flops / t / 1e12, nbytes / t / 1e9
    if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (FP8_PEAK_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / FP8_PEAK_TFLOPS, 4)}
    roof.update({"mfma_tflops": round(tf, 2), "mfma_frac": round(tf / FP8_PEAK_TFLOPS, 4),
                 "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    return roof


def sub_workload(name, args, moe, torch, st, dev, wq):
    """Another DeepSeek-V3-shaped workload on the same (already quantised)
    expert weights -- every V3-shaped workload draws its experts from the same
    generator stream -- timed the same way as the main one: ms and tokens/s
    per step, both GEMMs against their roofs, and the per-expert load
    max/mean after each of its batches (one pass from the workload's initial
    bias, before the timed steps)."""
    import synth
    w = synth.WORKLOADS[name]

    def gen(spec, seed=w.seed):
        t = torch.empty(spec.shape, dtype=torch.bfloat16, device=dev)
        synth.device_generate(spec, seed, t)
        return t

    wr = torch.from_numpy(w.router_weight().view(np.int16)).view(torch.bfloat16).to(dev)
    b0 = torch.from_numpy(w.bias().copy()).to(dev)
    bias = b0.clone()
    weights = moe.MoEWeights(wr, bias, w1q=wq[0], w1d=wq[1], w2q=wq[2], w2d=wq[3])
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma, device=dev)
    xs = [gen(w.x_spec(b)) for b in range(w.batches)]
    loads = []
    for x in xs:
        lay.forward(x)
        c = lay.counts.cpu().numpy()
        loads.append(round(float(c.max() / c.mean()), 3))
        used = int(np.count_nonzero(c > 0))
    bias.copy_(b0)
    cur = {"i": 0}
    names, fns = layer_step_fns(lay, xs, cur, False)
    ms_step, kern, step_ms, _, _ = time_layer_steps(torch, st, names, fns, cur, args.steps,
                                                    args.warmup)
    g1f, g2f, g1b, g2b = gemm_work(w, c)
    tf = (g1f + g2f) / ((kern["gemm1"] + kern["gemm2"]) * 1e-3) / 1e12
    res = {"config": f"{w.name}: T={w.T} tokens, hidden {w.H}, {w.N} routed experts top-{w.k} "
                     f"+ 1 shared, SwiGLU intermediate {w.I}"
                     + (f", {w.batches} batches cycled with sign bias updates" if w.batches > 1
                        else ""),
           "T": w.T,
           "ms_per_step": round(ms_step, 4),
           "tokens_per_s": round(w.T / (ms_step * 1e-3), 1),
           "layer_ms_median": round(float(np.median(step_ms)), 4),
           "gemm_tflops": round(tf, 2),
           "gemm_frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4),
           "gemm1_roofline": dict(roofline_of(g1f, g1b, kern["gemm1"]),
                                  kernel_avg_ms=round(kern["gemm1"], 4),
                                  algorithmic_bytes_per_launch=g1b),
           "gemm2_roofline": dict(roofline_of(g2f, g2b, kern["gemm2"]),
                                  kernel_avg_ms=round(kern["gemm2"], 4),
                                  algorithmic_bytes_per_launch=g2b),
           "kernel_ms": {n: round(v, 4) for n, v in kern.items()},
           "routed_experts_with_rows": used,
           "expert_load_max_over_mean": loads if w.batches > 1 else loads[0]}
    del lay, xs, weights
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(the expert-parallel design across GPUs is described, not built)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import fp8_block_scaled_sigmoid_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    # the backward workload runs the prefill layer's expert GEMMs backwards
    w = synth.WORKLOADS["prefill" if args.workload == "backward" else args.workload]
    dev = torch.device("cuda:0")

    def gen(spec, seed=w.seed):
        t = torch.empty(spec.shape, dtype=torch.bfloat16, device=dev)
        synth.device_generate(spec, seed, t)
        return t

    wr = torch.from_numpy(w.router_weight().view(np.int16)).view(torch.bfloat16).to(dev)
    bias = torch.from_numpy(w.bias().copy()).to(dev)
    st = torch.cuda.current_stream()
    if not w.with_experts:
        bench_routing(args, w, moe, torch, gen, wr, bias, st)
        return
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w1 = gen(w.w1_spec())
    e0.record(st)
    w1q, w1d = moe.fp8_quant_128x128(w1, interleave_gate_up=True)
    e1.record(st)
    torch.cuda.synchronize()
    t_wq1 = e0.elapsed_time(e1)
    del w1
    w2 = gen(w.w2_spec())
    e0.record(st)
    w2q, w2d = moe.fp8_quant_128x128(w2)
    e1.record(st)
    torch.cuda.synchronize()
    t_wq2 = e0.elapsed_time(e1)
    del w2
    torch.cuda.empty_cache()
    weights = moe.MoEWeights(wr, bias, w1q=w1q, w1d=w1d, w2q=w2q, w2d=w2d,
                             router_fp8=args.router_fp8)
    lay = moe.MoELayer(weights, w.T, w.k, w.gamma, device=dev, router_fp8=args.router_fp8)
    if args.workload == "backward":
        bench_backward(args, w, moe, torch, gen, lay, st)
        return
    # the batches of the workload (one for most; the skewed-load workload has
    # ten, batch b drawn with seed offset b); step i runs batch i % batches
    xs = [gen(w.x_spec(b)) for b in range(w.batches)]
    cur = {"i": 0}

    names, fns = layer_step_fns(lay, xs, cur, args.router_fp8)
    ms_step, kern, step_ms, wall, step = time_layer_steps(torch, st, names, fns, cur, args.steps,
                                                          args.warmup)
    # a second pass of K steps, each preceded by a write of flush_mb MiB (not
    # timed) so that no step finds the previous step's data in the caches
    flush = torch.empty(max(args.flush_mb, 1) << 20, dtype=torch.uint8, device=dev)
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        fev[i][0].record(st)
        step()
        fev[i][1].record(st)
    torch.cuda.synchronize()
    flushed_ms = [a.elapsed_time(b) for a, b in fev]
    # each HBM-bound phase once more on its own after the same cache-evicting
    # write, K times: inside a step a phase may find part of its input still
    # in the caches (combine reads the expert outputs GEMM2 has just written),
    # which would overstate its HBM rate
    cold = {}
    for n in [n_ for n_ in ("route", "permute", "quant_x", "combine") if n_ in names]:
        f = fns[names.index(n)]
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            flush.fill_(i & 0xFF)
            cev[i][0].record(st)
            f()
            cev[i][1].record(st)
        torch.cuda.synchronize()
        cold[n] = float(np.mean([a.elapsed_time(b) for a, b in cev]))
    del flush
    # one step captured in a HIP graph and replayed K times (the launches of a
    # step without their host-side cost); the captured step keeps the batch it
    # was captured with
    graph_ms = None
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(args.steps):
            g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        del g
    except RuntimeError as err:      # reported, not fatal: the eager numbers stand
        graph_ms = f"capture failed: {err}"
    # the same step as one library call (moe_layer_forward: the kernels of
    # step() in the same order, every intermediate in one workspace), K calls
    ws_native = torch.empty(moe.moe_layer_workspace_bytes(w.T, w.H, w.N, w.k, w.I,
                                                          lay.with_shared),
                            dtype=torch.uint8, device=dev)

    def native_step():
        moe.moe_layer_forward(weights, xs[cur["i"] % len(xs)], w.k, w.gamma,
                              router_fp8=args.router_fp8, y=lay.y, ws=ws_native, stream=st)
        cur["i"] += 1

    native_step()
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(args.steps):
        native_step()
    e1.record(st)
    torch.cuda.synchronize()
    native_ms = e0.elapsed_time(e1) / args.steps
    del ws_native
    # after the timed region: the per-expert load max/mean of the workload's
    # batches (one more pass over them, each followed by a read of the counts)
    load_ratio = []
    for _ in range(max(w.batches, 1)):
        step()
        c = lay.counts.cpu().numpy()
        load_ratio.append(round(float(c.max() / c.mean()), 3))

    R, G, T, H, I = w.R, w.G, w.T, w.H, w.I
    g1_flops, g2_flops, g1_bytes, g2_bytes = gemm_work(w, c)
    gemm_tflops = (g1_flops + g2_flops) / ((kern["gemm1"] + kern["gemm2"]) * 1e-3) / 1e12
    tokens_per_s = w.T / (ms_step * 1e-3)
    r1 = roofline_of(g1_flops, g1_bytes, kern["gemm1"])
    roof = {k_: r1[k_] for k_ in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update({"traffic": measured_traffic(args.workload),
                 "kernel": "grouped_gemm256_kernel<SWIGLU_FP8> (GEMM1, 256-row tiles)",
                 "kernel_avg_ms": round(kern["gemm1"], 4),
                 "algorithmic_bytes_per_launch": g1_bytes,
                 "algorithmic_flops_per_launch": g1_flops})
    roof.update({k_: r1[k_] for k_ in ("mfma_tflops", "mfma_frac", "hbm_gbs", "hbm_frac")})

    # the HBM-bound phases: algorithmic bytes (each input read once, each output
    # written once) over the measured kernel time
    N, k = w.N, w.k
    # (read, written) algorithmic bytes of each HBM phase
    # (the bf16 router also writes the 1x128 codes and scales of x)
    phase_rw = {
        "route": ((N * H + (N // 128) * (H // 128) * 4 + T * H + T * (H // 128) * 4 + N * 4,
                   T * N * 4 + T * k * 8) if args.router_fp8 else
                  (T * H * 2 + N * H * 2 + N * 4,
                   T * N * 4 + T * k * 8 + T * H + T * (H // 128) * 4)),
        "combine": (R * H * 2 + T * k * 8, T * H * 2),
        "permute": (T * k * 4, N * 4 + (N + 2) * 4 + T * k * 4 + R * 4),
    }
    if args.router_fp8:
        phase_rw["quant_x"] = (T * H * 2, T * H + T * (H // 128) * 4)
    peaks = measured_peaks(moe, torch, st)
    phases = {}
    for n, (rb, wb) in phase_rw.items():
        # rates from the launch on cold caches; ms_in_step is its time inside
        # the timed steps
        gbs = (rb + wb) / (cold[n] * 1e-3) / 1e9
        phases[n] = {"bytes": rb + wb, "bytes_read": rb, "bytes_written": wb,
                     "ms": round(cold[n], 4), "ms_in_step": round(kern[n], 4),
                     "GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "frac_measured_read_write_mix": round(gbs / attainable_GBps(rb, wb, peaks), 4)}
    # the other DeepSeek-V3-shaped workloads on the same quantised weights
    subs = {}
    if args.workload == "prefill" and not args.no_sub_workloads:
        for sub in ("decode", "skew"):
            subs[sub] = sub_workload(sub, args, moe, torch, st, dev, (w1q, w1d, w2q, w2d))
    res = {
        "metric": "MoE layer tokens/s + grouped FP8 GEMM TFLOP/s (% peak) at V3 shape, 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded counter-based generator, generated on the device)",
        "config": {"workload": f"{w.name}: T={w.T} tokens, hidden {w.H}, {w.N} routed experts "
                               f"top-{w.k} + 1 shared, SwiGLU intermediate {w.I}, FP8 E4M3 "
                               f"1x128 / 128x128 scales",
                   "T": w.T, "H": w.H, "N": w.N, "k": w.k, "I": w.I,
                   "router": "fp8" if args.router_fp8 else "bf16"},
        "roofline": roof,
        "gemm_tflops": round(gemm_tflops, 2),
        "gemm_frac_fp8_peak": round(gemm_tflops / FP8_PEAK_TFLOPS, 4),
        "gemm_frac_measured_mfma_peak": round(gemm_tflops / peaks["fp8_mfma_TFLOPs"], 4),
        "layer_ms_median": round(float(np.median(step_ms)), 4),
        "layer_ms_median_flushed": round(float(np.median(flushed_ms)), 4),
        "graph_ms_per_step": round(graph_ms, 4) if isinstance(graph_ms, float) else graph_ms,
        "native_call_ms_per_step": round(native_ms, 4),
        "flush_mb": args.flush_mb,
        "measured_peaks": peaks,
        "kernel_ms": {n: round(v, 4) for n, v in kern.items()},
        "hbm_phases": phases,
        "expert_load_max_over_mean": load_ratio if w.batches > 1 else load_ratio[-1],
        "routed_experts_with_rows": int(np.count_nonzero(c > 0)),
        "weight_quant_ms": round(t_wq1 + t_wq2, 3),
        "wall_s_timed": round(wall, 3),
    }
    res.update(subs)
    if args.copy_calibration:
        res["copy_calibration"] = {"bytes_read": peaks["copy_bytes_read"],
                                   "bytes_written": peaks["copy_bytes_written"],
                                   "ms": peaks["copy_ms"],
                                   "GBps_read_plus_write": peaks["copy_GBps_read_plus_write"]}
    if not args.no_cpu_baseline and w.with_experts:
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
