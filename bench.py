#!/usr/bin/env python3
"""Benchmark of one tensor-parallel rank's share of a Megatron MLP block on MI355X.

Headline step (the pages' prefill shape, per rank): bf16, H=8192, F=32768,
T=8, rank 0's own weight blocks (F/T=4096), M=8192 tokens (4 sequences of
2048).  One step is the rank's column-parallel up-projection with fused
bias + GeLU (one launch) and its row-parallel down-projection into an fp32
partial (one launch).  ``value`` is that step's GEMM throughput in TFLOP/s
(4*M*H*F/T flops per step; GeLU is not counted), with every input resident
in HBM before timing starts.  Inputs are the seeded host draws the parity
tests use (N(0,1) tokens, N(0,0.02) weights, N(0,0.01) bias, bf16 RNE).

Timing: the headline warms up for at least 200 ms of GPU time (and at least
--warmup steps), then the K timed steps carry HIP events only at their two
ends (``ms_per_step``, ``value``); then 20 or more trials of 5 steps each
give the median and spread (``trials``); then K more steps with an event
before every launch give each kernel's mean duration (``kernels``) and the
roofline's ``achieved``.

Also reported on the same JSON line:
  roofline      the dominant kernel's algorithmic TFLOP/s (flops per launch /
                mean launch duration from HIP events on the launch stream)
                against the 2.5 PFLOP/s dense-bf16 MFMA peak, with its HBM
                traffic from the committed rocprofv3 counter runs
  decode        rank 0's MLP shard + attention out-projection shard at the
                pages' decode shape (H=8192, F/T=4096, A/T=1024, M in
                {1, 8, 32}), rotating over weight sets larger than the
                last-level cache: HBM GB/s and fraction of 8 TB/s, with the
                rank's all-reduce ring volume for context
  gpt_block_shard  the GPT-style block (H=4096, F=16384, T=4, M=2048): all 4
                shards in one launch per projection and the on-device sum
  stack80       80 layers (H=8192, F=32768, A=8192, T=8, whole group per
                layer) at decode M=8 (weight GB/s) and prefill M=4096 (TFLOP/s)
  variants      rank 0's exact-GeLU and gated Gate/Up first layer
  attention     rank 0's attention front half (Q/K/V projection, core, cache)
  backward      rank 0's backward pass
  hipblaslt_context  the column-parallel launches next to torch.matmul
                (hipBLASLt) on the same shapes, same GPU, same run
  cpu_baseline  the fp64 oracle on a bounded sample of the headline's token
                rows (extrapolated to all rows, labelled), and on the whole
                decode step at M = 32
  parity        the headline's sampled rows and the decode step's outputs
                against the oracle

Only one GPU is used: ``--gpus`` above 1 is refused.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "TFLOP/s per-rank MLP shard (prefill) + HBM GB/s (decode), % of roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources the prefill GEMM kernels are compiled from
GEMM_SOURCES = ["gemm_bf16.hip", "device_common.h", "tp_kernels.h"]


def source_sha(names):
    """Hash of one source file, or of a list of them (in order)."""
    h = hashlib.sha256()
    for name in ([names] if isinstance(names, str) else names):
        h.update(open(os.path.join(ROOT, "megatron_tensor_transformer_colpar_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed counter runs, or None if the
    kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != source_sha(rec["source"]):
        return None
    return {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
            "total_bytes": rec["fetch_bytes"] + rec["write_bytes"], "scale": rec["scale"],
            "profile": rec["profile"]}


def warm(torch, f, min_ms=30.0, max_calls=4000, min_calls=0):
    """Untimed warm-up: call f(k) (a section's own launches) until at least
    min_ms of GPU time has passed and at least min_calls calls were made.
    After the GPU idles for a moment (inputs being generated, a section
    starting), the first few ms of launches run at a lower clock; a fixed
    count of a few calls would time that ramp."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    k = 0
    while True:
        f(k)
        k += 1
        if k % 4 == 0 or k >= max_calls:
            e1.record()
            e1.synchronize()
            if (e0.elapsed_time(e1) >= min_ms and k >= min_calls) or k >= max_calls:
                return k


class Timeline:
    """Events recorded between launches on torch's current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self, label):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append((label, e))

    def durations(self):
        """label -> list of ms, for each launch that ends at the next mark."""
        out = {}
        for (label, a), (_, b) in zip(self.marks, self.marks[1:]):
            if label is not None:
                out.setdefault(label, []).append(a.elapsed_time(b))
        return out


def trials(torch, f, n_trials=20, per=5):
    """Median and spread of n_trials runs of `per` calls of f, each run timed
    with HIP events at its two ends only (ms per call)."""
    ts = []
    for _ in range(n_trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per):
            f()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / per)
    ts.sort()
    q = lambda p: ts[min(len(ts) - 1, int(round(p * (len(ts) - 1))))]
    return {"trials": n_trials, "calls_per_trial": per, "median_ms": round(q(0.5), 5), "p10_ms": round(q(0.1), 5),
            "p90_ms": round(q(0.9), 5), "min_ms": round(ts[0], 5), "max_ms": round(ts[-1], 5)}


def prefill_headline(args, torch, tp, inputs):
    """Rank 0's MLP share at the pages' prefill shape (H=8192, F=32768, T=8,
    F/T=4096, M=8192), on the seeded host inputs of the parity tests."""
    w = inputs.WORKLOADS["prefill"]
    M, H, Fs = w.M, w.H, w.F // w.T
    log("[bench] generating %s inputs (M=%d H=%d F/T=%d, rank 0)" % (w.name, M, H, Fs))
    X, W1, b1, W2 = inputs.mlp_inputs(w, shard_only=0)
    dX, dW1t, db1, dW2t = X.torch(), W1.transposed().torch(), b1.torch(), W2.transposed().torch()
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    BF = tp.TP_BF16

    # one step = rank 0's column-parallel GEMM with bias + GeLU, then its
    # row-parallel GEMM into the fp32 partial (rank-local weights: F := F/T, T := 1)
    def step(tl=None):
        if tl: tl.mark("gemm_up_gelu")
        tp.tp_colpar_gelu(dX, dW1t, db1, Y, M, H, Fs, 1, 0, BF, stream)
        if tl: tl.mark("gemm_rowpar_partial")
        tp.tp_rowpar_partial(Y, dW2t, Z, M, H, Fs, 1, 0, BF, stream)

    # warm-up: at least --warmup steps and at least 200 ms of GPU time (the
    # clock settles under the power cap only after sustained matrix work)
    nwarm = warm(torch, lambda k: step(), min_ms=200.0, min_calls=args.warmup)
    log("[bench] warm-up: %d steps" % nwarm)

    # timed region: K steps with events only at its two ends (an event
    # recorded between two launches holds the next launch back by a few us)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    # median and spread over 20 trials of 5 steps
    tri = trials(torch, step)
    # the same K steps with an event before every launch, for each kernel's
    # mean launch duration (the roofline's `achieved`)
    tl = Timeline(torch)
    torch.cuda.synchronize()
    tl.mark(None)
    for _ in range(args.steps):
        step(tl)
    tl.mark(None)
    torch.cuda.synchronize()
    ms_events = tl.marks[0][1].elapsed_time(tl.marks[-1][1]) / args.steps
    flops_step = 4.0 * M * H * Fs
    alg_bytes = {"gemm_up_gelu": 2.0 * (M * H + Fs * H + Fs) + 2.0 * M * Fs,
                 "gemm_rowpar_partial": 2.0 * (M * Fs + H * Fs) + 4.0 * M * H}
    kernels = {}
    for name, d in tl.durations().items():
        mean = sum(d) / len(d)
        fl = 2.0 * M * H * Fs
        kernels[name] = {"launches": len(d), "mean_us": round(mean * 1e3, 2), "flops_per_launch": fl,
                         "algorithmic_bytes_per_launch": alg_bytes[name],
                         "tflops": round(fl / (mean * 1e-3) / 1e12, 1)}
    log("[bench] prefill headline: %.4f ms/step, %.1f TFLOP/s (median of %d trials %.4f ms), wall %.3fs "
        "(%.4f ms/step with an event before every launch)"
        % (ms, flops_step / (ms * 1e-3) / 1e12, tri["trials"], tri["median_ms"], wall, ms_events))
    # leave one step's result in Y and Z for the parity check
    step()
    torch.cuda.synchronize()
    return dict(w=w, ms=ms, ms_events=ms_events, flops=flops_step, kernels=kernels, trials=tri, X=X, W1=W1,
                b1=b1, W2=W2, Y=Y, Z=Z, wall=wall, warmup_steps=nwarm)


def gpt_block_shard(args, torch, tp, inputs):
    w = inputs.WORKLOADS["gpt_block_shard"]
    M, H, F, T = w.M, w.H, w.F, w.T
    Fs = F // T
    log("[bench] generating %s inputs (M=%d H=%d F=%d T=%d)" % (w.name, M, H, F, T))
    X, W1, b1, W2 = inputs.mlp_inputs(w)
    dX, dW1t, db1, dW2t = X.torch(), W1.transposed().torch(), b1.torch(), W2.transposed().torch()
    Ys = [torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda") for _ in range(T)]
    Zs = [torch.empty(M, H, dtype=torch.float32, device="cuda") for _ in range(T)]
    Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
    yarr, zarr = tp.partial_array(Ys), tp.partial_array(Zs)
    stream = torch.cuda.current_stream().cuda_stream
    BF = tp.TP_BF16

    # one step = the 4 ranks' column-parallel GEMMs (one launch), their
    # row-parallel GEMMs (one launch) and the on-device sum of the partials
    def step(tl=None):
        if tl: tl.mark("gemm_up_gelu")
        tp.tp_colpar_gelu_group(dX, dW1t, db1, yarr, M, H, F, T, BF, stream)
        if tl: tl.mark("gemm_rowpar_partial")
        tp.tp_rowpar_partial_group(yarr, dW2t, zarr, M, H, F, T, BF, stream)
        if tl: tl.mark("shard_reduce")
        tp.tp_shard_reduce(zarr, T, None, Z, None, M, H, 0, stream)

    warm(torch, lambda k: step(), min_ms=100.0)

    # timed region: K steps with events only at its two ends (an event
    # recorded between two launches holds the next launch back by a few us,
    # which is measurement, not work) ...
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    # ... then the same K steps again with an event before every launch, for
    # each kernel's mean launch duration (the roofline's `achieved`)
    tl = Timeline(torch)
    torch.cuda.synchronize()
    tl.mark(None)
    for _ in range(args.steps):
        step(tl)
    tl.mark(None)
    torch.cuda.synchronize()
    ms_events = tl.marks[0][1].elapsed_time(tl.marks[-1][1]) / args.steps
    flops_step = 4.0 * M * H * F
    kernels = {}
    for name, d in tl.durations().items():
        mean = sum(d) / len(d)
        entry = {"launches": len(d), "mean_us": round(mean * 1e3, 2)}
        if name != "shard_reduce":
            fl = 2.0 * M * H * F           # all T shards in one launch
            entry["flops_per_launch"] = fl
            entry["tflops"] = round(fl / (mean * 1e-3) / 1e12, 1)
        else:
            by = (T + 1) * M * H * 4.0
            entry["bytes_per_launch"] = by
            entry["gbs"] = round(by / (mean * 1e-3) / 1e9, 1)
        kernels[name] = entry
    log("[bench] gpt_block_shard: %.4f ms/step, %.1f TFLOP/s, wall %.3fs (%.4f ms/step with an event before every "
        "launch)" % (ms, flops_step / (ms * 1e-3) / 1e12, wall, ms_events))

    # one rank's own launches (what a single rank's GPU runs): shard 0 alone
    def rank_step(tl):
        tl.mark("up")
        tp.tp_colpar_gelu(dX, dW1t, db1, Ys[0], M, H, F, T, 0, BF, stream)
        tl.mark("down")
        tp.tp_rowpar_partial(Ys[0], dW2t, Zs[0], M, H, F, T, 0, BF, stream)
    for _ in range(3):
        rank_step(Timeline(torch))
    tl2 = Timeline(torch)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        rank_step(tl2)
    tl2.mark(None)
    torch.cuda.synchronize()
    d2 = {k: sum(v) / len(v) for k, v in tl2.durations().items()}
    fl = 2.0 * M * H * Fs
    per_rank = {"workload": "shard 0 alone, M=%d H=%d F/T=%d" % (M, H, Fs),
                "up_us": round(d2["up"] * 1e3, 2), "down_us": round(d2["down"] * 1e3, 2),
                "up_tflops": round(fl / (d2["up"] * 1e-3) / 1e12, 1),
                "down_tflops": round(fl / (d2["down"] * 1e-3) / 1e12, 1)}
    t = flops_step / (ms * 1e-3) / 1e12
    return {"workload": "gpt_block_shard: all %d TP shards + on-device reduce, M=%d H=%d F=%d" % (T, M, H, F),
            "ms_per_step": round(ms, 4), "tflops": round(t, 1), "frac": round(t / PEAK_BF16_TFLOPS, 4),
            "ms_per_step_with_kernel_events": round(ms_events, 4), "kernels": kernels, "per_rank": per_rank}


def variants(args, torch, tp):
    """The exact-GeLU and gated Gate/Up first layers of rank 0: prefill at
    H=8192, F/T=4096, M=8192 (TFLOP/s; gated counts both projections) and the
    gated decode step at M=8 over rotating weight sets (weight GB/s).  Each
    figure is the median of 20 timed trials (one pass's mean is fragile
    against a single stall of the GPU at these call lengths); the decode
    step's pass mean is kept beside it."""
    g = torch.Generator(device="cuda").manual_seed(9)
    stream = torch.cuda.current_stream().cuda_stream
    H, Fs = 8192, 4096

    def bf(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    def median_ms(f, per):
        ctr = [0]

        def call():
            f(ctr[0])
            ctr[0] += 1
        warm(torch, lambda k: call())
        return trials(torch, call, n_trials=20, per=per)["median_ms"]

    out = {}
    M = 8192
    X, Wg, Wu, bg, bu = bf(M, H), bf(Fs, H, std=0.02), bf(Fs, H, std=0.02), bf(Fs, std=0.01), bf(Fs, std=0.01)
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
    fl = 2.0 * M * H * Fs
    ms = median_ms(lambda k: tp.tp_colpar_act(X, Wg, bg, Y, M, H, Fs, 1, 0, tp.TP_GELU_ERF, tp.TP_BF16, stream), 3)
    out["prefill_exact_gelu_tflops"] = round(fl / (ms * 1e-3) / 1e12, 1)
    ms = median_ms(lambda k: tp.tp_colpar_gated(X, Wg, Wu, bg, bu, Y, M, H, Fs, 1, 0, tp.TP_GELU_TANH, tp.TP_BF16,
                                                stream), 3)
    out["prefill_gated_tflops"] = round(2 * fl / (ms * 1e-3) / 1e12, 1)
    del X, Y
    M, R = 8, args.decode_sets
    sets = [(bf(Fs, H, std=0.02), bf(Fs, H, std=0.02)) for _ in range(R)]
    X = bf(M, H)
    Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")

    def gated_decode(k):
        tp.tp_colpar_gated(X, sets[k % R][0], sets[k % R][1], bg, bu, Y, M, H, Fs, 1, 0, tp.TP_GELU_TANH,
                           tp.TP_BF16, stream)
    ms = median_ms(gated_decode, R)
    n = max(2 * R, args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for k in range(n):
        gated_decode(k)
    e1.record()
    torch.cuda.synchronize()
    by = 2.0 * (2 * Fs * H + 2 * Fs) + M * H * 2 + M * Fs * 2
    out["decode_gated_m8_us"] = round(ms * 1e3, 2)
    out["decode_gated_m8_pass_mean_us"] = round(e0.elapsed_time(e1) / n * 1e3, 2)
    out["decode_gated_m8_gbs"] = round(by / (ms * 1e-3) / 1e9, 1)
    out["decode_gated_m8_frac"] = round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    out["workload"] = "rank 0 first layer, H=8192 F/T=4096: prefill M=8192, decode M=8"
    log("[bench] variants: %s" % out)
    return out


def attention(args, torch, tp):
    """The attention front half of rank 0 (8 heads of 128 at H=8192, T=8).
    Prefill, 4 sequences of 2048 tokens: the Q/K/V projection (one launch of
    three problems), causal attention on the matrix cores, the row-parallel
    out-projection (TFLOP/s; attention counts 4*d flops per visible
    query-key pair).  Decode, M sequences of 2048 cached positions, one new
    token each: the Q/K/V projection writing the new key and value rows into
    the caches, and split-key attention over the caches (HBM GB/s of weights
    or cache bytes; weight sets and caches rotate over more than 1 GiB, so
    every call streams from HBM; medians of 20 trials, since a single mean
    of these short calls moved by half between runs)."""
    g = torch.Generator(device="cuda").manual_seed(11)
    stream = torch.cuda.current_stream().cuda_stream
    H, As, D, nh = 8192, 1024, 128, 8

    def bf(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    def timed(f, n):
        warm(torch, f)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(n):
            f(k)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def median_ms(f, per):
        ctr = [0]

        def call():
            f(ctr[0])
            ctr[0] += 1
        warm(torch, lambda k: call())
        return trials(torch, call, n_trials=20, per=per)["median_ms"]

    def rate(flops, ms):
        t = flops / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 2), "tflops": round(t, 1), "frac": round(t / PEAK_BF16_TFLOPS, 4)}

    def bw(nbytes, ms):
        b = nbytes / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 2), "gbs": round(b, 1), "frac": round(b / PEAK_HBM_GBS, 4)}

    out = {}
    n = max(5, args.steps // 5)
    # ---- prefill
    Bs, S = 4, 2048
    M = Bs * S
    X = bf(M, H)
    Wq, Wk, Wv = (bf(As, H, std=0.02) for _ in range(3))
    Wo = bf(H, As, std=0.02)
    bq, bk, bv = bf(As, std=0.01), bf(As, std=0.01), bf(As, std=0.01)
    Q, K, V = (torch.empty(M, As, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    ctx = torch.empty(M, As, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
    qkv = lambda k: tp.tp_qkv_colpar(X, Wq, Wk, Wv, bq, bk, bv, Q, As, K, V, As, M, H, As, As, 1, 0, tp.TP_BF16,
                                     stream)
    core = lambda k: tp.tp_attn_core(Q, K, V, ctx, None, Bs, S, S, nh, nh, D, As, As, As, 1, None, 0, stream)
    oproj = lambda k: tp.tp_rowpar_partial(ctx, Wo, Z, M, H, As, 1, 0, tp.TP_BF16, stream)
    pairs = Bs * nh * S * (S + 1) / 2
    pre = {"workload": "rank 0, 4 sequences x 2048 tokens, H=8192, 8 heads x 128, causal",
           "qkv_projection": rate(2.0 * M * H * 3 * As, timed(qkv, n)),
           "attention_core": rate(4.0 * D * pairs, timed(core, n)),
           "out_projection": rate(2.0 * M * As * H, timed(oproj, n))}
    out["prefill"] = pre
    log("[bench] attention prefill: %s" % pre)
    del X, Q, K, V, ctx, Z, Wq, Wk, Wv, Wo
    torch.cuda.empty_cache()
    # ---- decode
    L = 2048
    R = args.decode_sets
    wsets = [(bf(As, H, std=0.02), bf(As, H, std=0.02), bf(As, H, std=0.02)) for _ in range(R)]
    dec = {}
    for Bs in (1, 8, 32):
        cache_bytes = Bs * L * As * 2 * 2
        C = max(2, -(-(1 << 30) // cache_bytes))
        caches = [(bf(Bs * L, As), bf(Bs * L, As)) for _ in range(C)]
        X = bf(Bs, H)
        Q = torch.empty(Bs, As, dtype=torch.bfloat16, device="cuda")
        ctx = torch.empty(Bs, As, dtype=torch.bfloat16, device="cuda")
        nws = tp.tp_attn_workspace_bytes(Bs, 1, L, nh, nh)
        ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")   # arrival counters start at zero

        def qkv(k):
            wq, wk, wv = wsets[k % R]
            kc, vc = caches[k % C]
            tp.tp_qkv_colpar(X, wq, wk, wv, bq, bk, bv, Q, As, kc[L - 1:], vc[L - 1:], L * As, Bs, H, As, As, 1, 0,
                             tp.TP_BF16, stream)

        def core(k):
            kc, vc = caches[k % C]
            tp.tp_attn_core(Q, kc, vc, ctx, None, Bs, 1, L, nh, nh, D, As, As, As, 1, ws, nws, stream)

        wbytes = 3.0 * (As * H * 2 + As * 2) + Bs * H * 2 + 3 * Bs * As * 2
        e = {"qkv_projection": bw(wbytes, median_ms(qkv, max(R, C))),
             "attention_core": bw(cache_bytes + 2.0 * Bs * As * 2, median_ms(core, C)),
             "cache_bytes": cache_bytes}
        dec["M=%d" % Bs] = e
        log("[bench] attention decode M=%d: %s" % (Bs, e))
        del caches, X, Q, ctx, ws
        torch.cuda.empty_cache()
    dec["workload"] = "rank 0, M sequences each with 2048 cached positions, 8 heads x 128, H=8192"
    out["decode"] = dec
    return out


def backward(args, torch, tp):
    """The backward pass of rank 0's MLP share (bf16, fp32 gradients): the
    training forward that keeps the GeLU input, then the input gradient fused
    with GeLU' (dU), the input-gradient partial dX, the weight gradients dW1
    and dW2 (each 2*M*H*F/T flops) and the bias gradient (a column sum,
    HBM-bound), at the 2048-token block shape (H=4096, F/T=4096) and the
    8192-token prefill shape (H=8192, F/T=4096).  An entry point called with
    the other outputs NULL launches one kernel, so each is timed on its own;
    dW2 is the whole row-parallel backward minus its dU launch."""
    g = torch.Generator(device="cuda").manual_seed(13)
    stream = torch.cuda.current_stream().cuda_stream
    T1 = tp.TP_GELU_TANH
    out = {}
    for label, M, H, Fs in (("gpt_block_shard rank 0: M=2048 H=4096 F/T=4096", 2048, 4096, 4096),
                            ("prefill rank 0: M=8192 H=8192 F/T=4096", 8192, 8192, 4096)):
        def bf(*shape, std=1.0):
            return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)
        X, W1t, b1, W2t, dZ = bf(M, H), bf(Fs, H, std=0.02), bf(Fs, std=0.01), bf(H, Fs, std=0.02), bf(M, H)
        Y, U, dU = (torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda") for _ in range(3))
        dX = torch.empty(M, H, dtype=torch.float32, device="cuda")
        dW1t = torch.empty(Fs, H, dtype=torch.float32, device="cuda")
        db1 = torch.empty(Fs, dtype=torch.float32, device="cuda")
        dW2t = torch.empty(H, Fs, dtype=torch.float32, device="cuda")
        ops = [("forward_train", lambda: tp.tp_colpar_act_train(X, W1t, b1, Y, U, M, H, Fs, 1, 0, T1, stream)),
               ("dU", lambda: tp.tp_rowpar_bwd(dZ, W2t, Y, U, dU, None, M, H, Fs, 1, 0, T1, 0, stream)),
               ("dU+dW2", lambda: tp.tp_rowpar_bwd(dZ, W2t, Y, U, dU, dW2t, M, H, Fs, 1, 0, T1, 0, stream)),
               ("dX", lambda: tp.tp_colpar_bwd(X, W1t, dU, dX, None, None, M, H, Fs, 1, 0, 0, stream)),
               ("dW1", lambda: tp.tp_colpar_bwd(X, W1t, dU, None, dW1t, None, M, H, Fs, 1, 0, 0, stream)),
               ("db1", lambda: tp.tp_colpar_bwd(X, W1t, dU, None, None, db1, M, H, Fs, 1, 0, 0, stream)),
               ("backward", lambda: tp.tp_mlp_shard_bwd(X, W1t, W2t, U, Y, dZ, dU, dX, dW1t, db1, dW2t, M, H, Fs, 1,
                                                        0, T1, 0, stream))]
        ms = {}
        n = max(3, args.steps // 5)
        for name, f in ops:
            warm(torch, lambda k: f())
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(n):
                f()
            e1.record()
            torch.cuda.synchronize()
            ms[name] = e0.elapsed_time(e1) / n
        ms["dW2"] = ms.pop("dU+dW2") - ms["dU"]
        fl = 2.0 * M * H * Fs
        e = {}
        for name in ("forward_train", "dU", "dX", "dW1", "dW2"):
            t = fl / (ms[name] * 1e-3) / 1e12
            e[name] = {"us": round(ms[name] * 1e3, 2), "tflops": round(t, 1), "frac": round(t / PEAK_BF16_TFLOPS, 4)}
        e["dW2"]["derived"] = "row-parallel backward minus its dU launch"
        by = M * Fs * 2 + Fs * 4
        e["db1"] = {"us": round(ms["db1"] * 1e3, 2), "gbs": round(by / (ms["db1"] * 1e-3) / 1e9, 1),
                    "frac": round(by / (ms["db1"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        t = 4 * fl / (ms["backward"] * 1e-3) / 1e12
        e["backward"] = {"us": round(ms["backward"] * 1e3, 2), "tflops": round(t, 1),
                         "frac": round(t / PEAK_BF16_TFLOPS, 4)}
        out[label] = e
        log("[bench] backward %s: %s" % (label, e))
        del X, W1t, b1, W2t, dZ, Y, U, dU, dX, dW1t, db1, dW2t
        torch.cuda.empty_cache()
    # the whole group of the 2048-token block (T=4): training forward and
    # backward, one launch per projection over all ranks, then the backward
    # all-reduce of the dX partials
    M, H, F, T = 2048, 4096, 16384, 4
    Fs = F // T
    X, W1t, b1, W2t, dZ = (torch.randn(*sh, generator=g, device="cuda").mul(sd).to(torch.bfloat16)
                           for sh, sd in (((M, H), 1.0), ((F, H), 0.02), ((F,), 0.01), ((H, F), 0.02), ((M, H), 1.0)))
    Ys, Us, dUs = ([torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda") for _ in range(T)] for _ in range(3))
    dXs = [torch.empty(M, H, dtype=torch.float32, device="cuda") for _ in range(T)]
    dXsum = torch.empty(M, H, dtype=torch.float32, device="cuda")
    dW1t = torch.empty(F, H, dtype=torch.float32, device="cuda")
    db1 = torch.empty(F, dtype=torch.float32, device="cuda")
    dW2t = torch.empty(H, F, dtype=torch.float32, device="cuda")
    ya, ua, da, xa = (tp.partial_array(v) for v in (Ys, Us, dUs, dXs))
    fwd = lambda: tp.tp_mlp_group_fwd_train(X, W1t, b1, ya, ua, M, H, F, T, T1, stream)
    bwd = lambda: tp.tp_mlp_group_bwd(X, W1t, W2t, ua, ya, dZ, da, xa, dW1t, db1, dW2t, M, H, F, T, T1, 0, stream)
    red = lambda: tp.tp_shard_reduce(xa, T, None, dXsum, None, M, H, 0, stream)
    ms = {}
    n = max(3, args.steps // 5)
    for name, f in (("forward_train", fwd), ("backward", bwd), ("dX_reduce", red)):
        warm(torch, lambda k: f())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / n
    fl = 2.0 * M * H * F
    grp = {"workload": "gpt_block_shard, all 4 ranks: M=2048 H=4096 F=16384 T=4"}
    t = fl / (ms["forward_train"] * 1e-3) / 1e12
    grp["forward_train"] = {"us": round(ms["forward_train"] * 1e3, 2), "tflops": round(t, 1),
                            "frac": round(t / PEAK_BF16_TFLOPS, 4)}
    t = 4 * fl / (ms["backward"] * 1e-3) / 1e12
    grp["backward"] = {"us": round(ms["backward"] * 1e3, 2), "tflops": round(t, 1), "frac": round(t / PEAK_BF16_TFLOPS, 4)}
    by = (T + 1) * M * H * 4
    grp["dX_reduce"] = {"us": round(ms["dX_reduce"] * 1e3, 2), "gbs": round(by / (ms["dX_reduce"] * 1e-3) / 1e9, 1)}
    out["group"] = grp
    log("[bench] backward group: %s" % grp)
    del X, W1t, b1, W2t, dZ, Ys, Us, dUs, dXs, dXsum, dW1t, db1, dW2t
    torch.cuda.empty_cache()
    return out


def hipblaslt_context(args, torch, tp):
    """The library's column-parallel launches next to hipBLASLt (torch.matmul,
    bf16 out, no bias or GeLU) on the same shapes, timed alternately on the
    same GPU.  Context for the roofline figures only; never the reported value."""
    g = torch.Generator(device="cuda").manual_seed(7)
    stream = torch.cuda.current_stream().cuda_stream

    def timed(f, reps=20):
        warm(torch, lambda k: f())
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def bf(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device="cuda") * std).to(torch.bfloat16)

    out = {}
    for label, M, H, F, T in (("gpt_block_shard column-parallel, 4 shards", 2048, 4096, 16384, 4),
                              ("prefill column-parallel, rank 0", 8192, 8192, 4096, 1)):
        X, W1t, b1 = bf(M, H), bf(F, H, std=0.02), bf(F, std=0.01)
        Ys = [torch.empty(M, F // T, dtype=torch.bfloat16, device="cuda") for _ in range(T)]
        W1 = W1t.t().contiguous()
        lib = lambda: tp.tp_colpar_gelu_group(X, W1t, b1, Ys, M, H, F, T, tp.TP_BF16, stream)
        ref = lambda: torch.matmul(X, W1)
        a, b = [], []
        for _ in range(2):
            a.append(timed(lib))
            b.append(timed(ref))
        fl = 2.0 * M * H * F
        out[label] = {"library_tflops": round(fl / (min(a) * 1e-3) / 1e12, 1),
                      "hipblaslt_tflops": round(fl / (min(b) * 1e-3) / 1e12, 1)}
        del X, W1t, b1, Ys, W1
    log("[bench] hipBLASLt context: %s" % out)
    return out


def decode(args, torch, tp, inputs):
    """Rank 0's decode step at the pages' decode shape: H=8192, F/T=4096,
    A/T=1024 (8 heads of 128), M in {1, 8, 32} tokens: the MLP shard
    (column-parallel up-projection with bias + GeLU, row-parallel partial)
    and the head-sharded out-projection partial.  R weight sets rotate so
    that every call streams its weights from HBM (R * 144 MiB is more than
    4x the 256 MB last-level cache); set 0 is the seeded host draw of the
    parity tests, and its outputs are kept for the oracle check."""
    w = inputs.WORKLOADS["decode"]
    H, Fs, As, R = w.H, w.F // w.T, w.A // w.T, args.decode_sets
    X, W1, b1, W2 = inputs.mlp_inputs(w, shard_only=0)          # X: 32 token rows
    ctx, Wo = inputs.outproj_inputs(w, shard=0)
    host = dict(X=X, W1=W1, b1=b1, W2=W2, ctx=ctx, Wo=Wo)
    g = torch.Generator(device="cuda").manual_seed(3)
    sets = [dict(W1t=W1.transposed().torch(), b1=b1.torch(), W2t=W2.transposed().torch(), Wot=Wo.transposed().torch())]
    for _ in range(R - 1):
        sets.append(dict(
            W1t=(torch.randn(Fs, H, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
            b1=(torch.randn(Fs, generator=g, device="cuda") * 0.01).to(torch.bfloat16),
            W2t=(torch.randn(H, Fs, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
            Wot=(torch.randn(H, As, generator=g, device="cuda") * 0.02).to(torch.bfloat16)))
    stream = torch.cuda.current_stream().cuda_stream
    dX, dctx = X.torch(), ctx.torch()
    res, outs = {}, {}
    for M in (1, 8, 32):
        Y = torch.empty(M, Fs, dtype=torch.bfloat16, device="cuda")
        Z = torch.empty(M, H, dtype=torch.float32, device="cuda")
        O = torch.empty(M, H, dtype=torch.float32, device="cuda")

        def step(s, tl=None):
            if tl: tl.mark("up")
            tp.tp_colpar_gelu(dX, s["W1t"], s["b1"], Y, M, H, Fs, 1, 0, tp.TP_BF16, stream)
            if tl: tl.mark("down")
            tp.tp_rowpar_partial(Y, s["W2t"], Z, M, H, Fs, 1, 0, tp.TP_BF16, stream)
            if tl: tl.mark("outproj")
            tp.tp_rowpar_partial(dctx, s["Wot"], O, M, H, As, 1, 0, tp.TP_BF16, stream)

        warm(torch, lambda k: step(sets[k % R]))
        n = max(2 * R, args.steps)
        # the step itself, with events only around the whole run (an event
        # between two launches adds a gap of its own) ...
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(n):
            step(sets[k % R])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / n
        ctr = [0]

        def rotating():
            step(sets[ctr[0] % R])
            ctr[0] += 1
        tri = trials(torch, rotating, n_trials=20, per=R)
        # ... and a second run with an event before each launch for the
        # per-kernel durations
        tl = Timeline(torch)
        torch.cuda.synchronize()
        tl.mark(None)
        for k in range(n):
            step(sets[k % R], tl)
        tl.mark(None)
        torch.cuda.synchronize()
        mlp_bytes = 2.0 * (Fs * H * 2 + Fs) + M * H * 2 + M * H * 4
        op_bytes = 2.0 * H * As + M * As * 2 + M * H * 4
        by = mlp_bytes + op_bytes
        d = {k: sum(v) / len(v) for k, v in tl.durations().items()}
        e = {"us_per_step": round(ms * 1e3, 2), "bytes_per_step": by,
             "gbs": round(by / (ms * 1e-3) / 1e9, 1),
             "frac": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "median_us": round(tri["median_ms"] * 1e3, 2),
             "median_frac": round(by / (tri["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "p10_us": round(tri["p10_ms"] * 1e3, 2), "p90_us": round(tri["p90_ms"] * 1e3, 2),
             "trials": tri["trials"],
             "up_us": round(d["up"] * 1e3, 2), "down_us": round(d["down"] * 1e3, 2),
             "outproj_us": round(d["outproj"] * 1e3, 2),
             "mlp_kernels_gbs": round(mlp_bytes / ((d["up"] + d["down"]) * 1e-3) / 1e9, 1)}
        res["M=%d" % M] = e
        log("[bench] decode M=%d: %s" % (M, e))
        # the host set's outputs for the oracle check
        step(sets[0])
        torch.cuda.synchronize()
        outs[M] = (Y.clone(), Z.clone(), O.clone())
    # context: what the rank's two all-reduces per layer would move on a real
    # TP group (ring, bf16 payload), per decode step
    from megatron_tensor_transformer_colpar_amd import comm_volume as cv
    res["allreduce_ring_bytes_per_rank"] = {"M=%d" % M: int(2 * cv.ring_allreduce_bytes_per_rank(H, 2, w.T, tokens=M))
                                            for M in (1, 8, 32)}
    res["workload"] = ("rank 0 of T=8: H=8192, F/T=4096, A/T=1024; MLP shard + head-sharded out-projection; "
                       "%d rotating weight sets" % R)
    return res, dict(host, outs=outs)


def stack80(args, torch, tp):
    """The 80-layer stack (H=8192, F=32768, A=64x128, T=8), the whole TP group
    emulated: per layer all 8 ranks' out-projection partials, the reduce into
    the residual stream (with its row-RMS bf16 copy), all 8 ranks' MLP shares,
    the second reduce.  Independent seeded weights per layer."""
    L, H, F, A, T = 80, 8192, 32768, 8192, 8
    g = torch.Generator(device="cuda").manual_seed(80)
    layers = []
    for _ in range(L):
        layers.append(dict(Wot=(torch.randn(H, A, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
                           W1t=(torch.randn(F, H, generator=g, device="cuda") * 0.02).to(torch.bfloat16),
                           b1=(torch.randn(F, generator=g, device="cuda") * 0.01).to(torch.bfloat16),
                           W2t=(torch.randn(H, F, generator=g, device="cuda") * 0.02).to(torch.bfloat16)))
    stream = torch.cuda.current_stream().cuda_stream
    out = {"workload": "80 layers, H=8192 F=32768 A=8192 T=8, all 8 ranks per layer"}
    wbytes = L * (2.0 * (H * A + 2 * F * H + F))
    for M, steps in ((8, max(3, args.steps // 5)), (4096, 2)):
        ctx_t = [[torch.randn(M, A // T, generator=g, device="cuda").to(torch.bfloat16) for _ in range(T)]
                 for _ in range(L)]
        ctx = [tp.partial_array(c) for c in ctx_t]
        x0 = torch.randn(M, H, generator=g, device="cuda")
        h = torch.empty(M, H, dtype=torch.float32, device="cuda")
        xhat = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
        Y_t = [torch.empty(M, F // T, dtype=torch.bfloat16, device="cuda") for _ in range(T)]
        P_t = [torch.empty(M, H, dtype=torch.float32, device="cuda") for _ in range(T)]
        Y, parts = tp.partial_array(Y_t), tp.partial_array(P_t)

        def step():
            h.copy_(x0)
            for l, p in enumerate(layers):
                tp.tp_layer_fwd(h, xhat, ctx[l], p["Wot"], A, p["W1t"], p["b1"], p["W2t"], Y, parts, M, H, F, T,
                                stream)

        step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flops = L * (2.0 * M * A * H + 4.0 * M * H * F)
        e = {"steps": steps, "ms_per_step_group": round(ms, 3), "ms_per_step_per_rank_share": round(ms / T, 3),
             "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        if M == 8:
            from megatron_tensor_transformer_colpar_amd import comm_volume as cv
            e["weight_gbs"] = round(wbytes / (ms * 1e-3) / 1e9, 1)
            e["frac_hbm"] = round(wbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            e["us_per_token"] = round(ms * 1e3 / M, 2)
            # context: a real TP group's ring all-reduces (2 per layer, bf16) per rank per step
            e["allreduce_ring_bytes_per_rank"] = int(cv.stack_ring_bytes_per_rank(L, H, 2, T, tokens=M))
        else:
            e["frac_mfma"] = round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        out["M=%d" % M] = e
        log("[bench] stack80 M=%d: %s" % (M, e))
        assert bool(torch.isfinite(h).all()), "stack80 produced non-finite values"
    del layers
    torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo, or None where it is not readable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(args, hl, dec, stack=False):
    """The fp64 oracle on the host cores, timed on bounded samples of the
    bench's own inputs, and the GPU outputs of those inputs checked against
    it.  Prefill: a seeded sample of the headline's token rows, sized to take
    about --cpu-seconds (no step of the block mixes rows, so the time
    extrapolates linearly to all rows; labelled).  Decode: the whole M = 32
    step (MLP shard + out-projection shard).  With `stack`, one layer of the
    80-layer stack as well (cpu_stack80)."""
    import numpy as np

    import oracle
    from megatron_tensor_transformer_colpar_amd import inputs

    w = hl["w"]
    M, H, Fs = w.M, w.H, w.F // w.T
    W1, b1, W2 = hl["W1"].f64, hl["b1"].f64, hl["W2"].f64
    flops_row = 4.0 * H * Fs

    def run(rows):
        Xr = hl["X"].f64[rows]
        t0 = time.perf_counter()
        Yr, Zr = oracle.mlp_shard(Xr, W1, b1, W2, 1, 0)
        return time.perf_counter() - t0, Yr, Zr

    # the oracle threads over rows: probe with two rows per thread so that
    # the rate it measures is the one the full sample will see
    probe = inputs.row_sample(M, max(16, 2 * oracle.max_threads()), seed=1, include_ends=False)
    dt, _, _ = run(probe)
    n = int(min(M, max(32, len(probe) * args.cpu_seconds / max(dt, 1e-3))))
    rows = inputs.row_sample(M, n, seed=2)
    dt, Yr, Zr = run(rows)
    tflops = len(rows) * flops_row / dt / 1e12
    rel = lambda got, want: float(np.linalg.norm(got - want) / np.linalg.norm(want))
    ey = rel(hl["Y"].float().cpu().double().numpy()[rows], Yr)
    ez = rel(hl["Z"].double().cpu().numpy()[rows], Zr)
    log("[bench] cpu oracle, prefill: %d rows in %.2fs (%.3f GFLOP/s), parity Y %.2e Z %.2e"
        % (len(rows), dt, tflops * 1e3, ey, ez))
    cb = {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
          "sample": "%d of %d token rows of the headline step (rank 0's MLP shard, fp64), %.1f s; "
                    "all %d rows extrapolated: %.1f s" % (len(rows), M, dt, M, dt * M / len(rows)),
          "extrapolated_s_all_rows": round(dt * M / len(rows), 2), "cpu_model": cpu_model()}
    par = {"prefill": {"rows": len(rows), "rel_fro_Y": ey, "rel_fro_Z": ez, "tol": 5e-3,
                       "ok": ey <= 5e-3 and ez <= 5e-3}}
    if dec is not None:
        d = dec
        t0 = time.perf_counter()
        Yd, Zd = oracle.mlp_shard(d["X"].f64, d["W1"].f64, d["b1"].f64, d["W2"].f64, 1, 0)
        Od = oracle.rowpar_partial(d["ctx"].f64, d["Wo"].f64, 1, 0)
        dtd = time.perf_counter() - t0
        Md, Hd, Fsd, Asd = d["X"].shape[0], d["X"].shape[1], d["W1"].shape[1], d["ctx"].shape[1]
        by = 2.0 * (2 * Fsd * Hd + Fsd + Asd * Hd) + Md * (Hd * 2 + Asd * 2 + 2 * Hd * 4)
        cb["decode"] = {"value": round(by / dtd / 1e9, 4), "unit": "GB/s", "seconds": round(dtd, 3),
                        "sample": "the whole decode step at M=%d (MLP shard + out-projection shard, fp64)" % Md}
        errs = {}
        for m, (Y, Z, O) in d["outs"].items():
            errs["M=%d" % m] = {"Y": rel(Y.float().cpu().double().numpy(), Yd[:m]),
                                "Z": rel(Z.double().cpu().numpy(), Zd[:m]),
                                "O": rel(O.double().cpu().numpy(), Od[:m])}
        par["decode"] = {"rel_fro": errs, "tol": 5e-3,
                         "ok": all(v <= 5e-3 for e in errs.values() for v in e.values())}
        log("[bench] cpu oracle, decode: %.2fs, parity %s" % (dtd, errs))
    if stack:
        cb["stack80"] = cpu_stack80()
    return cb, par


def cpu_stack80():
    """The fp64 oracle on one layer of the 80-layer stack (H=8192, F=32768,
    A=8192, T=8, the whole TP group: out-projection partials, reduce with
    residual and RMS copy, MLP partials, reduce), on layer 0's seeded host
    weights: the decode layer at M=8 in full, and a 32-row sample of the
    prefill layer at M=4096.  Every layer has the same shape and no step of a
    layer mixes token rows, so the step times extrapolate linearly to 80
    layers and to all rows (labelled)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from megatron_tensor_transformer_colpar_amd import inputs

    w = inputs.WORKLOADS["stack80"]
    H, F, A, T, L = w.H, w.F, w.A, w.T, w.layers
    As = A // T
    kw = dict(workload=w.wid, layer=0)
    jobs = {"Wo": ((A, H), w.w_std, inputs.WO_ID), "W1": ((H, F), w.w_std, inputs.W1_ID),
            "b1": ((F,), w.b_std, inputs.B1_ID), "W2": ((F, H), w.w_std, inputs.W2_ID)}
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {k: ex.submit(inputs.normal, shape, std, "bf16", tensor=tid, **kw) for k, (shape, std, tid) in jobs.items()}
        wt = {k: f.result().f64 for k, f in futs.items()}     # converted to fp64 once, outside the timing
    out = {}
    flops_row = 2.0 * A * H + 4.0 * H * F            # the whole group's GEMM flops per token row
    wbytes = 2.0 * (H * A + 2 * F * H + F)            # the layer's bf16 weights
    for label, M, rows in (("decode", 8, 8), ("prefill", 4096, 32)):
        h = inputs.normal((rows, H), 1.0, "f32", tensor=inputs.X_ID, **kw).f64
        ctx = [inputs.normal((rows, As), 1.0, "bf16", tensor=inputs.CTX_ID, shard=i + 1, **kw).f64 for i in range(T)]
        t0 = time.perf_counter()
        oracle.layer_fwd(h, ctx, wt["Wo"], wt["W1"], wt["b1"], wt["W2"], T, 1e-6)
        dt = time.perf_counter() - t0
        step_s = dt * (M / rows) * L
        e = {"layer_seconds": round(dt, 3), "rows": rows, "M": M, "cores": oracle.max_threads(),
             "extrapolated_step_s_group": round(step_s, 2), "extrapolated_step_s_per_rank_share": round(step_s / T, 2),
             "tflops": round(rows * flops_row / dt / 1e12, 5)}
        if label == "decode":
            e["weight_gbs"] = round(L * wbytes / step_s / 1e9, 3)
            e["sample"] = "one layer of the whole TP group at M=8 (every row), fp64; x 80 layers extrapolated"
        else:
            e["sample"] = "32 of 4096 token rows of one layer of the whole TP group, fp64; x 4096/32 rows x 80 layers extrapolated"
        out[label] = e
        log("[bench] cpu oracle, stack80 %s: %s" % (label, e))
    return out


def copy_scale(kib):
    """Scale of a byte counter from its per-dispatch readings (KiB) for the
    runtime's copy kernel: the three 1 GiB calibration copies are the large
    readings; the runtime's own small copies in the same run (a few KiB) are
    left out."""
    big = [v for v in kib if v >= 0.25 * max(kib)]
    if len(big) != 3:
        raise ValueError("expected the three 1 GiB calibration copies, found %d large copies" % len(big))
    return round(1048576.0 / (sum(big) / len(big)), 4)


def write_traffic(prof_dir):
    """profiles/traffic.json from two rocprofv3 --pmc runs of the headline
    (FETCH_SIZE under <prof_dir>/pmcf, WRITE_SIZE under <prof_dir>/pmcw),
    each run starting with --copy-calibration: the counters are scaled by
    what they read for a plain 1 GiB copy (1 GiB read, 1 GiB written)."""
    import csv
    import re
    from collections import defaultdict

    def load(path):
        d = defaultdict(list)
        for r in csv.DictReader(open(path)):
            name = r["Kernel_Name"]
            m = re.search(r"(\w+<[^>]*>)\(", name)
            d[m.group(1) if m else name.split("(")[0]].append(float(r["Counter_Value"]))
        return d

    F = load(os.path.join(prof_dir, "pmcf", "p_counter_collection.csv"))
    W = load(os.path.join(prof_dir, "pmcw", "p_counter_collection.csv"))
    sf = copy_scale(F["__amd_rocclr_copyBuffer"])
    sw = copy_scale(W["__amd_rocclr_copyBuffer"])
    M, H, Fs = 8192, 8192, 4096
    alg = {"gemm_up_gelu": 2 * (M * H + Fs * H + Fs) + 2 * M * Fs, "gemm_rowpar_partial": 2 * (M * Fs + H * Fs) + 4 * M * H}
    # the headline's two launches: 256x256 tiles, 8 waves, epilogue 0 (bias +
    # GeLU) and 1 (fp32 partial), K-contiguous operands
    def pick(epi):
        for name in F:
            args = [a.strip() for a in name[name.find("<") + 1:name.rfind(">")].split(",")]
            if name.startswith("gemm_bf16_kernel<") and args[:5] == ["256", "256", "64", "2", "8"] and \
                    args[6:8] == [str(epi), "0"]:
                return name
        raise KeyError("no headline kernel with epilogue %d in the counter runs" % epi)
    kern = {"gemm_up_gelu": pick(0), "gemm_rowpar_partial": pick(1)}
    try:
        out = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        out = {}
    for key, k in kern.items():
        fr, wr = sum(F[k]) / len(F[k]), sum(W[k]) / len(W[k])
        out[key + "@prefill"] = {"source": GEMM_SOURCES, "source_sha": source_sha(GEMM_SOURCES),
                                 "kernel": k, "fetch_kib_raw": round(fr), "write_kib_raw": round(wr),
                                 "fetch_bytes": round(fr * 1024 * sf), "write_bytes": round(wr * 1024 * sw),
                                 "scale": {"fetch": sf, "write": sw}, "algorithmic_bytes": alg[key],
                                 "dispatches": len(F[k]), "profile": "profiles/gemm_prefill_rank0_h8192.md"}
        print(key, json.dumps(out[key + "@prefill"]))
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # a minimum: the headline also warms up for at least 200 ms of GPU time
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-sets", type=int, default=8)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline step only (for profiling)")
    ap.add_argument("--sections",
                    default="decode,gpt_block_shard,stack80,variants,attention,backward,context",
                    help="comma-separated extra sections to run after the headline step")
    ap.add_argument("--context-only", action="store_true",
                    help="only the library-vs-hipBLASLt comparison (for counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy 3 times (reference for HBM byte counters)")
    ap.add_argument("--write-traffic", metavar="PROF_DIR",
                    help="write profiles/traffic.json from the FETCH_SIZE/WRITE_SIZE counter runs under PROF_DIR "
                         "(CPU only) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return

    import torch

    from megatron_tensor_transformer_colpar_amd import inputs, tp

    torch.cuda.set_device(0)
    if args.context_only:
        print(json.dumps({"hipblaslt_context": hipblaslt_context(args, torch, tp)}), flush=True)
        return
    if args.copy_calibration:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    hl = prefill_headline(args, torch, tp, inputs)
    kernels = hl["kernels"]
    dom = max(kernels, key=lambda k: kernels[k]["mean_us"])
    ach = kernels[dom]["tflops"]
    traffic = measured_traffic(dom + "@prefill")
    roof = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else traffic["total_bytes"],
            "flops_per_launch": kernels[dom]["flops_per_launch"],
            "algorithmic_bytes_per_launch": kernels[dom]["algorithmic_bytes_per_launch"],
            "mean_launch_us": kernels[dom]["mean_us"]}
    if traffic is not None:
        roof["traffic_detail"] = traffic
    value = hl["flops"] / (hl["ms"] * 1e-3) / 1e12
    w = hl["w"]
    rec = {"metric": METRIC, "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(hl["ms"], 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic: seeded N(0,1) activations, N(0,0.02) weights, N(0,0.01) bias (bf16 RNE)",
           "config": {"workload": "prefill, rank 0 of T=8: H=8192, F=32768 (F/T=4096), M=8192 tokens "
                                  "(4 x 2048); column-parallel GEMM + bias + GeLU, row-parallel fp32 partial",
                      "M": w.M, "H": w.H, "F": w.F, "T": w.T, "shard": 0, "parallelism": "tp8, rank 0's share"},
           "frac": round(value / PEAK_BF16_TFLOPS, 4),
           "roofline": roof, "kernels": kernels, "trials": hl["trials"], "warmup_steps_run": hl["warmup_steps"],
           "median_tflops": round(hl["flops"] / (hl["trials"]["median_ms"] * 1e-3) / 1e12, 1),
           "ms_per_step_with_kernel_events": round(hl["ms_events"], 4)}
    sections = set() if args.no_extras else set(x for x in args.sections.split(",") if x)
    dec_host = None
    if "decode" in sections:
        rec["decode"], dec_host = decode(args, torch, tp, inputs)
        fr = {k: v["frac"] for k, v in rec["decode"].items() if k.startswith("M=")}
        rec["decode"]["roofline"] = {"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                     "achieved": {k: v["gbs"] for k, v in rec["decode"].items() if k.startswith("M=")},
                                     "frac": fr}
    torch.cuda.empty_cache()
    if "gpt_block_shard" in sections:
        rec["gpt_block_shard"] = gpt_block_shard(args, torch, tp, inputs)
        torch.cuda.empty_cache()
    if "stack80" in sections:
        rec["stack80"] = stack80(args, torch, tp)
    if "variants" in sections:
        rec["variants"] = variants(args, torch, tp)
    if "attention" in sections:
        rec["attention"] = attention(args, torch, tp)
        torch.cuda.empty_cache()
    if "backward" in sections:
        rec["backward"] = backward(args, torch, tp)
    if "context" in sections:
        rec["hipblaslt_context"] = hipblaslt_context(args, torch, tp)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["parity"] = cpu_baseline(args, hl, dec_host, stack="stack80" in sections)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
