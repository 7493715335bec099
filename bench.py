"""Benchmark of the gated-delta-rule forward on one MI355X.

A step is one pass of the prefill hot path over one batch of the bf16 prefill
workload (B=4, H=16, T=4096, K=V=128): causal conv1d + SiLU over the q|k|v
channels (C = 6144), gate preparation, and the chunked forward (per-chunk WY
solve, then the sequential state scan with the outputs and the final state),
run as the library's whole-prefill entry in its two phases: the per-chunk
solve (convolving the q and k rows and forming the gates itself) and the scan
(convolving the value rows as it reads them). Inputs are resident in HBM
before timing starts. `value` is tokens/s of the whole step (16,384 tokens
per step). The same computation is also timed as the four per-step calls
(conv1d, gates, chunk_prepare, chunk_scan; `chain`), whose chunk_prepare +
chunk_scan is the chunked forward on resident q, k, v, g, beta
(`chain.chunk_fwd`: tokens/s and fractions of the MFMA and HBM peaks). The one-token Gated
DeltaProduct decode (n=256 requests, M=2, H=32, G=16, P=N=128, 1000 steps,
fp32 state updated in place) and the steps around it are reported beside it.

Per-kernel durations come from HIP events recorded between the launches on
the stream the kernels run on (torch's current stream, which the binding
passes to the library). `roofline` describes the kernel that takes the most
time per step; `traffic` comes from committed rocprofv3 counter summaries
(profiles/traffic.json) and is null when absent or when the kernel's source
has changed since they were taken.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu] [--no-chain]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = "linear_attention_ssm_amd/csrc/"
KERNELS = {   # bench op -> (kernel symbol stem, source file)
    "prefill_prepare": ("chunk_prep_kernelIDF16bLi128ELb1ELb1E", CSRC + "chunk.hip"),
    "prefill_scan": ("chunk_scan_roles_kernel<128, 2, 3, true>", CSRC + "chunk.hip"),
    "decode": ("gdp_decode_kernel", CSRC + "decode.hip"),
}
REC_BYTES_BF16 = 2 * 6 * 64 * 16 + 4 * 64 * 4   # per (chunk, value head) workspace record


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # (the GPU needs some tens of milliseconds of work to reach its sustained
    # clock: 10 warm-up steps time 10% slow, 200 (about 35 ms) do not)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--decode-steps", type=int, default=1000)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-batch", type=int, default=4,
                   help="sequences of the prefill workload the oracle baseline runs (4 = all)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration runs)")
    p.add_argument("--only", choices=["prefill", "decode"], default=None)
    p.add_argument("--no-flush", action="store_true",
                   help="skip the per-iteration timings with the caches flushed between "
                        "iterations (profiling runs: every traced launch then runs warm, as in "
                        "the timed steps)")
    p.add_argument("--no-chain", action="store_true",
                   help="skip the four-call chain (conv1d, gates, chunk_prepare, chunk_scan)")
    p.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_STATS_CSV", "OUT_MD"),
                   help="turn a rocprofv3 --stats kernel_stats.csv into a profiles/ summary")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (made with "
                        "--copy-probe) into profiles/traffic.json")
    p.add_argument("--summarize-mfma", nargs=2, metavar=("COUNTER_CSV", "OUT_MD"),
                   help="write the MFMA-busy summary of a --pmc SQ_VALU_MFMA_BUSY_CYCLES "
                        "SQ_INSTS_MFMA GRBM_GUI_ACTIVE run")
    p.add_argument("--command", default="", help="the command that produced the CSVs")
    p.add_argument("--bench-log", default=None,
                   help="with --summarize-stats: the profiled run's output, whose bench line "
                        "gives the same run's kernel times measured with HIP events")
    return p.parse_args()


def prefill_accounting(B, T, H, Hk, K, V):
    """Algorithmic HBM bytes (and MFMA flops) per launch of each prefill kernel:
    every input read once, every output written once."""
    C = 2 * Hk * K + H * V
    tok = B * T
    chunks = B * ((T + 63) // 64)
    qk = 2 * tok * Hk * K * 2
    v = tok * H * V * 2
    o = tok * H * V * 2
    gb = 2 * tok * H * 4
    state = B * H * K * V * 4
    rec = chunks * H * REC_BYTES_BF16
    d, Cc = K, 64
    ab = 2 * tok * H * 2
    return {
        # the two launches of the whole prefill: per-chunk solve (x's q|k channels
        # and a, b in; convolved q|k rows and records out), scan (q|k rows, x's
        # value channels, records in; o and the final state out)
        "prefill_prepare": {"bytes": 2 * qk + 2 * Hk * K * 4 * 2 + ab + rec,
                            "flops": chunks * (Hk * 2 * 10 * 16 * 16 * K * 2 + H * 64 ** 3 / 3)},
        "prefill_scan": {"bytes": qk + v + rec + o + state,
                         "flops": chunks * H * (3 * 64 * K * V * 2 + 2 * 0.5 * 64 * 64 * V * 2)},
        # the whole step, single-pass: x, a, b in; o and the final state out
        "prefill": {"bytes": tok * C * 2 + ab + o + state},
        "conv1d": {"bytes": 2 * tok * C * 2 + C * 4 * 2},
        "gate_prepare": {"bytes": 2 * tok * H * 2 + gb},
        "chunk_prepare": {"bytes": qk + gb + rec,
                          # lower-triangular K K^T and Q K^T tiles plus the 64x64 solve
                          "flops": chunks * (Hk * 2 * 10 * 16 * 16 * K * 2 + H * 64 ** 3 / 3)},
        "chunk_scan": {"bytes": qk + v + rec + o + state,
                       # K h, Q h, K^T U (dense) + T V', P U (lower-triangular), per chunk and head
                       "flops": chunks * H * (3 * 64 * K * V * 2 + 2 * 0.5 * 64 * 64 * V * 2)},
        # the whole chunked forward, single-pass: q, k, v, g, beta in; o, final state out;
        # flops per token and head 6 d^2 + 5 C d + 2/3 C^2 (triangular count)
        "chunk_fwd": {"bytes": qk + v + gb + o + state,
                      "flops": tok * H * (6 * d * d + 5 * Cc * d + (2 * Cc * Cc) / 3),
                      # dense count: the intra-chunk products as full C x C blocks
                      "flops_dense": tok * H * (6 * d * d + 10 * Cc * d + (2 * Cc * Cc) / 3)},
    }


def chunk_fwd_report(acc, tokens, ms):
    """tokens/s of the chunked forward and its fractions of the bf16 MFMA peak
    (triangular flop count) and of HBM (single-pass bytes)."""
    s = ms / 1e3
    return {"tokens_per_s": tokens / s, "us": s * 1e6,
            "mfma_frac": acc["chunk_fwd"]["flops"] / s / (BF16_PEAK_TFLOPS * 1e12),
            "mfma_frac_dense": acc["chunk_fwd"]["flops_dense"] / s / (BF16_PEAK_TFLOPS * 1e12),
            "hbm_frac": acc["chunk_fwd"]["bytes"] / s / (HBM_PEAK_GBS * 1e9),
            "algorithmic_flops": acc["chunk_fwd"]["flops"],
            "algorithmic_bytes": acc["chunk_fwd"]["bytes"]}


def decode_accounting(n, M, H, G, P, N):
    xl = M * H * P + M * G * N + G * N
    state = n * H * N * P * 4
    return 2 * state + n * xl * 2 + n * (M * H + H) * 2 + n * H * P * 2


def source_hash(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(op):
    """HBM bytes per launch (FETCH + WRITE, scaled by the copy-kernel factor)
    from profiles/traffic.json, or None when absent or stale."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get("kernels", {}).get(KERNELS[op][0])
    if not ent or ent.get("source_sha") != source_hash(KERNELS[op][1]):
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(w, batch):
    """The fp64 oracle chain (conv -> gates -> recurrence) on `batch` sequences
    (all heads, full length) of the prefill workload; batch = 4 is one whole step."""
    import numpy as np
    import torch

    import oracle
    import workloads as wl
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    d = wl.prefill_inputs(w, B=batch)
    tokens = batch * w.T
    f64 = lambda t: t.to(torch.float32).numpy().astype(np.float64)
    x, cw, a, b = f64(d["x"]), f64(d["w"]), f64(d["a"]), f64(d["b"])
    A_log, dt_bias = f64(d["A_log"]), f64(d["dt_bias"])
    t0 = time.perf_counter()
    y = oracle.conv1d_causal(x, cw, silu=True)
    nq = w.Hk * w.K
    q = y[:, :, :nq].reshape(batch, w.T, w.Hk, w.K)
    k = y[:, :, nq:2 * nq].reshape(batch, w.T, w.Hk, w.K)
    v = y[:, :, 2 * nq:].reshape(batch, w.T, w.H, w.V)
    g, beta = oracle.gate_prepare(a, b, A_log, dt_bias)
    oracle.gated_delta_rule(q, k, v, g, beta)
    dt = time.perf_counter() - t0
    used = min(threads, batch * w.H)   # the recurrence runs (sequence, head) units in parallel
    return {"value": tokens / dt, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{batch} x {w.T} tokens x {w.H} heads of the prefill workload (fp64 "
                      f"conv1d + gates + timestep recurrence), {dt:.2f} s on {used} threads"}


def _timed_steps(args, torch, stream, step, n_ev):
    """W untimed steps, then K timed steps with nothing else on the stream (the
    wall time per step, ms, between two synchronisations), then K more with
    n_ev HIP events each on `stream`, bracketing each kernel (its duration).
    The two passes are separate because an event recorded between two
    kernels leaves a gap of several microseconds between them."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    return evs, step_ms


class Flush:
    """Writes a 512 MB scratch buffer: evicts the 256 MB Infinity Cache (and the
    L2s) between timed iterations, outside the timed region."""
    def __init__(self, torch, dev):
        self.buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xff)


def iter_stats(fn, torch, stream, iters, flush=None):
    """Median, p10 and p90 (us) of `iters` single calls timed with HIP events on
    `stream`, each preceded (outside its events) by `flush` when given."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)

    def pct(q):
        return us[min(len(us) - 1, int(round(q * (len(us) - 1))))]
    return {"median_us": pct(0.5), "p10_us": pct(0.1), "p90_us": pct(0.9), "iters": iters}


def copy_peak(torch, dev, stream):
    """GB/s of a plain 1 GiB device-to-device copy (read + write bytes)."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = iter_stats(lambda: dst.copy_(src), torch, stream, 5)
    return 2 * (1 << 30) / (st["median_us"] / 1e6) / 1e9


def run_prefill(args, gdn, wl, torch, dev, stream):
    """The whole prefill through its three phase entry points (each one kernel),
    with events between them."""
    w = wl.WORKLOADS["prefill"]
    d = wl.prefill_inputs(w)
    x, cw = d["x"].to(dev), d["w"].to(dev)
    a, b = d["a"].to(dev), d["b"].to(dev)
    A_log, dt_bias = d["A_log"].to(dev), d["dt_bias"].to(dev)
    o = torch.empty((w.B, w.T, w.H, w.V), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((w.B, w.H, w.K, w.V), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.gdn_prefill_workspace_size(w.B, w.T, w.H, w.Hk, w.K, w.V, 0),
                     dtype=torch.uint8, device=dev)
    dims = dict(Hk=w.Hk, K=w.K, H=w.H, V=w.V)
    ops = ["prefill_prepare", "prefill_scan"]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        gdn.gdn_prefill_prepare(x, cw, a, b, A_log, dt_bias, ws, **dims)
        if evs:
            evs[1].record(stream)
        gdn.gdn_prefill_scan(x, cw, ws, o=o, final_state=fs, **dims)
        if evs:
            evs[2].record(stream)

    evs, step_ms = _timed_steps(args, torch, stream, step, 3)
    op_ms = {op: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
             for j, op in enumerate(ops)}
    # per-iteration statistics: back to back, and with the caches flushed
    # between iterations (outside the timed region)
    stats = {"back_to_back": iter_stats(step, torch, stream, args.steps)}
    if not args.no_flush:
        stats["flushed"] = iter_stats(step, torch, stream, args.steps, Flush(torch, dev))
    return w, op_ms, step_ms, stats


def run_chain(args, gdn, wl, torch, dev, stream):
    """The same computation as four calls: conv1d over all of q|k|v, gates,
    chunk_prepare, chunk_scan (the per-step entry points)."""
    w = wl.WORKLOADS["prefill"]
    d = wl.prefill_inputs(w)
    x, cw = d["x"].to(dev), d["w"].to(dev)
    a, b = d["a"].to(dev), d["b"].to(dev)
    A_log, dt_bias = d["A_log"].to(dev), d["dt_bias"].to(dev)
    y = torch.empty_like(x)
    g = torch.empty((w.B, w.T, w.H), dtype=torch.float32, device=dev)
    beta = torch.empty_like(g)
    o = torch.empty((w.B, w.T, w.H, w.V), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((w.B, w.H, w.K, w.V), dtype=torch.float32, device=dev)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(w.B, w.T, w.H, w.Hk, w.K, w.V, 0,
                                                      torch.bfloat16), dtype=torch.uint8, device=dev)
    q, k, v = gdn.split_qkv(y, w.Hk, w.K, w.H, w.V)
    ops = ["conv1d", "gate_prepare", "chunk_prepare", "chunk_scan"]

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        gdn.gdn_conv1d_causal(x, cw, y=y, silu=True)
        if evs:
            evs[1].record(stream)
        gdn.gdn_gate_prepare(a, b, A_log, dt_bias, g=g, beta=beta)
        if evs:
            evs[2].record(stream)
        gdn.gdn_chunk_prepare(q, k, g, beta, ws)
        if evs:
            evs[3].record(stream)
        gdn.gdn_chunk_scan(q, k, v, o, ws, final_state=fs)
        if evs:
            evs[4].record(stream)

    evs, step_ms = _timed_steps(args, torch, stream, step, 5)
    op_us = {op: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps * 1e3
             for j, op in enumerate(ops)}
    tokens = w.B * w.T

    # the chunked forward alone on the resident q, k, v, g, beta (the
    # headline metric's unit): per-iteration statistics, flushed and not
    def chunk():
        gdn.gdn_chunk_prepare(q, k, g, beta, ws)
        gdn.gdn_chunk_scan(q, k, v, o, ws, final_state=fs)
    chunk_stats = {"back_to_back": iter_stats(chunk, torch, stream, args.steps)}
    if not args.no_flush:
        chunk_stats["flushed"] = iter_stats(chunk, torch, stream, args.steps, Flush(torch, dev))
    return {"us": step_ms * 1e3, "tokens_per_s": tokens / (step_ms / 1e3), "ops_us": op_us,
            "chunk_fwd_iters": chunk_stats}


def run_decode(args, gdn, wl, torch, dev, stream):
    wd = wl.WORKLOADS["decode"]
    st = wl.decode_state_inputs(wd)
    state = st["state"].to(dev)
    A_log, dt_bias = st["A_log"].to(dev), st["dt_bias"].to(dev)
    xl, bl = wl.decode_row_sizes(wd.M, wd.H, wd.G, wd.V, wd.K)
    steps = args.decode_steps
    # per-step inputs pre-staged in HBM (same distributions as the parity tests,
    # drawn on the device with a seeded generator)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wd.seed)
    xs = torch.randn((steps, wd.n, xl), generator=gen, device=dev).to(torch.bfloat16)
    bas = torch.randn((steps, wd.n, bl), generator=gen, device=dev).to(torch.bfloat16)
    o = torch.empty((wd.n, wd.H, wd.V), dtype=torch.bfloat16, device=dev)
    for i in range(min(10, steps)):
        gdn.gdn_recurrent_decode(xs[i], bas[i], A_log, dt_bias, state, wd.M, wd.H, wd.G, wd.V,
                                 wd.K, o=o)
    state.copy_(st["state"].to(dev))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        gdn.gdn_recurrent_decode(xs[i], bas[i], A_log, dt_bias, state, wd.M, wd.H, wd.G, wd.V,
                                 wd.K, o=o)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per_s = ms / steps / 1e3
    nbytes = decode_accounting(wd.n, wd.M, wd.H, wd.G, wd.V, wd.K)
    return {"req_per_s": wd.n * steps / (ms / 1e3), "us_per_step": per_s * 1e6,
            "kernel": KERNELS["decode"][0],
            "roofline": {"bound": "hbm", "achieved": nbytes / per_s / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": nbytes / per_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("decode")},
            "algorithmic_bytes_per_step": nbytes,
            "workload": f"decode bf16 n={wd.n} M={wd.M} H={wd.H} G={wd.G} P=N={wd.K}, "
                        f"fp32 state in place, {steps} steps"}


def _time_launches(torch, stream, fn, reps):
    """Average µs of fn() over reps launches, HIP events on the launch stream."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _time_graph(torch, fn, reps):
    """Average µs per launch of fn() replayed from a captured HIP graph of reps
    launches (no per-launch host overhead: what a decode loop captured in a
    graph sees)."""
    fn()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    e0.record(cur)
    graph.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def _hbm(nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": us, "algorithmic_bytes": nbytes, "achieved_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}


def run_gdp_steps(gdn, wl, torch, dev, stream):
    """The Gated DeltaProduct steps around the core, each on its own: the
    decode short-conv update and the five-tensor decode preparation at the
    decode workload's shape (timed as graph replays: one decode token's launches
    are that small), and a GDP prefill (interleave + chunked forward)."""
    wd = wl.WORKLOADS["decode"]
    n, M, H, G, P, N = wd.n, wd.M, wd.H, wd.G, wd.V, wd.K
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wd.seed + 1)
    bf = torch.bfloat16
    x = torch.randn((n, xl), generator=gen, device=dev).to(bf)
    ba = torch.randn((n, bl), generator=gen, device=dev).to(bf)
    cw = (torch.randn((xl, 4), generator=gen, device=dev) * 0.5).to(bf)
    cst = torch.randn((n, 3, xl), generator=gen, device=dev).to(bf)
    slot = torch.randperm(n, generator=gen, device=dev).to(torch.int32)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen, device=dev))
    dt_bias = torch.randn(H, generator=gen, device=dev) * 0.1
    y = torch.empty_like(x)
    out = {}
    us = _time_graph(torch, lambda: gdn.gdn_conv1d_update(x, cst, slot, cw, y=y), 100)
    out["conv1d_update"] = _hbm(2 * n * xl * 2 + 2 * n * 3 * xl * 2 + xl * 4 * 2, us)
    out["conv1d_update"]["workload"] = f"n={n} requests, C={xl} bf16, W=4, one slot each"
    dq = torch.empty((n, M, H, N), dtype=bf, device=dev)
    dout = (dq, torch.empty_like(dq), torch.empty((n, M, H, P), dtype=bf, device=dev),
            torch.empty((n, M, H), device=dev), torch.empty((n, M, H), device=dev))
    us = _time_graph(torch, lambda: gdn.gdn_decode_prepare(x, ba, A_log, dt_bias, M, H, G, P, N,
                                                           out=dout), 100)
    out["decode_prepare"] = _hbm(n * xl * 2 + n * bl * 2 + n * M * H * (2 * N + P) * 2
                                 + 2 * n * M * H * 4, us)
    out["decode_prepare"]["workload"] = f"n={n} M={M} H={H} G={G} P=N={N} bf16"
    # GDP prefill at the decode layer's shape: B sequences of T tokens
    B, T = 2, 2048
    xp = torch.randn((B, T, xl), generator=gen, device=dev).to(bf)
    bp = torch.randn((B, T, bl), generator=gen, device=dev).to(bf)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, M * T, H, G, N, P, 0, bf),
                     dtype=torch.uint8, device=dev)
    q, k, v, g, beta, _ = gdn.gdn_gdp_prefill_prepare(xp, bp, A_log, dt_bias, M, H, G, P, N)
    us_prep = _time_launches(torch, stream, lambda: gdn.gdn_gdp_prefill_prepare(
        xp, bp, A_log, dt_bias, M, H, G, P, N, out=(q, k, v, g, beta)), 20)
    o = torch.empty((B, M * T, H, P), dtype=bf, device=dev)
    us_fwd = _time_launches(torch, stream, lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, workspace=ws, o=o), 20)
    prep_bytes = B * T * (xl + bl) * 2 + B * M * T * (2 * G * N + H * P) * 2 + 2 * B * M * T * H * 4
    out["gdp_prefill"] = {"tokens_per_s": B * T / ((us_prep + us_fwd) * 1e-6), "us": us_prep + us_fwd,
                          "interleave": _hbm(prep_bytes, us_prep), "chunk_fwd_us": us_fwd,
                          "workload": f"B={B} T={T} M={M} H={H} G={G} P=N={N} bf16 "
                                      f"(chunked forward over {M * T} positions per sequence)"}
    return out


def _kernel_stem(name):
    """Readable name of a kernel symbol: our mangled template kernels become
    name<args> (bf16 template arguments are beyond the image's c++filt)."""
    import re
    m = re.match(r"_ZN3gdn\d+(\w+?)I(.*?)EEv", name)
    if m:
        parts = []
        for tok in re.finditer(r"DF16b|Li(\d+)E|Lb([01])E|f", m.group(2)):
            s = tok.group(0)
            parts.append("bf16" if s == "DF16b" else "float" if s == "f" else
                         tok.group(1) if tok.group(1) else ("true" if tok.group(2) == "1" else "false"))
        return f"{m.group(1)}<{', '.join(parts)}>"
    m = re.match(r"_ZN3gdn\d+(\w+?)I", name)
    if m:
        return m.group(1)
    s = name.split("(")[0]
    return (s[5:] if s.startswith("void ") else s)[:60]


def _phases(rows, id_key, name_key):
    """The benchmark runs its parts in a fixed order: the prefill step, then the
    decode step, then the Gated DeltaProduct steps. The decode kernel's
    dispatches mark the boundaries, so a kernel used by two parts (the chunked
    forward) is summarised per part instead of as a blended average."""
    ids = [int(r[id_key]) for r in rows if KERNELS["decode"][0] in r[name_key]]
    lo, hi = (min(ids), max(ids)) if ids else (None, None)

    def phase(r):
        d = int(r[id_key])
        if lo is None or d < lo:
            return "prefill"
        return "decode" if d <= hi else "gdp steps"
    return phase


def summarize_stats(csv_path, out_md, command, bench_log=None):
    """Kernel time table from rocprofv3's kernel trace (one row per dispatch),
    one line per (benchmark part, kernel, grid, workgroup)."""
    import collections
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    phase = _phases(rows, "Dispatch_Id", "Kernel_Name")
    groups = collections.OrderedDict()
    for r in rows:
        key = (phase(r), r["Kernel_Name"],
               int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    order = {"prefill": 0, "decode": 1, "gdp steps": 2}
    items = sorted(groups.items(), key=lambda kv: (order[kv[0][0]], -sum(kv[1])))
    lines = ["# Kernel time summary (rocprofv3 --kernel-trace --stats)", "",
             f"Command: `{command}`", "",
             "One line per part of the benchmark (prefill step, decode step, Gated DeltaProduct",
             "steps), kernel and launch shape (grid = work-items), from the kernel trace.", "",
             "| part | kernel | grid | workgroup | calls | average (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (ph, name, grid, wg), d in items:
        lines.append(f"| {ph} | `{_kernel_stem(name)}` | {grid} | {wg} | {len(d)} | "
                     f"{sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                     f"{100 * sum(d) / total:.1f}% |")
    if bench_log:
        js = [ln for ln in open(bench_log) if ln.startswith("{")]
        b = json.loads(js[-1])
        lines += ["", "The same run's bench line (HIP events on the launch stream, averaged over",
                  "the timed steps), for comparison with the trace averages above:", ""]
        for op, us in b.get("ops_us", {}).items():
            lines.append(f"- {op} (`{KERNELS[op][0]}`): {us:.2f} us")
        if "decode" in b:
            lines.append(f"- decode step (`{b['decode']['kernel']}`): {b['decode']['us_per_step']:.2f} us")
    lines += ["", "Full symbols:", ""]
    seen = set()
    for (_, name, _, _), _ in items:
        if name not in seen:
            seen.add(name)
            lines.append(f"- `{name[:200]}`")
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_traffic(fetch_csv, write_csv, command):
    """Per-kernel HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that makes the plain 1 GiB device copy
    (the runtime's buffer-copy kernel, --copy-probe) read and write 1 GiB."""
    import collections
    import csv

    def per_dispatch(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        phase = _phases(rows, "Dispatch_Id", "Kernel_Name")
        acc = collections.defaultdict(float)
        names, phases = {}, {}
        for r in rows:
            d = int(r["Dispatch_Id"])
            acc[d] += float(r["Counter_Value"]) * 1024.0   # KiB -> bytes
            names[d] = r["Kernel_Name"]
            phases[d] = phase(r)
        return acc, names, phases

    fetch, fnames, fphase = per_dispatch(fetch_csv, "FETCH_SIZE")
    write, wnames, wphase = per_dispatch(write_csv, "WRITE_SIZE")
    gib = float(1 << 30)
    # the probe copies are the buffer-copy dispatches that move 1 GiB: the last three
    # of that kernel in each run (earlier ones are uploads and the state reset)
    def probe(table, names):
        ids = sorted(d for d, n in names.items() if "copybuffer" in n.lower())[-3:]
        vals = [table[d] for d in ids]
        return sum(vals) / len(vals) if vals else None
    pf, pw = probe(fetch, fnames), probe(write, wnames)
    ff = gib / pf if pf else None
    fw = gib / pw if pw else None
    res = {"command": command, "copy_kernel_bytes": gib, "copy_fetch_raw": pf, "copy_write_raw": pw,
           "fetch_factor": ff, "write_factor": fw, "kernels": {}}
    for op, (stem, src) in KERNELS.items():
        ids = sorted(d for d in fetch if stem in fnames[d])
        if not ids or ff is None or fw is None:
            continue
        # the part of the benchmark where the kernel first runs is its own
        # workload; later launches (the Gated DeltaProduct steps) are kept apart
        part = fphase[ids[0]]
        fv = [fetch[d] for d in ids if fphase[d] == part]
        wv = [v for d, v in write.items() if stem in wnames[d] and wphase[d] == part]
        fb = sum(fv) / len(fv) * ff
        wb = (sum(wv) / len(wv) * fw) if wv else 0.0
        res["kernels"][stem] = {"part": part, "fetch_bytes": fb, "write_bytes": wb,
                                "bytes_per_launch": fb + wb, "launches": len(fv),
                                "source_sha": source_hash(src)}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "traffic.json"), "w") as f:
        json.dump(res, f, indent=1)
    return res


def summarize_mfma(csv_path, out_md, command, cus=256, simds=4, xcds=8):
    """Per kernel and bench part: MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES /
    (active cycles x CUs x SIMDs), the active cycles being GRBM_GUI_ACTIVE per
    XCD (the counter is summed over the XCDs); and MFMA instructions per launch."""
    import collections
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    phase = _phases(rows, "Dispatch_Id", "Kernel_Name")
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = (phase(r), r["Kernel_Name"])
    groups = collections.OrderedDict()
    for d in sorted(per):
        groups.setdefault(names[d], []).append(per[d])
    lines = ["# MFMA busy (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             f"busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x {cus} CUs x {simds} SIMDs),",
             "averaged over the launches of each kernel in each part of the bench.", "",
             "| part | kernel | launches | MFMA busy | MFMA instructions / launch |",
             "|---|---|---|---|---|"]
    for (ph, name), cs in groups.items():
        act = sum(c.get("GRBM_GUI_ACTIVE", 0) for c in cs) / xcds
        busy = sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) for c in cs)
        insts = sum(c.get("SQ_INSTS_MFMA", 0) for c in cs) / len(cs)
        if insts == 0:
            continue
        frac = busy / (act * cus * simds) if act else 0.0
        lines.append(f"| {ph} | `{_kernel_stem(name)}` | {len(cs)} | {frac:.3f} | {insts:.4g} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def main():
    args = parse()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma[0], args.summarize_mfma[1], args.command)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.command,
                        args.bench_log)
        return
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1],
                                           args.command), indent=1))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the kernels are "
                                   "single-GPU and no multi-GPU path exists", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import linear_attention_ssm_amd as gdn
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    w = wl.WORKLOADS["prefill"]
    out = {"metric": "GDN chunk-fwd tokens/s (H=16,d=128,T=4096); decode req/s; % of roofline",
           "value_covers": "the whole prefill step: conv1d + SiLU, gates and the chunked forward",
           "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"prefill bf16 B={w.B} H={w.H} Hk={w.Hk} T={w.T} K=V={w.K} "
                                  "chunk=64, conv1d W=4 + SiLU over C=6144, fp32 state",
                      "global_batch": w.B, "seq_len": w.T, "parallelism": "single-gpu"}}

    if args.only != "decode":
        w, op_ms, step_ms, step_stats = run_prefill(args, gdn, wl, torch, dev, stream)
        acc = prefill_accounting(w.B, w.T, w.H, w.Hk, w.K, w.V)
        tokens = w.B * w.T
        out["value"] = tokens / (step_ms / 1e3)
        out["ms_per_step"] = step_ms
        out["ops_us"] = {op: ms * 1e3 for op, ms in op_ms.items()}
        dom = max(op_ms, key=op_ms.get)
        sec = op_ms[dom] / 1e3
        ach = acc[dom]["bytes"] / sec / 1e9
        out["roofline"] = {"kernel": KERNELS[dom][0], "bound": "hbm", "achieved": ach,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                           "traffic": load_traffic(dom),
                           "algorithmic_bytes": acc[dom]["bytes"]}
        if "flops" in acc[dom]:
            out["roofline"]["mfma_frac"] = acc[dom]["flops"] / sec / (BF16_PEAK_TFLOPS * 1e12)
        step_s = step_ms / 1e3
        out["step"] = {"algorithmic_bytes": acc["prefill"]["bytes"],
                       "hbm_frac": acc["prefill"]["bytes"] / step_s / (HBM_PEAK_GBS * 1e9),
                       "iters": step_stats}
        # the chunked forward: the prepare and scan phases (which here also form
        # the gates and convolve the value rows)
        out["chunk_fwd"] = chunk_fwd_report(acc, tokens, op_ms["prefill_prepare"] + op_ms["prefill_scan"])
        out["kernels"] = {op: {"us": op_ms[op] * 1e3,
                               "achieved_GBs": acc[op]["bytes"] / (op_ms[op] / 1e3) / 1e9,
                               "hbm_frac": acc[op]["bytes"] / (op_ms[op] / 1e3) / 1e9 / HBM_PEAK_GBS}
                          for op in op_ms}
    if not args.no_chain and args.only != "decode":
        out["chain"] = run_chain(args, gdn, wl, torch, dev, stream)
        ch = out["chain"]["ops_us"]
        out["chain"]["chunk_fwd"] = chunk_fwd_report(acc, tokens, (ch["chunk_prepare"] + ch["chunk_scan"]) / 1e3)
        for kind, st in out["chain"].pop("chunk_fwd_iters").items():
            out["chain"]["chunk_fwd"][kind] = dict(
                st, tokens_per_s_median=tokens / (st["median_us"] / 1e6),
                mfma_frac_median=acc["chunk_fwd"]["flops"] / (st["median_us"] / 1e6) / (BF16_PEAK_TFLOPS * 1e12))
    if args.only != "prefill" and not args.no_decode:
        out["decode"] = run_decode(args, gdn, wl, torch, dev, stream)
        out["gdp_steps"] = run_gdp_steps(gdn, wl, torch, dev, stream)
    # the copy-kernel peak, the practical HBM ceiling the fractions are also read
    # against (read + write bytes of a plain device copy)
    cp = copy_peak(torch, dev, stream)
    out["copy_peak_GBs"] = cp
    for kk in out.get("kernels", {}).values():
        kk["copy_frac"] = kk["achieved_GBs"] / cp
    if "roofline" in out:
        out["roofline"]["copy_frac"] = out["roofline"]["achieved"] / cp
    if "decode" in out:
        out["decode"]["roofline"]["copy_frac"] = out["decode"]["roofline"]["achieved"] / cp
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu and args.only != "decode":
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
