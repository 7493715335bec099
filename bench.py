"""Benchmark of the gated-delta-rule forward on one MI355X.

A step is one pass of the prefill hot path over one batch of the bf16 prefill
workload (B=4, H=16, T=4096, K=V=128): causal conv1d + SiLU over the q|k|v
channels (C = 6144), gate preparation, and the chunked forward (per-chunk WY
solve + sequential state scan + outputs + final state). Inputs are resident in
HBM before timing starts. `value` is tokens/s of the whole step (16,384 tokens
per step); the chunked forward alone and the one-token Gated DeltaProduct
decode (n=256 requests, M=2, H=32, G=16, P=N=128, 1000 steps, state in place)
are reported beside it.

Per-op durations come from HIP events recorded on the stream the kernels are
launched on (torch's current stream, which the binding passes to the library).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]
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
KERNEL_SOURCES = {
    "conv1d_causal_kernel": "linear_attention_ssm_amd/csrc/conv1d.hip",
    "chunk_scan_kernel": "linear_attention_ssm_amd/csrc/chunk.hip",
    "chunk_prep_kernel": "linear_attention_ssm_amd/csrc/chunk.hip",
    "gdp_decode_kernel": "linear_attention_ssm_amd/csrc/decode.hip",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--decode-steps", type=int, default=1000)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-batch", type=int, default=4,
                   help="sequences of the prefill workload the oracle baseline runs (4 = all)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration runs)")
    p.add_argument("--only", choices=["prefill", "decode"], default=None)
    return p.parse_args()


# algorithmic traffic / work of the prefill workload (one step)
def prefill_accounting(B, T, H, Hk, K, V):
    C = 2 * Hk * K + H * V
    tok = B * T
    conv_bytes = 2 * tok * C * 2 + C * 4 * 2                    # x in + y out (bf16) + w
    gate_bytes = 2 * tok * H * 2 + 2 * tok * H * 4              # a, b in (bf16); g, beta out (fp32)
    chunk_bytes = (2 * tok * Hk * K * 2 + tok * H * V * 2       # q, k, v in (bf16)
                   + 2 * tok * H * 4                            # g, beta in (fp32)
                   + tok * H * V * 2                            # o out (bf16)
                   + B * H * K * V * 4)                         # final state out (fp32)
    d, Cc = K, 64
    flops_tri = tok * H * (6 * d * d + 5 * Cc * d + (2 * Cc * Cc) / 3)
    return dict(conv=conv_bytes, gate=gate_bytes, chunk=chunk_bytes, chunk_flops=flops_tri)


def decode_accounting(n, M, H, G, P, N):
    xl = M * H * P + M * G * N + G * N
    state = n * H * N * P * 4
    return 2 * state + n * xl * 2 + n * (M * H + H) * 2 + n * H * P * 2


def source_hash(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 --pmc summaries, or None
    when absent or taken on a different version of the kernel source."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU runs "
                                   "are not part of this build", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import linear_attention_ssm_amd as gdn
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    result = {}

    w = wl.WORKLOADS["prefill"]
    acc = prefill_accounting(w.B, w.T, w.H, w.Hk, w.K, w.V)
    tokens = w.B * w.T

    if args.only != "decode":
        d = wl.prefill_inputs(w)
        x, cw = d["x"].to(dev), d["w"].to(dev)
        a, b = d["a"].to(dev), d["b"].to(dev)
        A_log, dt_bias = d["A_log"].to(dev), d["dt_bias"].to(dev)
        bufs = {
            "y": torch.empty_like(x),
            "g": torch.empty((w.B, w.T, w.H), dtype=torch.float32, device=dev),
            "beta": torch.empty((w.B, w.T, w.H), dtype=torch.float32, device=dev),
            "o": torch.empty((w.B, w.T, w.H, w.V), dtype=torch.bfloat16, device=dev),
            "final_state": torch.empty((w.B, w.H, w.K, w.V), dtype=torch.float32, device=dev),
            "workspace": torch.empty(gdn.gdn_chunk_fwd_workspace_size(
                w.B, w.T, w.H, w.Hk, w.K, w.V, 0, torch.bfloat16), dtype=torch.uint8, device=dev),
        }

        def step(evs=None):
            if evs:
                evs[0].record(stream)
            y = gdn.gdn_conv1d_causal(x, cw, y=bufs["y"], silu=True)
            if evs:
                evs[1].record(stream)
            g, beta = gdn.gdn_gate_prepare(a, b, A_log, dt_bias, g=bufs["g"], beta=bufs["beta"])
            if evs:
                evs[2].record(stream)
            q, k, v = gdn.split_qkv(y, w.Hk, w.K, w.H, w.V)
            gdn.gdn_chunk_fwd(q, k, v, g, beta, workspace=bufs["workspace"], o=bufs["o"],
                              final_state=bufs["final_state"])
            if evs:
                evs[3].record(stream)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        # per-op events inside the timed region
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        conv_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
        gate_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
        chunk_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
        step_ms = wall * 1e3 / args.steps
        result["prefill"] = dict(step_ms=step_ms, conv_ms=conv_ms, gate_ms=gate_ms,
                                 chunk_ms=chunk_ms, tokens=tokens)

    if args.only != "prefill" and not args.no_decode:
        wd = wl.WORKLOADS["decode"]
        st = wl.decode_state_inputs(wd)
        state = st["state"].to(dev)
        A_log_d, dt_bias_d = st["A_log"].to(dev), st["dt_bias"].to(dev)
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
            gdn.gdn_recurrent_decode(xs[i], bas[i], A_log_d, dt_bias_d, state, wd.M, wd.H, wd.G,
                                     wd.V, wd.K, o=o)
        state.copy_(st["state"].to(dev))
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            gdn.gdn_recurrent_decode(xs[i], bas[i], A_log_d, dt_bias_d, state, wd.M, wd.H, wd.G,
                                     wd.V, wd.K, o=o)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1)
        per = dec_ms / steps
        dbytes = decode_accounting(wd.n, wd.M, wd.H, wd.G, wd.V, wd.K)
        result["decode"] = dict(ms_total=dec_ms, us_per_step=per * 1e3,
                                req_per_s=wd.n * steps / (dec_ms / 1e3),
                                achieved_GBs=dbytes / (per / 1e3) / 1e9,
                                bytes_per_step=dbytes, steps=steps, n=wd.n)
        del xs, bas

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    out = {"metric": "GDN prefill tokens/s (conv1d + gates + chunk_fwd; H=16, d=128, T=4096)",
           "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "prefill bf16 B=4 H=16 Hk=16 T=4096 K=V=128 chunk=64, "
                                  "conv1d W=4 + SiLU over C=6144, fp32 state",
                      "global_batch": w.B, "seq_len": w.T, "parallelism": "single-gpu"}}
    if "prefill" in result:
        p = result["prefill"]
        out["value"] = tokens / (p["step_ms"] / 1e3)
        out["ms_per_step"] = p["step_ms"]
        chunk_s = p["chunk_ms"] / 1e3
        conv_s = p["conv_ms"] / 1e3
        out["ops_ms"] = {"conv1d": p["conv_ms"], "gate_prepare": p["gate_ms"],
                         "chunk_fwd": p["chunk_ms"]}
        out["chunk_fwd_tokens_per_s"] = tokens / chunk_s
        out["chunk_fwd_roofline"] = {
            "mfma_frac": acc["chunk_flops"] / chunk_s / (BF16_PEAK_TFLOPS * 1e12),
            "hbm_frac": acc["chunk"] / chunk_s / (HBM_PEAK_GBS * 1e9),
            "algorithmic_flops": acc["chunk_flops"], "algorithmic_bytes": acc["chunk"]}
        # the dominant kernel of the step: report its roofline
        ops = {"conv1d": (conv_s, acc["conv"], "conv1d_causal_kernel")}
        name, (sec, nbytes, kname) = max(ops.items(), key=lambda kv: kv[1][0])
        if p["chunk_ms"] > p["conv_ms"]:
            out["roofline"] = {"kernel": "gdn_chunk_fwd (chunk_prep + chunk_scan)",
                               "bound": "hbm", "achieved": acc["chunk"] / chunk_s / 1e9,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": acc["chunk"] / chunk_s / 1e9 / HBM_PEAK_GBS,
                               "traffic": None}
        else:
            tr = load_traffic(kname)
            out["roofline"] = {"kernel": kname, "bound": "hbm",
                               "achieved": nbytes / sec / 1e9, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": nbytes / sec / 1e9 / HBM_PEAK_GBS,
                               "traffic": tr}
    if "decode" in result:
        dd = result["decode"]
        out["decode"] = {"req_per_s": dd["req_per_s"], "us_per_step": dd["us_per_step"],
                         "achieved_GBs": dd["achieved_GBs"],
                         "hbm_frac": dd["achieved_GBs"] / HBM_PEAK_GBS,
                         "workload": "decode bf16 n=256 M=2 H=32 G=16 P=N=128, fp32 state "
                                     f"in place, {dd['steps']} steps",
                         "traffic": load_traffic("gdp_decode_kernel")}
    if not args.no_cpu and args.only != "decode":
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
