"""Benchmark of the gated-delta-rule forward on one MI355X.

A step is one pass of the prefill hot path over one batch of the bf16 prefill
workload (B=4, H=16, T=4096, K=V=128): causal conv1d + SiLU over the q|k|v
channels (C = 6144), gate preparation, and the chunked forward (per-chunk WY
solve, then the sequential state scan with the outputs and the final state),
run as the library's whole-prefill entry in its two phases: the per-chunk
solve (convolving the q and k rows and forming the gates itself) and the scan
(convolving the value rows as it reads them). Inputs are resident in HBM
before timing starts. `value` is tokens/s of the whole step (16,384 tokens
per step) over K back-to-back steps; `value_flushed` is the same step timed
per iteration with the caches flushed between iterations (a 512 MB write
outside the timed region), the median of K.

The other workloads are measured beside it, each in its own block of
`configs`: the tiny fp32 workload (c1), the prefill workload's four per-step
calls and the chunked forward alone on resident q, k, v, g, beta (c2), the
GQA long prefill (c3, one sequence of 65,536 tokens, 32 value heads over 16
q/k heads, initial state), the packed varlen prefill (c4, 64 sequences of
1..2048 tokens) and the Gated DeltaProduct decode (c5, n=256, M=2, H=32,
G=16, P=N=128, 1000 steps, fp32 state in place). c3 and c4 draw their inputs
on the GPU with a seeded generator; every other input is the seeded CPU draw
of workloads.py.

Per-kernel durations come from HIP events recorded between the launches on
the stream the kernels run on (torch's current stream, which the binding
passes to the library). Each kernel is charged with its share of the
method's single-pass bytes (each tensor of the step's inputs and outputs that
the kernel reads or writes, counted once); workspace traffic (records,
convolved rows) is not in that share and shows up in `traffic` (rocprofv3
FETCH_SIZE + WRITE_SIZE per launch, from profiles/traffic.json, null when
absent or when the kernel's source has changed since) and in
`traffic_ratio` = traffic / share.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only c1,c2,c3,c4,c5] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix / vector, TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = "linear_attention_ssm_amd/csrc/"
PARTS = ["c2", "c1", "c3", "c4", "c5"]
PART_WORKLOAD = {"c1": "tiny", "c2": "prefill", "c3": "gqa", "c4": "varlen", "c5": "decode"}

# bench op -> (kernel name as _kernel_stem() prints it, source file), per part;
# a launch shape that differs between parts selects a different instance
_PREP = "chunk_prep_kernel<bf16, 128, true, true>"
_CPREP = "chunk_prep_kernel<bf16, 128, false, false>"
_CHUNK = CSRC + "chunk.hip"
KERNELS = {
    "c1": {"conv1d": ("conv1d_causal_kernel<float, 16, 256>", CSRC + "conv1d.hip"),
           "gate_prepare": ("gate_prepare_kernel<float>", CSRC + "gate.hip"),
           "chunk_prepare": ("chunk_prep_kernel<float, 64, false, false>", _CHUNK),
           "chunk_scan": ("chunk_scan_kernel<float, 64, 1, 2>", _CHUNK)},
    "c2": {"prefill_prepare": (_PREP, _CHUNK),
           "prefill_scan": ("chunk_scan_roles_kernel<128, 2, 3, true>", _CHUNK),
           "conv1d": ("conv1d_causal_kernel<bf16, 16, 256>", CSRC + "conv1d.hip"),
           "gate_prepare": ("gate_prepare4_kernel<bf16>", CSRC + "gate.hip"),
           "chunk_prepare": (_CPREP, _CHUNK),
           "chunk_scan": ("chunk_scan_roles_kernel<128, 2, 3, false>", _CHUNK)},
    "c3": {"prefill_prepare": (_PREP, _CHUNK),
           "prefill_scan": ("chunk_scan_roles_kernel<128, 1, 3, true>", _CHUNK),
           "chunk_prepare": (_CPREP, _CHUNK),
           "chunk_scan": ("chunk_scan_roles_kernel<128, 1, 3, false>", _CHUNK)},
    "c4": {"prefill_prepare": (_PREP, _CHUNK),
           "prefill_scan": ("chunk_scan_wide_kernel<128, 8, 2, false, true>", _CHUNK),
           "chunk_prepare": (_CPREP, _CHUNK),
           "chunk_scan": ("chunk_scan_wide_kernel<128, 8, 2, true, false>", _CHUNK)},
    "c5": {"decode": ("gdp_decode_kernel<bf16, 128, 128>", CSRC + "decode.hip"),
           "conv1d_update": ("conv1d_update_kernel<bf16>", CSRC + "gdp.hip"),
           "decode_prepare": ("gdp_decode_prepare_kernel<bf16>", CSRC + "gdp.hip")},
}


# the bf16 scan instances when the workgroup form is forced (--scan-form)
_ROLES = {"prefill_scan": ("chunk_scan_roles_kernel<128, 2, 3, true>", _CHUNK),
          "chunk_scan": ("chunk_scan_roles_kernel<128, 2, 3, false>", _CHUNK)}
_WIDE = {"prefill_scan": ("chunk_scan_wide_kernel<128, 8, 2, false, true>", _CHUNK),
         "chunk_scan": ("chunk_scan_wide_kernel<128, 8, 2, true, false>", _CHUNK)}
SCAN_FORM = 0


def kernel_of(part, op):
    """(kernel stem, source) that op runs in part under the scan form in force."""
    if op in _ROLES and SCAN_FORM == 1 and part == "c4":
        return _ROLES[op]     # (c2 and c3 run the column-group form by default)
    if op in _ROLES and SCAN_FORM == 2 and part in ("c2", "c3"):
        return _WIDE[op]      # (c4 runs the whole-unit form by default)
    return KERNELS.get(part, {}).get(op)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # (the GPU needs some tens of milliseconds of work to reach its sustained
    # clock: 10 warm-up steps time 10% slow, 200 (about 35 ms) do not)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--decode-steps", type=int, default=1000)
    p.add_argument("--only", default=",".join(PARTS),
                   help="comma-separated parts to run (c1 tiny fp32, c2 prefill, c3 GQA long "
                        "prefill, c4 varlen, c5 decode); the headline needs c2")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--cpu-batch", type=int, default=4,
                   help="sequences of the prefill workload the oracle baseline runs (4 = all)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration runs)")
    p.add_argument("--no-flush", action="store_true",
                   help="skip the per-iteration timings with the caches flushed between "
                        "iterations (profiling runs: every traced launch then runs warm, as in "
                        "the timed steps)")
    p.add_argument("--scan-form", type=int, default=0,
                   help="GDN_TUNE_SCAN_FORM for the run (0 automatic, 1 column groups, 2 whole "
                        "units): before/after comparisons of the bf16 scan schedules")
    p.add_argument("--summarize-stats", nargs=2, metavar=("KERNEL_TRACE_CSV", "OUT_MD"),
                   help="turn a rocprofv3 --kernel-trace csv into a profiles/ summary")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="merge rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of one part (made "
                        "with --copy-probe) into profiles/traffic.json")
    p.add_argument("--summarize-counters", nargs=2, metavar=("COUNTER_CSV", "OUT_MD"),
                   help="per-kernel table of a --pmc run's counters")
    p.add_argument("--part", default=None, help="with --summarize-*: the part the run covered")
    p.add_argument("--command", default="", help="the command that produced the CSVs")
    p.add_argument("--bench-log", default=None,
                   help="with --summarize-stats: the profiled run's output, whose bench line "
                        "gives the same run's kernel times measured with HIP events")
    return p.parse_args()


# ------------------------------------------------------------------ accounting

def accounting(tok, n_chunks, N, H, Hk, K, V, es=2, s0=False):
    """Algorithmic HBM bytes of the method's tensors (each read or written
    once) and MFMA flops, for a prefill of `tok` tokens in `n_chunks` chunks
    per head and N sequences; es = bytes per activation element; s0: an
    initial state is read."""
    C = 2 * Hk * K + H * V
    xqk = tok * 2 * Hk * K * es          # q|k channels (before or after the conv)
    xv = tok * H * V * es                # value channels
    o = tok * H * V * es
    ab = 2 * tok * H * es                # gate inputs a, b
    gb = 2 * tok * H * 4                 # g, beta (fp32)
    state = N * H * K * V * 4 * (2 if s0 else 1)   # final state written (+ initial read)
    taps = C * 4 * es
    d, Cc = K, 64
    flops = tok * H * (6 * d * d + 5 * Cc * d + (2 * Cc * Cc) / 3)
    flops_dense = tok * H * (6 * d * d + 10 * Cc * d + (2 * Cc * Cc) / 3)
    return {
        # whole prefill (x, a, b in; o and the final state out), split between
        # its two launches by the tensors each touches
        "prefill": {"bytes": xqk + xv + ab + o + state + taps},
        "prefill_prepare": {"bytes": xqk + ab + 2 * Hk * K * 4 * es},
        "prefill_scan": {"bytes": xv + o + state + H * V * 4 * es},
        # per-step calls
        "conv1d": {"bytes": 2 * tok * C * es + taps},
        "gate_prepare": {"bytes": ab + gb},
        "chunk_prepare": {"bytes": xqk + gb},
        "chunk_scan": {"bytes": xqk + xv + o + state},
        # the chunked forward alone (q, k, v, g, beta in; o, final state out);
        # flops per token and head 6 d^2 + 5 C d + 2/3 C^2 (intra-chunk products
        # as lower triangles), dense count beside it
        "chunk_fwd": {"bytes": xqk + xv + gb + o + state, "flops": flops,
                      "flops_dense": flops_dense},
        "n_chunks": n_chunks,
    }


def decode_accounting(n, M, H, G, P, N):
    xl = M * H * P + M * G * N + G * N
    state = n * H * N * P * 4
    return 2 * state + n * xl * 2 + n * (M * H + H) * 2 + n * H * P * 2


def source_hash(path):
    """Hash of a kernel source with its comments and spacing removed: an edit
    to the comments alone leaves the kernels, and their counters, as they were."""
    with open(os.path.join(ROOT, path), encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def load_traffic(part, op):
    """HBM bytes per launch (FETCH + WRITE, scaled by the copy-kernel factor)
    of op's kernel in `part`, from profiles/traffic.json; None when absent or
    stale (the kernel's source has changed since the counters were taken)."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path) or kernel_of(part, op) is None:
        return None
    with open(path) as f:
        data = json.load(f)
    stem, src = kernel_of(part, op)
    ent = data.get("parts", {}).get(part, {}).get("kernels", {}).get(stem)
    if not ent or ent.get("source_sha") != source_hash(src):
        return None
    return ent.get("bytes_per_launch")


def kernel_report(part, op, us, share, us_repeated=None):
    """One kernel's duration (in the passes; back to back alone beside it), its
    share of the single-pass bytes and the HBM rate that share implies, beside
    the measured traffic."""
    gbs = share / (us * 1e-6) / 1e9
    tr = load_traffic(part, op)
    return {"kernel": (kernel_of(part, op) or (None,))[0], "us": us,
            "us_repeated": us_repeated, "share_bytes": share,
            "achieved_GBs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "traffic": tr,
            "traffic_ratio": None if tr is None else tr / share}


def chunk_fwd_report(acc, tokens, us, peak_tflops=BF16_PEAK_TFLOPS):
    """tokens/s of the chunked forward and its fractions of the MFMA peak
    (triangular flop count; dense beside it) and of HBM (single-pass bytes)."""
    s = us * 1e-6
    cf = acc["chunk_fwd"]
    return {"tokens_per_s": tokens / s, "us": us,
            "mfma_frac": cf["flops"] / s / (peak_tflops * 1e12),
            "mfma_frac_dense": cf["flops_dense"] / s / (peak_tflops * 1e12),
            "hbm_frac": cf["bytes"] / s / (HBM_PEAK_GBS * 1e9),
            "algorithmic_flops": cf["flops"], "algorithmic_bytes": cf["bytes"]}


# --------------------------------------------------------------------- timing

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
    """Median, p10 and p90 (us) of `iters` single calls timed with HIP events
    (TimingEvent) on `stream`, each preceded (outside its events) by `flush`
    when given."""
    evs = [(TimingEvent(), TimingEvent()) for _ in range(iters)]
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


class TimingEvent:
    """A HIP event created with hipEventDisableSystemFence, for timing only:
    recording it does not write back and invalidate the caches (a default
    event's system-scope release does, which slows the kernel after it by
    some microseconds and changes what it finds in the caches). Made through
    the HIP runtime torch has loaded (found in the process's mappings)."""
    _hip = None

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
            TimingEvent._hip = ctypes.CDLL(path)
        self._c = ctypes
        self.h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.h), ctypes.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = TimingEvent._hip.hipEventRecord(self.h, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        ms = self._c.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(self._c.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if TimingEvent._hip is not None and self.h:
            TimingEvent._hip.hipEventDestroy(self.h)


def timed_ops(torch, stream, calls, steps, warmup):
    """calls: list of (op, fn). `warmup` untimed passes, then `steps` timed
    passes with nothing else on the stream (wall time per pass, us, between
    two synchronisations). Each op's launch duration is then taken inside
    `steps` more passes, HIP events (TimingEvent) recorded right before and
    after that op only (one event pair per pass, so the op runs where it runs in the timed
    passes, on the caches the ops before it leave), the passes queued behind
    a spin kernel so the host's call overhead leaves no idle gaps; the average
    over the passes. Also returned: the average of `steps` back-to-back
    launches of the op alone (the same spin-and-queue timing), for reference."""
    def run():
        for _, fn in calls:
            fn()
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    pass_us = (time.perf_counter() - t0) * 1e6 / steps
    op_us = {}
    for j, (op, _) in enumerate(calls):
        evs = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(steps * len(calls) * 300000))   # over 100 us per queued launch
        for e0, e1 in evs:
            for i, (_, fn) in enumerate(calls):
                if i == j:
                    e0.record(stream)
                fn()
                if i == j:
                    e1.record(stream)
        torch.cuda.synchronize()
        op_us[op] = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps * 1e3
    rep_us = {op: repeated_us(torch, stream, fn, steps) for op, fn in calls}
    return pass_us, op_us, rep_us, run


def repeated_us(torch, stream, fn, reps):
    """Average duration (us) of `reps` back-to-back launches of fn, timed with
    HIP events on the launch stream behind a spin kernel (so the host's call
    overhead does not leave the GPU idle between the launches)."""
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(reps * 300000))   # over 100 us of spinning per queued launch
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def copy_peak(torch, dev, stream):
    """GB/s of a plain 1 GiB device-to-device copy (read + write bytes)."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    st = iter_stats(lambda: dst.copy_(src), torch, stream, 5)
    return 2 * (1 << 30) / (st["median_us"] / 1e6) / 1e9


# ------------------------------------------------------------------ workloads

def device_inputs(w, wl, torch, dev):
    """The prefill inputs of workload w on the device. The prefill workload
    and the tiny one use the seeded CPU draws of workloads.py; the GQA and
    varlen workloads (1 GB and more) are drawn on the GPU with a seeded
    generator, in the same distributions (workloads.device_prefill_inputs;
    varlen: the lengths are the CPU draw, made first as in workloads.py)."""
    if w.name in ("prefill", "tiny"):
        d = wl.prefill_inputs(w)
        t = {n: d[n].to(dev) for n in ("x", "w", "a", "b", "A_log", "dt_bias")}
        t["S0"] = None if d["S0"] is None else d["S0"].to(dev)
        t["cu"] = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(dev)
        return t, d["B"], d["T"], d["N"]
    d = wl.device_prefill_inputs(w, dev)
    t = {n: d[n] for n in ("x", "w", "a", "b", "A_log", "dt_bias", "S0")}
    t["cu"] = d["cu_seqlens"]
    return t, d["B"], d["T"], d["N"]


def run_prefill_part(part, args, gdn, wl, torch, dev, stream, chain_ops=False):
    """One prefill workload: the whole prefill (two launches, events between
    them), per-iteration statistics back to back and flushed; the chunked
    forward alone (prepare + scan) on resident q, k, v, g, beta; with
    chain_ops, the four per-step calls timed one by one as well."""
    w = wl.WORKLOADS[PART_WORKLOAD[part]]
    t, B, T, N = device_inputs(w, wl, torch, dev)
    Hk, K, H, V = w.Hk, w.K, w.H, w.V
    dims = dict(Hk=Hk, K=K, H=H, V=V)
    n_seqs = 0 if t["cu"] is None else N
    cu = t["cu"]
    if cu is None:
        n_chunks = B * ((T + 63) // 64)
    else:
        lens = (cu[1:] - cu[:-1]).cpu()
        n_chunks = int(((lens + 63) // 64).sum())
    es = 2 if w.dtype == torch.bfloat16 else 4
    acc = accounting(B * T, n_chunks, N, H, Hk, K, V, es, s0=t["S0"] is not None)
    tokens = B * T
    res = {"workload": _workload_name(w, B, T, N), "tokens": tokens}
    o = torch.empty((B, T, H, V), dtype=w.dtype, device=dev)
    fs = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    flush = None if args.no_flush else Flush(torch, dev)
    kernels = {}
    steps, warm = args.steps, args.warmup

    if w.dtype == torch.bfloat16:
        ws = torch.empty(max(1, gdn.gdn_prefill_workspace_size(B, T, H, Hk, K, V, n_seqs)),
                         dtype=torch.uint8, device=dev)
        calls = [("prefill_prepare",
                  lambda: gdn.gdn_prefill_prepare(t["x"], t["w"], t["a"], t["b"], t["A_log"],
                                                  t["dt_bias"], ws, cu_seqlens=cu, **dims)),
                 ("prefill_scan",
                  lambda: gdn.gdn_prefill_scan(t["x"], t["w"], ws, initial_state=t["S0"],
                                               cu_seqlens=cu, o=o, final_state=fs, **dims))]
        pass_us, op_us, rep_us, run = timed_ops(torch, stream, calls, steps, warm)
        st = {"back_to_back": iter_stats(run, torch, stream, steps)}
        if flush:
            st["flushed"] = iter_stats(run, torch, stream, steps, flush)
        res["prefill"] = {"us": pass_us, "tokens_per_s": tokens / (pass_us * 1e-6),
                          "hbm_frac": acc["prefill"]["bytes"] / (pass_us * 1e-6) / (HBM_PEAK_GBS * 1e9),
                          "algorithmic_bytes": acc["prefill"]["bytes"], "iters": st}
        for kind, s in st.items():
            s["tokens_per_s"] = tokens / (s["median_us"] * 1e-6)
            s["hbm_frac"] = acc["prefill"]["bytes"] / (s["median_us"] * 1e-6) / (HBM_PEAK_GBS * 1e9)
        res["prefill"]["chunk_fwd"] = chunk_fwd_report(acc, tokens, sum(op_us.values()))
        for op, us in op_us.items():
            kernels[op] = kernel_report(part, op, us, acc[op]["bytes"], rep_us[op])
        del ws

    # the per-step path: conv1d + gates produce resident q, k, v, g, beta; the
    # chunked forward alone (the headline metric's unit) is prepare + scan
    y = torch.empty_like(t["x"])
    g = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    beta = torch.empty_like(g)
    q, k, v = gdn.split_qkv(y, Hk, K, H, V)
    ws2 = torch.empty(gdn.gdn_chunk_fwd_workspace_size(B, T, H, Hk, K, V, n_seqs, w.dtype),
                      dtype=torch.uint8, device=dev)
    conv = ("conv1d", lambda: gdn.gdn_conv1d_causal(t["x"], t["w"], y=y, cu_seqlens=cu, silu=True))
    gate = ("gate_prepare", lambda: gdn.gdn_gate_prepare(t["a"], t["b"], t["A_log"], t["dt_bias"],
                                                         g=g, beta=beta))
    prep = ("chunk_prepare", lambda: gdn.gdn_chunk_prepare(q, k, g, beta, ws2, cu_seqlens=cu))
    scan = ("chunk_scan", lambda: gdn.gdn_chunk_scan(q, k, v, o, ws2, initial_state=t["S0"],
                                                     final_state=fs, cu_seqlens=cu))
    conv[1]()
    gate[1]()
    calls = [conv, gate, prep, scan] if chain_ops else [prep, scan]
    pass_us, op_us, rep_us, run = timed_ops(torch, stream, calls, steps, warm)
    if chain_ops:
        res["chain"] = {"us": pass_us, "tokens_per_s": tokens / (pass_us * 1e-6)}

    def chunk():
        prep[1]()
        scan[1]()
    res["chunk_fwd"] = chunk_fwd_report(acc, tokens, op_us["chunk_prepare"] + op_us["chunk_scan"],
                                        BF16_PEAK_TFLOPS if es == 2 else FP32_PEAK_TFLOPS)
    st = {"back_to_back": iter_stats(chunk, torch, stream, steps)}
    if flush:
        st["flushed"] = iter_stats(chunk, torch, stream, steps, flush)
    for kind, s in st.items():
        s.update({kk: vv for kk, vv in chunk_fwd_report(
            acc, tokens, s["median_us"], BF16_PEAK_TFLOPS if es == 2 else FP32_PEAK_TFLOPS).items()
            if kk in ("tokens_per_s", "mfma_frac", "hbm_frac")})
    res["chunk_fwd"]["iters"] = st
    for op, us in op_us.items():
        kernels[op] = kernel_report(part, op, us, acc[op]["bytes"], rep_us[op])
    res["kernels"] = kernels
    return res, acc


def _workload_name(w, B, T, N):
    dt = "bf16" if w.dtype.is_floating_point and w.dtype.itemsize == 2 else "fp32"
    s = f"{w.name} {dt} B={B} T={T} H={w.H} Hk={w.Hk} K={w.K} V={w.V} chunk=64"
    if w.n_seqs:
        s += f" ({N} packed sequences, lengths 1..{w.max_len})"
    if w.s0_std:
        s += f", S0 ~N(0, {w.s0_std})"
    return s + ", conv1d W=4 + SiLU over q|k|v, fp32 state"


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
    tr = load_traffic("c5", "decode")
    return {"req_per_s": wd.n * steps / (ms / 1e3), "us_per_step": per_s * 1e6,
            "kernel": KERNELS["c5"]["decode"][0],
            "roofline": {"bound": "hbm", "achieved": nbytes / per_s / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": nbytes / per_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": tr, "traffic_ratio": None if tr is None else tr / nbytes},
            "algorithmic_bytes_per_step": nbytes,
            "workload": f"decode bf16 n={wd.n} M={wd.M} H={wd.H} G={wd.G} P=N={wd.K}, "
                        f"fp32 state in place, {steps} steps"}


def _time_launches(torch, stream, fn, reps):
    """Average us of fn() over reps launches, HIP events on the launch stream."""
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
    """Average us per launch of fn() replayed from a captured HIP graph of reps
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


# ----------------------------------------------------------- profile summaries

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
    s = name.split("(")[0]
    s = s[5:] if s.startswith("void ") else s
    s = s[5:] if s.startswith("gdn::") else s
    return s.replace("__bf16", "bf16")[:80]


def _read_csv(path):
    import csv
    return list(csv.DictReader(open(path)))


def summarize_stats(csv_path, out_md, command, part, bench_log=None):
    """Kernel time table from rocprofv3's kernel trace (one row per dispatch),
    one line per (kernel, grid, workgroup)."""
    import collections
    rows = _read_csv(csv_path)
    groups = collections.OrderedDict()
    for r in rows:
        key = (_kernel_stem(r["Kernel_Name"]),
               int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]),
               int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in groups.values())
    items = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    w = PART_WORKLOAD.get(part, part)
    title = (f"{w} workload ({part})" if part in PART_WORKLOAD else
             "the default bench run (every workload, cache-flushed iterations included)")
    lines = [f"# Kernel times, {title} (rocprofv3 --kernel-trace --stats)", "",
             f"Command: `{command}`", "",
             "One line per kernel and launch shape (grid = work-items), from the kernel trace.", "",
             "| kernel | grid | workgroup | calls | average (us) | median (us) | min (us) | max (us) | share |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (name, grid, wg), d in items:
        med = sorted(d)[len(d) // 2]
        lines.append(f"| `{name}` | {grid} | {wg} | {len(d)} | {sum(d) / len(d):.2f} | {med:.2f} | "
                     f"{min(d):.2f} | {max(d):.2f} | {100 * sum(d) / total:.1f}% |")
    lines += ["", "(`at::cuda::` rows are the spin kernels that hold the stream while the host",
              "queues the repeated launches of one op; the calls include the warm-up passes.)"]
    if bench_log:
        js = [ln for ln in open(bench_log) if ln.startswith("{")]
        b = json.loads(js[-1])
        lines += ["", "The same run's bench figures (HIP events on the launch stream around the",
                  "op inside the passes; in brackets, back-to-back launches of the op alone), for",
                  "comparison with the trace above:", ""]
        parts_ = [part] if part in PART_WORKLOAD else list(b.get("configs", {}))
        for p_ in parts_:
            cfg = b.get("configs", {}).get(p_, {})
            for op, k in cfg.get("kernels", {}).items():
                rep = f" ({k['us_repeated']:.2f} us)" if k.get("us_repeated") else ""
                lines.append(f"- {p_} {op} (`{k['kernel']}`): {k['us']:.2f} us{rep}")
            if "decode" in cfg:
                lines.append(f"- {p_} decode step (`{cfg['decode']['kernel']}`): "
                             f"{cfg['decode']['us_per_step']:.2f} us")
        lines += ["", "The same run's pass figures (wall clock over the timed passes; per-iteration",
                  "HIP-event medians back to back and with the caches flushed between iterations):",
                  ""]
        if b.get("value"):
            head = f"- headline: {b['value'] / 1e6:.2f} M tokens/s ({b['ms_per_step'] * 1e3:.1f} us per step)"
            if "value_flushed" in b:
                fl = b["value_flushed"]
                head += (f"; flushed {fl['value'] / 1e6:.2f} M tokens/s ({fl['median_us']:.1f} us), "
                         f"HBM fraction {fl['hbm_frac']:.3f}")
            if "roofline" in b:
                rf = b["roofline"]
                head += (f"; roofline `{rf['kernel']}` {rf['achieved']:.0f} GB/s = {rf['frac']:.3f} "
                         f"of {rf['peak']:.0f}")
            lines.append(head)
        for p_ in parts_:
            cfg = b.get("configs", {}).get(p_, {})
            for key in ("prefill", "chunk_fwd"):
                e = cfg.get(key) if key in cfg else None
                if not e:
                    continue
                it = e.get("iters", {})
                bb, fl = it.get("back_to_back", {}), it.get("flushed", {})
                extra = (f", MFMA fraction {e['mfma_frac']:.3f} (dense count {e['mfma_frac_dense']:.3f})"
                         if "mfma_frac" in e else "")
                lines.append(f"- {p_} {key}: {e['us']:.1f} us, {e['tokens_per_s'] / 1e6:.2f} M tokens/s, "
                             f"HBM fraction {e['hbm_frac']:.3f}{extra}; medians {bb.get('median_us', 0):.1f} us "
                             f"back to back, {fl.get('median_us', 0):.1f} us flushed")
            if "chain" in cfg:
                lines.append(f"- {p_} four per-step calls: {cfg['chain']['us']:.1f} us")
            if "decode" in cfg:
                dd = cfg["decode"]
                lines.append(f"- {p_} decode: {dd['req_per_s'] / 1e6:.3f} M requests/s, "
                             f"{dd['roofline']['achieved']:.0f} GB/s = {dd['roofline']['frac']:.3f} of HBM")
        if "cpu_baseline" in b:
            cb = b["cpu_baseline"]
            lines.append(f"- oracle on the host: {cb['value']:.0f} {cb['unit']} on {cb['cores']} threads "
                         f"({cb['sample']})")
    open(out_md, "w").write("\n".join(lines) + "\n")


def summarize_traffic(fetch_csv, write_csv, command, part):
    """Per-kernel HBM bytes per launch in one part's run: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by the factor that makes the
    plain 1 GiB device copy (the runtime's buffer-copy kernel, --copy-probe)
    read and write 1 GiB. Merged into profiles/traffic.json under the part."""
    import collections

    def per_dispatch(path, counter):
        rows = [r for r in _read_csv(path) if r["Counter_Name"] == counter]
        acc = collections.defaultdict(float)
        names = {}
        for r in rows:
            d = int(r["Dispatch_Id"])
            acc[d] += float(r["Counter_Value"]) * 1024.0   # KiB -> bytes
            names[d] = r["Kernel_Name"]
        return acc, names

    fetch, fnames = per_dispatch(fetch_csv, "FETCH_SIZE")
    write, wnames = per_dispatch(write_csv, "WRITE_SIZE")
    gib = float(1 << 30)

    # the probe copies are the last three buffer-copy dispatches of each run
    def probe(table, names):
        ids = sorted(d for d, n in names.items() if "copybuffer" in n.lower())[-3:]
        vals = [table[d] for d in ids]
        return sum(vals) / len(vals) if vals else None
    pf, pw = probe(fetch, fnames), probe(write, wnames)
    ff = gib / pf if pf else None
    fw = gib / pw if pw else None
    path = os.path.join(PROFILES, "traffic.json")
    res = json.load(open(path)) if os.path.exists(path) else {}
    res.setdefault("parts", {})
    res["calibration"] = {"copy_kernel_bytes": gib, "copy_fetch_raw": pf, "copy_write_raw": pw,
                          "fetch_factor": ff, "write_factor": fw}
    ent = {}
    srcs = {stem: src for stem, src in KERNELS.get(part, {}).values()}
    by_name = collections.defaultdict(list)
    for d, n in fnames.items():
        by_name[_kernel_stem(n)].append(d)
    wby = collections.defaultdict(list)
    for d, n in wnames.items():
        wby[_kernel_stem(n)].append(write[d])
    for stem, ids in by_name.items():
        if stem not in srcs or ff is None or fw is None:
            continue
        fb = sum(fetch[d] for d in ids) / len(ids) * ff
        wv = wby.get(stem, [])
        wb = sum(wv) / len(wv) * fw if wv else 0.0
        ent[stem] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                     "launches": len(ids), "source_sha": source_hash(srcs[stem])}
    res["parts"][part] = {"command": command, "kernels": ent}
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    return res


def summarize_counters(csv_path, out_md, command, part, cus=256, simds=4, xcds=8):
    """Per kernel: every counter of a --pmc run, summed over the XCDs and
    averaged over its launches; with GRBM_GUI_ACTIVE, per-CU busy fractions
    of the SQ/TA/TD/TCP busy counters (counter / (active cycles per XCD x CUs),
    and / SIMDs for the per-SIMD MFMA busy counter)."""
    import collections
    rows = _read_csv(csv_path)
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in rows:
        d = int(r["Dispatch_Id"])
        per[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = _kernel_stem(r["Kernel_Name"])
    groups = collections.OrderedDict()
    for d in sorted(per):
        groups.setdefault(names[d], []).append(per[d])
    counters = sorted({c for d in per.values() for c in d})
    w = PART_WORKLOAD.get(part, part)
    lines = [f"# Counters, {w} workload ({part}) (rocprofv3 --pmc)", "", f"Command: `{command}`", "",
             "Values per launch (summed over the XCDs, averaged over launches). Busy fractions:",
             f"counter / (GRBM_GUI_ACTIVE / {xcds} x {cus} CUs), and x {simds} SIMDs more for",
             "SQ_VALU_MFMA_BUSY_CYCLES.", "",
             "| kernel | launches | " + " | ".join(counters) + " | busy fractions |",
             "|---|---|" + "---|" * len(counters) + "---|"]
    for name, cs in groups.items():
        avg = {c: sum(x.get(c, 0.0) for x in cs) / len(cs) for c in counters}
        act = avg.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        fr = []
        for c in counters:
            if not act or not c.endswith(("BUSY", "BUSY_CYCLES", "_BUSY_CU")) and "BUSY" not in c:
                continue
            den = act * cus * (simds if c == "SQ_VALU_MFMA_BUSY_CYCLES" else 1)
            fr.append(f"{c} {avg[c] / den:.3f}")
        lines.append(f"| `{name}` | {len(cs)} | " + " | ".join(f"{avg[c]:.4g}" for c in counters)
                     + f" | {'; '.join(fr)} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


# ------------------------------------------------------------------------ main

def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.command,
                           args.part)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats[0], args.summarize_stats[1], args.command, args.part,
                        args.bench_log)
        return
    if args.summarize_traffic:
        print(json.dumps(summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1],
                                           args.command, args.part), indent=1))
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
    parts = [p for p in args.only.split(",") if p]
    global SCAN_FORM
    SCAN_FORM = args.scan_form
    gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, args.scan_form)
    for p in parts:
        if p not in PARTS:
            raise SystemExit(f"unknown part {p} (one of {PARTS})")

    w = wl.WORKLOADS["prefill"]
    out = {"metric": "GDN chunk-fwd tokens/s (H=16,d=128,T=4096); decode req/s; % of roofline",
           "value_covers": "the whole prefill step: conv1d + SiLU, gates and the chunked forward",
           "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"prefill bf16 B={w.B} H={w.H} Hk={w.Hk} T={w.T} K=V={w.K} "
                                  "chunk=64, conv1d W=4 + SiLU over C=6144, fp32 state",
                      "global_batch": w.B, "seq_len": w.T, "parallelism": "single-gpu"},
           "configs": {}}

    for p in parts:
        if p == "c5":
            out["configs"]["c5"] = {"decode": run_decode(args, gdn, wl, torch, dev, stream),
                                    "gdp_steps": run_gdp_steps(gdn, wl, torch, dev, stream)}
            continue
        res, acc = run_prefill_part(p, args, gdn, wl, torch, dev, stream, chain_ops=p in ("c1", "c2"))
        out["configs"][p] = res
        if p == "c2":
            pf = res["prefill"]
            out["value"] = pf["tokens_per_s"]
            out["ms_per_step"] = pf["us"] / 1e3
            if "flushed" in pf["iters"]:
                fl = pf["iters"]["flushed"]
                out["value_flushed"] = {
                    "value": fl["tokens_per_s"], "median_us": fl["median_us"],
                    "hbm_frac": fl["hbm_frac"],
                    "protocol": "the same step timed per iteration with HIP events, a 512 MB "
                                "write between iterations (outside the timed region) evicting the "
                                "256 MB Infinity Cache and the L2s; median of the timed iterations"}
            ops = {op: k for op, k in res["kernels"].items() if op.startswith("prefill_")}
            dom = max(ops, key=lambda op: ops[op]["us"])
            k = ops[dom]
            out["roofline"] = {"kernel": k["kernel"], "bound": "hbm", "achieved": k["achieved_GBs"],
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": k["hbm_frac"],
                               "traffic": k["traffic"], "traffic_ratio": k["traffic_ratio"],
                               "share_bytes": k["share_bytes"], "us": k["us"]}
    # the copy-kernel rate, a practical HBM reference point (read + write bytes
    # of a plain device copy)
    out["copy_peak_GBs"] = copy_peak(torch, dev, stream)
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu and "c2" in parts:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_batch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
