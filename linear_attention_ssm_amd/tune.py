"""Offline sweep of the launch-configuration knobs (gdn_tune_set).

The pages tune their kernels' block sizes per shape with an autotuner (the
"ZzCompute" entry, item 1; item 4 settles on one configuration for every
shape). Here the same question is answered offline: for each workload and
each value of each knob, the entry points the knob affects run on the same
seeded inputs, their outputs are compared bit for bit with those of the
automatic setting (a knob changes scheduling only), and they are timed with
HIP events on the stream they run on.

Knobs swept:
  GDN_TUNE_SCAN_FORM     bf16 scan workgroup form: value-column groups with
                         role-split waves (1) or one workgroup per (sequence,
                         head) unit (2), swept together with
  GDN_TUNE_SCAN_TILES    value-column tiles per scan workgroup (BV = 16 x tiles),
                         per compute wave in the whole-unit form
  GDN_TUNE_CONV_RUN      tokens per thread of the prefill conv
  GDN_TUNE_CONV_THREADS  threads per workgroup of the prefill conv
The decode kernel has no knob; its step is timed once for reference. The
kernels are all non-persistent (one workgroup per unit of work), so there is
no persistent-versus-not axis to sweep.

    python -m linear_attention_ssm_amd.tune [--reps N] [--out FILE.md] [--only NAME ...]

Prints one JSON line per measurement; with --out also writes a markdown table.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import torch  # noqa: E402

import linear_attention_ssm_amd as gdn  # noqa: E402
import workloads as wl  # noqa: E402

# (scan form, scan tiles); (0, 0) is the automatic choice
SCAN_VALUES = {torch.bfloat16: [(0, 0), (1, 1), (1, 2), (2, 2), (2, 1)],
               torch.float32: [(0, 0), (0, 1), (0, 4)]}
CONV_RUNS = [8, 16, 32]
CONV_THREADS = [64, 128, 256]


def _time(fn, reps, stream):
    """us per call: `reps` calls captured in a HIP graph and replayed, so that
    host-side argument marshalling does not show in short launches (direct
    calls where capture is not possible)."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph = None
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                for _ in range(reps):
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = g
    except RuntimeError:
        graph = None
    torch.cuda.synchronize()
    if graph is not None:
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    else:
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def _cases():
    """(name, workload, prefill_inputs overrides): the five configurations'
    prefill shapes plus the prefill workload at other sequence lengths."""
    W = wl.WORKLOADS
    return [
        ("tiny", W["tiny"], {}),
        ("prefill", W["prefill"], {}),
        ("prefill T=1024", W["prefill"], dict(T=1024)),
        ("prefill T=16384", W["prefill"], dict(T=16384)),
        ("gqa", W["gqa"], {}),
        ("varlen", W["varlen"], {}),
    ]


def _reset():
    for k in (gdn.GDN_TUNE_SCAN_TILES, gdn.GDN_TUNE_CONV_RUN, gdn.GDN_TUNE_CONV_THREADS,
              gdn.GDN_TUNE_SCAN_FORM):
        gdn.gdn_tune_set(k, 0)


def sweep_prefill(name, w, kw, reps, rounds, dev, stream, emit):
    d = wl.prefill_inputs(w, **kw)
    x, cw = d["x"].to(dev), d["w"].to(dev)
    a, b = d["a"].to(dev), d["b"].to(dev)
    A_log, dt_bias = d["A_log"].to(dev), d["dt_bias"].to(dev)
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(dev)
    S0 = None if d["S0"] is None else d["S0"].to(dev)
    dims = dict(Hk=w.Hk, K=w.K, H=w.H, V=w.V)
    tokens = d["B"] * d["T"]
    y = torch.empty_like(x)

    # the forward: the whole-prefill entry for bf16, the per-step chain for fp32
    if w.dtype == torch.bfloat16:
        n = 0 if cu is None else cu.numel() - 1
        ws = torch.empty(gdn.gdn_prefill_workspace_size(d["B"], d["T"], w.H, w.Hk, w.K, w.V, n),
                         dtype=torch.uint8, device=dev)

        def fwd():
            return gdn.gdn_prefill(x, cw, a, b, A_log, dt_bias, initial_state=S0, cu_seqlens=cu,
                                   workspace=ws, **dims)
        entry = "gdn_prefill"
    else:
        def fwd():
            return gdn.prefill_chain(x, cw, a, b, A_log, dt_bias, initial_state=S0,
                                     cu_seqlens=cu, **dims)
        entry = "prefill_chain"

    # each setting is timed in `rounds` interleaved passes (the best pass
    # counts), so that clock changes during the sweep do not favour an order
    _reset()
    ref = [t.clone() for t in fwd()]
    values = SCAN_VALUES[w.dtype]
    best = {v: float("inf") for v in values}
    equal = {v: True for v in values}
    for _ in range(rounds):
        for v in values:
            gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, v[0])
            gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, v[1])
            got = fwd()
            equal[v] &= all(torch.equal(g_, r_) for g_, r_ in zip(got, ref))
            best[v] = min(best[v], _time(fwd, reps, stream))
    for v in values:
        emit(dict(workload=name, entry=entry, knob="scan_form,scan_tiles",
                  value=0 if v == (0, 0) else f"{v[0]},{v[1]}", us=best[v],
                  tokens_per_s=tokens / (best[v] / 1e6), equal=equal[v]))
    _reset()

    def conv():
        return gdn.gdn_conv1d_causal(x, cw, y=y, cu_seqlens=cu, silu=True)
    yref = conv().clone()
    cfgs = [(run, nth) for run in CONV_RUNS for nth in CONV_THREADS]
    best = {c: float("inf") for c in cfgs}
    equal = {c: True for c in cfgs}
    for _ in range(rounds):
        for run, nth in cfgs:
            gdn.gdn_tune_set(gdn.GDN_TUNE_CONV_RUN, run)
            gdn.gdn_tune_set(gdn.GDN_TUNE_CONV_THREADS, nth)
            equal[(run, nth)] &= torch.equal(conv(), yref)
            best[(run, nth)] = min(best[(run, nth)], _time(conv, reps, stream))
    for run, nth in cfgs:
        us = best[(run, nth)]
        emit(dict(workload=name, entry="gdn_conv1d_causal", knob="conv_run,conv_threads",
                  value=f"{run},{nth}", us=us,
                  GBs=2 * x.numel() * x.element_size() / (us / 1e6) / 1e9,
                  equal=equal[(run, nth)]))
    _reset()


def time_decode(reps, dev, stream, emit):
    wd = wl.WORKLOADS["decode"]
    st = wl.decode_state_inputs(wd)
    x, ba = wl.decode_step_inputs(wd, 0)
    state = st["state"].to(dev)
    x, ba = x.to(dev), ba.to(dev)
    A_log, dt_bias = st["A_log"].to(dev), st["dt_bias"].to(dev)
    o = torch.empty((wd.n, wd.H, wd.V), dtype=torch.bfloat16, device=dev)

    def step():
        gdn.gdn_recurrent_decode(x, ba, A_log, dt_bias, state, wd.M, wd.H, wd.G, wd.V, wd.K, o=o)
    us = _time(step, reps, stream)
    emit(dict(workload="decode", entry="gdn_recurrent_decode", knob="(none)", value="-", us=us,
              req_per_s=wd.n / (us / 1e6), equal=True))


def write_table(rows, path, command):
    lines = ["# Launch-configuration sweep (gdn_tune_set)", "",
             f"Command: `{command}`", "",
             "Each knob value against the automatic setting (value 0 / `auto`) on the same",
             "seeded inputs; `equal` = outputs identical bit for bit to the automatic setting;",
             "each time is the best of interleaved passes over the settings.", "",
             "| workload | entry | knob | value | us / call | rate | equal | best |",
             "|---|---|---|---|---|---|---|---|"]
    groups = {}
    for r in rows:
        groups.setdefault((r["workload"], r["entry"], r["knob"]), []).append(r)
    for (wk, entry, knob), rs in groups.items():
        best = min(rs, key=lambda r: r["us"])
        for r in rs:
            rate = (f"{r['tokens_per_s'] / 1e6:.1f} M tok/s" if "tokens_per_s" in r else
                    f"{r['GBs']:.0f} GB/s" if "GBs" in r else
                    f"{r['req_per_s'] / 1e6:.2f} M req/s" if "req_per_s" in r else "")
            v = "auto" if r["value"] == 0 else r["value"]
            lines.append(f"| {wk} | `{entry}` | {knob} | {v} | {r['us']:.1f} | {rate} | "
                         f"{'yes' if r['equal'] else 'NO'} | {'*' if r is best else ''} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--reps", type=int, default=20, help="calls per timing")
    p.add_argument("--rounds", type=int, default=3, help="interleaved passes over the settings")
    p.add_argument("--out", default=None, help="markdown table to write")
    p.add_argument("--only", nargs="*", default=None, help="workload names to run")
    args = p.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the sweep needs a GPU")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rows = []

    def emit(r):
        rows.append(r)
        print(json.dumps(r), flush=True)

    # bring the clocks up before the first timing: half a second of work
    t0 = time.time()
    warm = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    while time.time() - t0 < 0.5:
        warm.add_(1)
    torch.cuda.synchronize()
    del warm
    for name, w, kw in _cases():
        if args.only and name not in args.only:
            continue
        sweep_prefill(name, w, kw, args.reps, args.rounds, dev, stream, emit)
    if not args.only or "decode" in args.only:
        time_decode(args.reps, dev, stream, emit)
    _reset()
    if args.out:
        write_table(rows, args.out, "python -m linear_attention_ssm_amd.tune" +
                    (f" --reps {args.reps}" if args.reps != 20 else "") + f" --out {args.out}")
    bad = [r for r in rows if not r["equal"]]
    print(json.dumps({"cases": len(rows), "not_equal": len(bad), "seconds": time.time() - t0}),
          flush=True)
    if bad:
        raise SystemExit(f"{len(bad)} settings changed the results")


if __name__ == "__main__":
    main()
