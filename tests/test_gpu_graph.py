"""The entry points under HIP graph capture, the way a serving loop uses them:
inputs, outputs and the workspace preallocated, the call captured once and
replayed. Every replay runs on fresh inputs (copied into the captured buffers
by eager work between replays, with synchronisations) and must give the bits
of the same call made eagerly on those inputs. The library itself records no
memset and makes no host synchronisation, so the captured graph holds only
its kernel launches."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16 = torch.bfloat16
REPLAYS = 4


def _prefill_bufs(gdn, w, d):
    n_seqs = 0 if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    N = n_seqs or d["B"]
    t = {n: d[n].to(DEV) for n in ("x", "w", "a", "b", "A_log", "dt_bias")}
    t["S0"] = None if d["S0"] is None else d["S0"].to(DEV)
    t["cu"] = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(DEV)
    t["ws"] = torch.empty(gdn.gdn_prefill_workspace_size(d["B"], d["T"], w.H, w.Hk, w.K, w.V, n_seqs),
                          dtype=torch.uint8, device=DEV)
    t["o"] = torch.empty((d["B"], d["T"], w.H, w.V), dtype=BF16, device=DEV)
    t["sf"] = torch.empty((N, w.H, w.K, w.V), dtype=torch.float32, device=DEV)
    return t


@pytest.mark.parametrize("case", ["dense", "packed"])
def test_prefill_graph_replays(gpu, case):
    if case == "dense":
        w = wl.WORKLOADS["gqa"]
        inputs = [wl.prefill_inputs(w, T=500, seed=50 + r) for r in range(REPLAYS + 1)]
    else:
        w = wl.WORKLOADS["varlen"]
        inputs = [wl.prefill_inputs(w, lengths=[3, 200, 0, 129], seed=60 + r) for r in range(REPLAYS + 1)]
    t = _prefill_bufs(gpu, w, inputs[0])
    dims = dict(Hk=w.Hk, K=w.K, H=w.H, V=w.V)

    def call(o, sf):
        gpu.gdn_prefill(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"], initial_state=t["S0"],
                        cu_seqlens=t["cu"], workspace=t["ws"], o=o, final_state=sf, **dims)

    call(t["o"], t["sf"])            # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(t["o"], t["sf"])
    o_e, sf_e = torch.empty_like(t["o"]), torch.empty_like(t["sf"])
    for r in range(1, REPLAYS + 1):
        d = inputs[r]
        for n in ("x", "w", "a", "b", "A_log", "dt_bias"):
            t[n].copy_(d[n].to(DEV))
        if t["S0"] is not None:
            t["S0"].copy_(d["S0"].to(DEV))
        call(o_e, sf_e)              # eager, on the same inputs
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(t["o"], o_e), f"replay {r}: o differs from the eager call"
        assert torch.equal(t["sf"], sf_e), f"replay {r}: final state differs from the eager call"


def test_decode_graph_replays(gpu):
    # one decode token captured; each replay advances the captured state in
    # place, as eager calls advance their own copy
    w = wl.WORKLOADS["decode"]
    n = 64
    st = wl.decode_state_inputs(w, n=n)
    state_g = st["state"].to(DEV)
    state_e = state_g.clone()
    A_log, dt_bias = st["A_log"].to(DEV), st["dt_bias"].to(DEV)
    x0, ba0 = wl.decode_step_inputs(w, 0, n=n)
    x, ba = x0.to(DEV), ba0.to(DEV)
    o_g = torch.empty((n, w.H, w.V), dtype=BF16, device=DEV)
    args = (w.M, w.H, w.G, w.V, w.K)
    scratch = state_g.clone()
    gpu.gdn_recurrent_decode(x, ba, A_log, dt_bias, scratch, *args, o=o_g)   # warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu.gdn_recurrent_decode(x, ba, A_log, dt_bias, state_g, *args, o=o_g)
    for s in range(1, REPLAYS + 1):
        xs, bas = wl.decode_step_inputs(w, s, n=n)
        x.copy_(xs.to(DEV))
        ba.copy_(bas.to(DEV))
        o_e = gpu.gdn_recurrent_decode(x, ba, A_log, dt_bias, state_e, *args)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {s}: o differs"
        assert torch.equal(state_g, state_e), f"replay {s}: state differs"
