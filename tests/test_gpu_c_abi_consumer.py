"""The C ABI from C++ alone: tests/c_abi/consumer (built by
__graft_entry__.build()) runs gdn_chunk_fwd and gdn_prefill in a process of
its own through include/gdn.h, on device memory it allocates itself and a
stream it creates, with no Python and no torch. Its results must equal the
Python binding's bit for bit on the same inputs (the binding only marshals),
and match the fp64 oracle."""
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16 = torch.bfloat16
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CONSUMER = os.path.join(ROOT, "tests", "c_abi", "consumer")


def _save(dirpath, name, t):
    t = t.contiguous().cpu()
    if t.dtype == BF16:
        t = t.view(torch.int16)
    t.numpy().tofile(os.path.join(dirpath, name + ".bin"))


def _consume(mode, dirpath, d, scale=1.0, l2norm=True):
    if not os.path.exists(CONSUMER):
        pytest.fail("tests/c_abi/consumer is not built: run __graft_entry__.build()")
    n_seqs = 0 if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    if d["S0"] is not None:
        _save(dirpath, "S0", d["S0"])
    if n_seqs:
        _save(dirpath, "cu", d["cu_seqlens"])
    args = [CONSUMER, mode, dirpath] + [str(x) for x in (
        d["B"], d["T"], d["H"], d["Hk"], d["K"], d["V"], n_seqs, scale, int(l2norm),
        int(d["S0"] is not None))]
    print(f"consumer: {mode} B={d['B']} T={d['T']} n_seqs={n_seqs}", flush=True)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"consumer exit {r.returncode}: {r.stderr}"
    N = n_seqs or d["B"]
    o = torch.from_numpy(np.fromfile(os.path.join(dirpath, "o.bin"), np.int16)).view(BF16)
    sf = torch.from_numpy(np.fromfile(os.path.join(dirpath, "sf.bin"), np.float32))
    return (o.reshape(d["B"], d["T"], d["H"], d["V"]), sf.reshape(N, d["H"], d["K"], d["V"]))


CHUNK_CASES = {
    "dense": dict(B=2, T=200, H=4, Hk=2, K=128, V=128, s0_std=0.05),
    "packed": dict(B=1, T=1 + 64 + 130, H=2, Hk=2, K=64, V=128, lengths=[1, 64, 0, 130]),
}


@pytest.mark.parametrize("case", list(CHUNK_CASES))
def test_consumer_chunk_fwd(gpu, case):
    kw = dict(CHUNK_CASES[case])
    d = wl.chunk_inputs(dtype=BF16, decay="weak", seed=31, **kw)
    with tempfile.TemporaryDirectory() as tmp:
        for n in ("q", "k", "v", "g", "beta"):
            _save(tmp, n, d[n])
        o, sf = _consume("chunk_fwd", tmp, d, scale=0.5)
    t = {n: (None if d[n] is None else d[n].to(DEV)) for n in ("q", "k", "v", "g", "beta", "S0", "cu_seqlens")}
    bo, bsf = gpu.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["S0"],
                                cu_seqlens=t["cu_seqlens"], scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(o, bo.cpu()) and torch.equal(sf, bsf.cpu()), "consumer differs from the binding"
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    ro, rs = oracle.gated_delta_rule(to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["g"]),
                                     to_np(d["beta"]), S0=None if d["S0"] is None else to_np(d["S0"]),
                                     cu_seqlens=cu, scale=0.5)
    assert_close(to_np(o), ro, BF16, f"consumer chunk_fwd {case} o")
    assert_close(to_np(sf), rs, BF16, f"consumer chunk_fwd {case} state")


PREFILL_CASES = {
    "dense": dict(T=150, B=2),
    "packed": dict(lengths=[3, 70, 0, 129]),
}


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_consumer_prefill(gpu, case):
    w = wl.WORKLOADS["prefill"] if case == "dense" else wl.WORKLOADS["varlen"]
    d = wl.prefill_inputs(w, **PREFILL_CASES[case])
    with tempfile.TemporaryDirectory() as tmp:
        for n in ("x", "w", "a", "b", "A_log", "dt_bias"):
            _save(tmp, n, d[n])
        o, sf = _consume("prefill", tmp, d)
    t = {n: (None if d[n] is None else d[n].to(DEV))
         for n in ("x", "w", "a", "b", "A_log", "dt_bias", "S0", "cu_seqlens")}
    bo, bsf = gpu.gdn_prefill(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"], Hk=w.Hk,
                              K=w.K, H=w.H, V=w.V, initial_state=t["S0"], cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o, bo.cpu()) and torch.equal(sf, bsf.cpu()), "consumer differs from the binding"
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    B, T, C = d["x"].shape
    y = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]), cu_seqlens=cu, silu=True)
    nq = w.Hk * w.K
    q = y[:, :, :nq].reshape(B, T, w.Hk, w.K)
    k = y[:, :, nq:2 * nq].reshape(B, T, w.Hk, w.K)
    v = y[:, :, 2 * nq:].reshape(B, T, w.H, w.V)
    g, beta = oracle.gate_prepare(to_np(d["a"]), to_np(d["b"]), to_np(d["A_log"]), to_np(d["dt_bias"]))
    ro, rs = oracle.gated_delta_rule(q, k, v, g, beta, S0=None if d["S0"] is None else to_np(d["S0"]),
                                     cu_seqlens=cu)
    assert_close(to_np(o), ro, BF16, f"consumer prefill {case} o")
    assert_close(to_np(sf), rs, BF16, f"consumer prefill {case} state")
