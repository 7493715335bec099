"""gdn_prefill (HIP, two launches) against the four-step chain and the oracle.

gdn_prefill folds the short convolution and the gates into the chunked
forward: the per-chunk solve convolves the q and k rows and forms the gates,
the scan convolves the value rows. Its contract is that it equals conv1d + SiLU -> gates -> chunk_fwd on
the same inputs bit for bit, so every case compares o and the final state
with torch.equal against that chain (whose kernels have their own parity
tests against the fp64 oracle); the small cases, which also carry a conv bias,
a scale and the no-normalisation branch, are compared with the oracle's
conv -> gates -> timestep recurrence directly. Inputs are the workloads'
seeded draws; the conv bias, where used, is a seeded N(0, 0.5) draw.
"""
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16 = torch.bfloat16


def _bias(C, seed=7):
    gen = torch.Generator().manual_seed(seed)
    return (torch.randn(C, generator=gen) * 0.5).to(BF16)


def _dev(d, bias):
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(DEV)
    S0 = None if d["S0"] is None else d["S0"].to(DEV)
    bb = None if bias is None else bias.to(DEV)
    return ({n: d[n].to(DEV) for n in ("x", "w", "a", "b", "A_log", "dt_bias")}, cu, S0, bb)


def _chain(gdn, d, bias=None, scale=1.0, l2norm=True):
    t, cu, S0, bb = _dev(d, bias)
    y = gdn.gdn_conv1d_causal(t["x"], t["w"], bias=bb, cu_seqlens=cu, silu=True)
    q, k, v = gdn.split_qkv(y, d["Hk"], d["K"], d["H"], d["V"])
    g, beta = gdn.gdn_gate_prepare(t["a"], t["b"], t["A_log"], t["dt_bias"])
    o, sf = gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu, scale=scale,
                              qk_l2norm=l2norm)
    torch.cuda.synchronize()
    return o, sf


def _fused(gdn, d, bias=None, scale=1.0, l2norm=True, **kw):
    t, cu, S0, bb = _dev(d, bias)
    o, sf = gdn.gdn_prefill(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                            Hk=d["Hk"], K=d["K"], H=d["H"], V=d["V"], bias=bb, initial_state=S0,
                            cu_seqlens=cu, scale=scale, qk_l2norm=l2norm, **kw)
    torch.cuda.synchronize()
    return o, sf


def _oracle(d, bias=None, scale=1.0, l2norm=True):
    B, T, C = d["x"].shape
    Hk, K, H, V = d["Hk"], d["K"], d["H"], d["V"]
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    y = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]),
                             bias=None if bias is None else to_np(bias), cu_seqlens=cu, silu=True)
    q = y[:, :, :Hk * K].reshape(B, T, Hk, K)
    k = y[:, :, Hk * K:2 * Hk * K].reshape(B, T, Hk, K)
    v = y[:, :, 2 * Hk * K:].reshape(B, T, H, V)
    g, beta = oracle.gate_prepare(to_np(d["a"]), to_np(d["b"]), to_np(d["A_log"]),
                                  to_np(d["dt_bias"]))
    S0 = None if d["S0"] is None else to_np(d["S0"])
    return oracle.gated_delta_rule(q, k, v, g, beta, S0=S0, cu_seqlens=cu, scale=scale,
                                   l2norm=l2norm)


def _equal(got, ref, what):
    (o, sf), (ro, rsf) = got, ref
    assert o.shape == ro.shape and sf.shape == rsf.shape, what
    assert torch.equal(o, ro), f"{what}: o differs from the chain"
    assert torch.equal(sf, rsf), f"{what}: final state differs from the chain"


def _shape(name, H, Hk, K, V, **kw):
    return wl.Workload(name, 2, BF16, H=H, Hk=Hk, K=K, V=V, **kw)


# small cases: (workload, prefill_inputs overrides)
SMALL = {
    # 5 chunks + a 1-row tail, two batch rows
    "prefill-321": (wl.WORKLOADS["prefill"], dict(T=321, B=2)),
    # GQA with an initial state and a 60-row tail
    "gqa-700": (wl.WORKLOADS["gqa"], dict(T=700)),
    # packed: sequences of 1..3 rows (the taps reach across), exact chunks,
    # one past a chunk, an empty sequence
    "varlen-edges": (wl.WORKLOADS["varlen"], dict(lengths=[1, 2, 3, 64, 0, 65, 130, 5, 200, 63])),
    # the other head dims
    "k64-v128": (_shape("k64", H=4, Hk=2, K=64, V=128, B=2, T=200), {}),
    "k128-v64": (_shape("v64", H=4, Hk=4, K=128, V=64, B=1, T=150), {}),
    "k64-v64": (_shape("kv64", H=8, Hk=8, K=64, V=64, B=3, T=97), {}),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_prefill_equals_chain_small(gpu, case):
    w, kw = SMALL[case]
    d = wl.prefill_inputs(w, **kw)
    _equal(_fused(gpu, d), _chain(gpu, d), case)


@pytest.mark.parametrize("case", ["prefill-321", "varlen-edges", "k64-v128"])
def test_prefill_bias_scale_no_norm_equals_chain(gpu, case):
    w, kw = SMALL[case]
    d = wl.prefill_inputs(w, **kw)
    bias = _bias(d["C"])
    _equal(_fused(gpu, d, bias=bias, scale=0.125), _chain(gpu, d, bias=bias, scale=0.125),
           case + " bias, scale")
    _equal(_fused(gpu, d, bias=bias, l2norm=False), _chain(gpu, d, bias=bias, l2norm=False),
           case + " bias, no l2norm")


@pytest.mark.parametrize("case", ["prefill-321", "varlen-edges", "k128-v64"])
def test_prefill_matches_oracle(gpu, case):
    w, kw = SMALL[case]
    d = wl.prefill_inputs(w, **kw)
    bias = _bias(d["C"])
    o, sf = _fused(gpu, d, bias=bias, scale=0.5)
    ro, rs = _oracle(d, bias=bias, scale=0.5)
    assert_close(to_np(o), ro, BF16, case + " o")
    assert_close(to_np(sf), rs, BF16, case + " state")


def test_prefill_no_tokens_and_no_final_state(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["gqa"], T=130)
    # no final state requested: o unchanged
    o1, sf1 = _fused(gpu, d)
    o2, sf2 = _fused(gpu, d, output_final_state=False)
    assert sf2 is None and torch.equal(o1, o2)
    # T = 0: nothing to do, the final state is the initial one
    d0 = wl.prefill_inputs(wl.WORKLOADS["gqa"], T=1)
    for n in ("x", "a", "b"):
        d0[n] = d0[n][:, :0]
    d0["T"] = 0
    o, sf = _fused(gpu, d0)
    assert o.shape[1] == 0 and torch.equal(sf.cpu(), d0["S0"])


def test_prefill_workspace_reuse_and_determinism(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["varlen"], lengths=[300, 7, 90])
    t, cu, _, _ = _dev(d, None)
    ws_bytes = gpu.gdn_prefill_workspace_size(1, d["T"], d["H"], d["Hk"], d["K"], d["V"], 3)
    ws = torch.full((ws_bytes,), 0xAB, dtype=torch.uint8, device=DEV)   # stale contents
    r1 = _fused(gpu, d, workspace=ws)
    r2 = _fused(gpu, d, workspace=ws)
    _equal(r1, r2, "reused workspace")
    _equal(r1, _chain(gpu, d), "vs chain")


def test_prefill_phases_equal_whole(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["gqa"], T=333)
    t, cu, S0, _ = _dev(d, None)
    Hk, K, H, V = d["Hk"], d["K"], d["H"], d["V"]
    ws = torch.empty(gpu.gdn_prefill_workspace_size(1, d["T"], H, Hk, K, V, 0), dtype=torch.uint8,
                     device=DEV)
    gpu.gdn_prefill_prepare(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"], ws, Hk=Hk,
                            K=K, H=H, V=V)
    o, sf = gpu.gdn_prefill_scan(t["x"], t["w"], ws, Hk=Hk, K=K, H=H, V=V, initial_state=S0)
    torch.cuda.synchronize()
    _equal((o, sf), _fused(gpu, d), "phases")


# full workload sizes: bit-equal to the chain (which is checked against the
# oracle at these sizes on sampled heads and sequences), plus a sampled oracle check

def test_prefill_full_equals_chain(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["prefill"])
    got = _fused(gpu, d)
    _equal(got, _chain(gpu, d), "prefill workload")
    # one whole (sequence, head) unit against the oracle
    from tests.test_gpu_chunk import _oracle_chain
    ro, rs, _ = _oracle_chain(d, heads=[5])
    assert_close(to_np(got[0][:, :, [5]]), ro, BF16, "prefill head 5 o")
    assert_close(to_np(got[1][:, [5]]), rs, BF16, "prefill head 5 state")


def test_prefill_gqa_full_equals_chain(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["gqa"])
    _equal(_fused(gpu, d), _chain(gpu, d), "gqa workload")


def test_prefill_varlen_full_equals_chain(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["varlen"])
    _equal(_fused(gpu, d), _chain(gpu, d), "varlen workload")


def test_prefill_concurrent_streams(gpu):
    # calls on separate streams, each with its own workspace and outputs, run
    # concurrently (three streams, several rounds) and give the bits of the
    # same calls made one after another
    cases = [wl.prefill_inputs(wl.WORKLOADS["prefill"], T=700, B=2, seed=41),
             wl.prefill_inputs(wl.WORKLOADS["varlen"], lengths=[5, 300, 64, 129], seed=42)]
    dev = [_dev(d, None) for d in cases]

    def call(d, t):
        tt, cu, S0, _ = t
        return gpu.gdn_prefill(tt["x"], tt["w"], tt["a"], tt["b"], tt["A_log"], tt["dt_bias"],
                               Hk=d["Hk"], K=d["K"], H=d["H"], V=d["V"], initial_state=S0,
                               cu_seqlens=cu)

    ref = [call(d, t) for d, t in zip(cases, dev)]
    dc = wl.chunk_inputs(B=2, T=300, H=4, Hk=2, K=128, V=128, dtype=BF16, s0_std=0.05, seed=43)
    tc = {n: (None if dc[n] is None else dc[n].to(DEV)) for n in ("q", "k", "v", "g", "beta", "S0")}

    def chunk():
        return gpu.gdn_chunk_fwd(tc["q"], tc["k"], tc["v"], tc["g"], tc["beta"], initial_state=tc["S0"])

    ref.append(chunk())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in range(3)]
    for _ in range(4):
        out = [None] * 3
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                out[i] = call(cases[i], dev[i]) if i < 2 else chunk()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(out[i][0], ref[i][0]) and torch.equal(out[i][1], ref[i][1]), f"stream {i}"
