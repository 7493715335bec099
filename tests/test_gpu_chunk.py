"""Parity of gdn_chunk_fwd (HIP) with the fp64 oracle's timestep recurrence.

Stage tests draw q, k, v, g, beta directly (workloads.chunk_inputs) and feed
the same host tensors to both sides. Chain tests run conv1d -> gates -> chunk
on the GPU and the oracle's own conv -> gates -> recurrence from the same raw
inputs (x, w, a, b, A_log, dt_bias), at the workloads' full sizes; where the
oracle would take minutes it checks whole sampled (sequence, head) units,
which is exact because units are independent.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import TOL, assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _gpu_chunk(gdn, d, scale=1.0, l2norm=True, final=True):
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    g, beta = d["g"].to(DEV), d["beta"].to(DEV)
    S0 = None if d["S0"] is None else d["S0"].to(DEV)
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(DEV)
    o, sf = gdn.gdn_chunk_fwd(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu, scale=scale,
                              qk_l2norm=l2norm, output_final_state=final)
    torch.cuda.synchronize()
    return o, sf


def _oracle_chunk(d, scale=1.0, l2norm=True):
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    return oracle.gated_delta_rule(to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["g"]),
                                   to_np(d["beta"]), S0=None if d["S0"] is None else to_np(d["S0"]),
                                   cu_seqlens=cu, scale=scale, l2norm=l2norm)


def _check(gdn, d, scale=1.0, l2norm=True, what=""):
    o, sf = _gpu_chunk(gdn, d, scale, l2norm)
    ro, rs = _oracle_chunk(d, scale, l2norm)
    eo = assert_close(to_np(o), ro, d["dtype"], f"{what} o")
    es = assert_close(to_np(sf), rs, d["dtype"], f"{what} final state")
    return eo, es


# ---------------------------------------------------------------- stage tests

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_chunk_lengths(gpu, dtype, T):
    d = wl.chunk_inputs(B=2, T=T, H=2, Hk=2, K=64, V=64, dtype=dtype, decay="weak", s0_std=0.1,
                        seed=T)
    _check(gpu, d, what=f"T={T}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K,V", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_chunk_head_dims(gpu, dtype, K, V):
    # K != V pins the state orientation (K x V) at the boundary
    d = wl.chunk_inputs(B=1, T=150, H=3, Hk=3, K=K, V=V, dtype=dtype, decay="weak", s0_std=0.05,
                        seed=K + V)
    _check(gpu, d, what=f"K={K} V={V}")


@pytest.mark.parametrize("decay", ["strong", "weak", "none"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_decay_regimes(gpu, decay, dtype):
    d = wl.chunk_inputs(B=2, T=320, H=4, Hk=4, K=128, V=128, dtype=dtype, decay=decay,
                        s0_std=0.02, seed=3)
    _check(gpu, d, what=decay)


def test_chunk_gqa_and_scale(gpu):
    d = wl.chunk_inputs(B=2, T=190, H=8, Hk=2, K=128, V=128, dtype=torch.bfloat16, decay="weak",
                        s0_std=0.02, seed=11)
    _check(gpu, d, scale=128 ** -0.5, what="gqa")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_without_l2norm(gpu, dtype):
    d = wl.chunk_inputs(B=1, T=100, H=2, Hk=2, K=64, V=64, dtype=dtype, decay="strong", seed=4)
    # pre-normalised keys (the recurrence is only stable for |k| <= ~1)
    for n in ("q", "k"):
        t = d[n].float()
        d[n] = (t / t.norm(dim=-1, keepdim=True)).to(dtype)
    _check(gpu, d, l2norm=False, what="no l2norm")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_varlen(gpu, dtype):
    lengths = [1, 64, 65, 3, 200, 127, 1, 128]
    d = wl.chunk_inputs(B=1, T=sum(lengths), H=4, Hk=2, K=128, V=64, dtype=dtype, decay="weak",
                        s0_std=0.05, lengths=lengths, seed=21)
    _check(gpu, d, what="varlen")


def test_chunk_empty_sequence_and_empty_batch(gpu):
    # zero-length packed sequences pass their initial state through
    lengths = [0, 5, 0, 70, 0]
    d = wl.chunk_inputs(B=1, T=75, H=2, Hk=2, K=64, V=64, dtype=torch.bfloat16, decay="weak",
                        s0_std=0.1, lengths=lengths, seed=8)
    _check(gpu, d, what="empty seqs")
    o, sf = _gpu_chunk(gpu, d)
    np.testing.assert_array_equal(to_np(sf[0]), to_np(d["S0"][0]))
    # T = 0 (dense): o is empty, final state = initial state
    d0 = wl.chunk_inputs(B=2, T=0, H=2, Hk=2, K=64, V=64, dtype=torch.bfloat16, s0_std=0.1, seed=9)
    o, sf = _gpu_chunk(gpu, d0)
    assert o.numel() == 0
    np.testing.assert_array_equal(to_np(sf), to_np(d0["S0"]))


def test_chunk_no_final_state_and_zero_state(gpu):
    d = wl.chunk_inputs(B=1, T=70, H=2, Hk=2, K=64, V=64, dtype=torch.float32, decay="weak", seed=5)
    o, sf = _gpu_chunk(gpu, d, final=False)
    assert sf is None
    ro, _ = _oracle_chunk(d)
    assert_close(to_np(o), ro, torch.float32, "no final state")


# ------------------------------------------------------------- invariants

def test_chunk_deterministic(gpu):
    d = wl.chunk_inputs(B=2, T=300, H=4, Hk=2, K=128, V=128, dtype=torch.bfloat16, s0_std=0.02,
                        seed=6)
    o1, s1 = _gpu_chunk(gpu, d)
    o2, s2 = _gpu_chunk(gpu, d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_chunk_packing_invariance(gpu):
    # a packed batch equals per-sequence dense calls, bit for bit
    lengths = [70, 1, 128, 33]
    d = wl.chunk_inputs(B=1, T=sum(lengths), H=2, Hk=2, K=128, V=128, dtype=torch.bfloat16,
                        decay="weak", s0_std=0.05, lengths=lengths, seed=12)
    o, sf = _gpu_chunk(gpu, d)
    cu = d["cu_seqlens"].tolist()
    for i in range(len(lengths)):
        s, e = cu[i], cu[i + 1]
        di = dict(d, q=d["q"][:, s:e], k=d["k"][:, s:e], v=d["v"][:, s:e], g=d["g"][:, s:e].contiguous(),
                  beta=d["beta"][:, s:e].contiguous(), S0=d["S0"][i:i + 1], cu_seqlens=None,
                  T=e - s)
        oi, si = _gpu_chunk(gpu, di)
        assert torch.equal(o[:, s:e], oi), i
        assert torch.equal(sf[i:i + 1], si), i


def test_chunk_gqa_invariance(gpu):
    # Hk < H equals the same call with q/k heads explicitly repeated, bit for bit
    d = wl.chunk_inputs(B=1, T=130, H=4, Hk=2, K=128, V=128, dtype=torch.bfloat16, s0_std=0.02,
                        seed=13)
    o, sf = _gpu_chunk(gpu, d)
    dr = dict(d, q=d["q"].repeat_interleave(2, dim=2).contiguous(),
              k=d["k"].repeat_interleave(2, dim=2).contiguous(), Hk=4)
    o2, sf2 = _gpu_chunk(gpu, dr)
    assert torch.equal(o, o2) and torch.equal(sf, sf2)


# --------------------------------------------------------------- chain tests

def _gpu_chain(gdn, d):
    dev = DEV
    S0 = None if d["S0"] is None else d["S0"].to(dev)
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(dev)
    o, sf = gdn.prefill_chain(d["x"].to(dev), d["w"].to(dev), d["a"].to(dev), d["b"].to(dev),
                              d["A_log"].to(dev), d["dt_bias"].to(dev), Hk=d["Hk"], K=d["K"],
                              H=d["H"], V=d["V"], initial_state=S0, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o, sf


def _oracle_chain(d, heads=None, seqs=None):
    """The oracle chain on sampled value heads (pairs sharing q/k heads) and
    sampled packed sequences; returns (o [.., len(heads), V], S_final)."""
    B, T, C = d["x"].shape
    H, Hk, K, V = d["H"], d["Hk"], d["K"], d["V"]
    per = H // Hk
    heads = list(range(H)) if heads is None else list(heads)
    hks = sorted({h // per for h in heads})
    assert all(h // per in hks for h in heads)
    # channels the sampled heads need: q | k of their q/k heads, v of the value heads
    qch = np.concatenate([np.arange(hk * K, (hk + 1) * K) for hk in hks])
    kch = qch + Hk * K
    vch = np.concatenate([np.arange(2 * Hk * K + h * V, 2 * Hk * K + (h + 1) * V) for h in heads])
    cu = d["cu_seqlens"]
    x = d["x"]
    if seqs is not None:
        cuv = cu.tolist()
        parts = [x[:, cuv[i]:cuv[i + 1]] for i in seqs]
        x = torch.cat(parts, dim=1)
        lens = [cuv[i + 1] - cuv[i] for i in seqs]
        cu_s = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        tok = np.concatenate([np.arange(cuv[i], cuv[i + 1]) for i in seqs])
    else:
        cu_s = None if cu is None else cu.numpy()
        tok = None
    ch = np.concatenate([qch, kch, vch])
    wsel = to_np(d["w"][ch])
    y = oracle.conv1d_causal(to_np(x[:, :, ch]), wsel, cu_seqlens=cu_s, silu=True)
    nq = len(hks) * K
    Tn = y.shape[1]
    q = y[:, :, :nq].reshape(B, Tn, len(hks), K)
    k = y[:, :, nq:2 * nq].reshape(B, Tn, len(hks), K)
    v = y[:, :, 2 * nq:].reshape(B, Tn, len(heads), V)
    a = to_np(d["a"])[:, :, heads]
    b = to_np(d["b"])[:, :, heads]
    if tok is not None:
        a, b = a[:, tok], b[:, tok]
    g, beta = oracle.gate_prepare(a, b, to_np(d["A_log"])[heads], to_np(d["dt_bias"])[heads])
    S0 = None
    if d["S0"] is not None:
        S0 = to_np(d["S0"])[:, heads]
        if seqs is not None:
            S0 = S0[list(seqs)]
    o, sf = oracle.gated_delta_rule(q, k, v, g, beta, S0=S0, cu_seqlens=cu_s)
    return o, sf, tok


def test_chain_tiny_workload(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["tiny"])
    o, sf = _gpu_chain(gpu, d)
    ro, rs, _ = _oracle_chain(d)
    assert_close(to_np(o), ro, torch.float32, "tiny o")
    assert_close(to_np(sf), rs, torch.float32, "tiny state")


def test_chain_prefill_small(gpu):
    # the prefill workload's distributions at a length the oracle runs in seconds
    d = wl.prefill_inputs(wl.WORKLOADS["prefill"], T=321, B=2)
    o, sf = _gpu_chain(gpu, d)
    ro, rs, _ = _oracle_chain(d)
    assert_close(to_np(o), ro, torch.bfloat16, "prefill-small o")
    assert_close(to_np(sf), rs, torch.bfloat16, "prefill-small state")


def test_chain_prefill_full(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["prefill"])
    o, sf = _gpu_chain(gpu, d)
    heads = [0, 1, 7, 15]
    ro, rs, _ = _oracle_chain(d, heads=heads)
    assert_close(to_np(o[:, :, heads]), ro, torch.bfloat16, "prefill o")
    assert_close(to_np(sf[:, heads]), rs, torch.bfloat16, "prefill state")


def test_chain_gqa_full(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["gqa"])
    o, sf = _gpu_chain(gpu, d)
    heads = [0, 1, 30, 31]            # q/k heads 0 and 15, two value heads each
    ro, rs, _ = _oracle_chain(d, heads=heads)
    assert_close(to_np(o[:, :, heads]), ro, torch.bfloat16, "gqa o")
    assert_close(to_np(sf[:, heads]), rs, torch.bfloat16, "gqa state")


def test_chain_varlen_full(gpu):
    d = wl.prefill_inputs(wl.WORKLOADS["varlen"])
    o, sf = _gpu_chain(gpu, d)
    lens = (d["cu_seqlens"][1:] - d["cu_seqlens"][:-1]).tolist()
    order = np.argsort(lens)
    seqs = sorted(set(order[:3].tolist() + order[-3:].tolist() + [0, 31, 63]))
    ro, rs, tok = _oracle_chain(d, seqs=seqs)
    assert_close(to_np(o[:, tok]), ro, torch.bfloat16, "varlen o")
    assert_close(to_np(sf[seqs]), rs, torch.bfloat16, "varlen state")


def test_chain_weak_decay_carry(gpu):
    # the workload gates decay fast; with weak decay the inter-chunk carry and S0 matter
    d = wl.prefill_inputs(wl.WORKLOADS["gqa"], T=700)
    d["A_log"] = torch.full_like(d["A_log"], -6.0)    # exp(A_log) ~ 0.0025: alpha ~ 0.998
    o, sf = _gpu_chain(gpu, d)
    ro, rs, _ = _oracle_chain(d)
    assert_close(to_np(o), ro, torch.bfloat16, "weak-decay o")
    assert_close(to_np(sf), rs, torch.bfloat16, "weak-decay state")
