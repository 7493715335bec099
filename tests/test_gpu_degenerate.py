"""Degenerate cases of the gated delta rule on the GPU path (gdn_chunk_fwd),
on every scan schedule of each dtype.

Closed forms, independent of the oracle:
* beta = 0 and g = 0: nothing is written and nothing decays, so the final
  state is the initial state bit for bit and o_t = scale * q_t^T S0 (q_t
  L2-normalised);
* beta = 0, g < 0: pure decay, o_t = scale * exp(G_t) q_t^T S0 and the final
  state exp(G_T) S0, G_t the cumulative log-decay of the sequence.
Against the oracle: zero key and query rows (their normalised vectors are
zero: the token only decays the state and reads nothing), one key repeated
over whole chunks with beta = 1 (each token overwrites what the last wrote),
and decay strong enough that exp of the in-chunk cumulative sum underflows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16, FP32 = torch.bfloat16, torch.float32
# (GDN_TUNE_SCAN_FORM, GDN_TUNE_SCAN_TILES)
SCHEDULES = {BF16: [(0, 0), (1, 1), (1, 2), (2, 0), (2, 1)], FP32: [(0, 0), (0, 1), (0, 4)]}


def _runs(gdn, d, **kw):
    """gdn_chunk_fwd on every schedule of d's dtype: [(schedule, o, final state)]."""
    t = {n: (None if d[n] is None else d[n].to(DEV)) for n in ("q", "k", "v", "g", "beta", "S0", "cu_seqlens")}
    out = []
    for f, tiles in SCHEDULES[d["dtype"]]:
        gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, f)
        gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, tiles)
        try:
            o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["S0"],
                                      cu_seqlens=t["cu_seqlens"], **kw)
            torch.cuda.synchronize()
        finally:
            gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, 0)
            gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, 0)
        out.append(((f, tiles), o, sf))
    return out


def _unit_q(d):
    q = to_np(d["q"])
    return q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)


def _seq_of_token(d):
    B, T = d["q"].shape[:2]
    if d["cu_seqlens"] is None:
        return np.repeat(np.arange(B), T).reshape(B, T)
    cu = d["cu_seqlens"].numpy()
    return np.searchsorted(cu, np.arange(T), side="right")[None] - 1


def _closed_form(d, scale):
    """o and final state of beta = 0: o_t = scale exp(G_t) q_t^T S0[seq(t)]."""
    qn = _unit_q(d)                                     # [B, T, Hk, K]
    S0 = to_np(d["S0"])                                 # [N, H, K, V]
    g = to_np(d["g"])                                   # [B, T, H]
    B, T, Hk, K = qn.shape
    H, V = S0.shape[1], S0.shape[3]
    per = H // Hk
    seq = _seq_of_token(d)
    o = np.zeros((B, T, H, V))
    G = np.zeros((B, T, H))
    for b in range(B):
        run = np.zeros(H)
        for t in range(T):
            if t > 0 and seq[b, t] != seq[b, t - 1]:
                run = np.zeros(H)
            run = run + g[b, t]
            G[b, t] = run
    for h in range(H):
        for b in range(B):
            s = seq[b]
            o[b, :, h] = scale * np.exp(G[b, :, h])[:, None] * np.einsum(
                "tk,tkv->tv", qn[b, :, h // per], S0[s, h])
    sf = S0.copy()
    for n in range(S0.shape[0]):
        if d["cu_seqlens"] is None:
            if T:
                sf[n] *= np.exp(G[n, -1])[:, None, None]
        else:
            cu = d["cu_seqlens"].numpy()
            if cu[n + 1] > cu[n]:
                sf[n] *= np.exp(G[0, cu[n + 1] - 1])[:, None, None]
    return o, sf


@pytest.mark.parametrize("dtype", [BF16, FP32])
def test_no_write_no_decay_keeps_the_state(gpu, dtype):
    # beta = 0, g = 0: the final state is S0 bit for bit, o = scale q^T S0
    d = wl.chunk_inputs(B=2, T=200, H=4, Hk=2, K=128, V=128, dtype=dtype, s0_std=0.1, seed=21)
    d["g"] = torch.zeros_like(d["g"])
    d["beta"] = torch.zeros_like(d["beta"])
    ro, _ = _closed_form(d, 0.5)
    for sched, o, sf in _runs(gpu, d, scale=0.5):
        assert torch.equal(sf.cpu(), d["S0"]), f"{sched}: the state changed"
        assert_close(to_np(o), ro, dtype, f"frozen state {sched} o")


@pytest.mark.parametrize("dtype", [BF16, FP32])
def test_pure_decay(gpu, dtype):
    # beta = 0, g < 0 (packed, with an empty sequence): the state only decays
    lengths = [70, 0, 129, 64, 1]
    d = wl.chunk_inputs(B=1, T=sum(lengths), H=2, Hk=2, K=64, V=128, dtype=dtype, decay="weak",
                        s0_std=0.1, lengths=lengths, seed=22)
    d["g"] = -torch.rand(d["g"].shape, generator=torch.Generator().manual_seed(3)) * 0.2
    d["beta"] = torch.zeros_like(d["beta"])
    ro, rs = _closed_form(d, 1.0)
    for sched, o, sf in _runs(gpu, d):
        assert_close(to_np(o), ro, dtype, f"pure decay {sched} o")
        assert_close(to_np(sf), rs, dtype, f"pure decay {sched} state")


def _oracle(d, **kw):
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    return oracle.gated_delta_rule(to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["g"]),
                                   to_np(d["beta"]), S0=None if d["S0"] is None else to_np(d["S0"]),
                                   cu_seqlens=cu, **kw)


def _against_oracle(gpu, d, what):
    ro, rs = _oracle(d)
    for sched, o, sf in _runs(gpu, d):
        assert_close(to_np(o), ro, d["dtype"], f"{what} {sched} o")
        assert_close(to_np(sf), rs, d["dtype"], f"{what} {sched} state")


@pytest.mark.parametrize("dtype", [BF16, FP32])
def test_zero_keys_and_queries(gpu, dtype):
    d = wl.chunk_inputs(B=2, T=150, H=2, Hk=2, K=128, V=64, dtype=dtype, decay="weak", s0_std=0.05,
                        seed=23)
    d["k"][:, ::7] = 0
    d["k"][:, 64:128] = 0          # a whole chunk of zero keys
    d["q"][:, 3::11] = 0
    _against_oracle(gpu, d, "zero keys / queries")


@pytest.mark.parametrize("dtype", [BF16, FP32])
def test_repeated_key_overwrites(gpu, dtype):
    # one key per chunk for every token, beta = 1: each token replaces the
    # value stored under that key (the triangular solve at its most coupled)
    d = wl.chunk_inputs(B=1, T=200, H=2, Hk=2, K=64, V=64, dtype=dtype, decay="none", seed=24)
    k = d["k"].clone()
    for c0 in range(0, 200, 64):
        k[:, c0:c0 + 64] = k[:, c0:c0 + 1]
    d["k"] = k
    d["beta"] = torch.ones_like(d["beta"])
    _against_oracle(gpu, d, "repeated key")


@pytest.mark.parametrize("dtype", [BF16, FP32])
def test_decay_underflow(gpu, dtype):
    # g ~ -U[0, 60]: exp of the in-chunk cumulative sum underflows to zero;
    # every output is the token's own write plus vanishing history
    d = wl.chunk_inputs(B=2, T=130, H=2, Hk=1, K=128, V=128, dtype=dtype, decay="none", s0_std=0.1,
                        seed=25)
    d["g"] = -60 * torch.rand(d["g"].shape, generator=torch.Generator().manual_seed(4))
    _against_oracle(gpu, d, "decay underflow")


def test_prefill_frozen_gates_keep_the_state(gpu):
    # whole prefill with b = -inf (beta = sigmoid(b) = 0) and A_log = -inf (g = 0):
    # the final state is S0 bit for bit and o = scale q^T S0 with q the
    # convolved, normalised query rows, in both scan workgroup forms
    w = wl.Workload("frozen", 3, BF16, H=4, Hk=2, K=128, V=128, s0_std=0.1)
    d = wl.prefill_inputs(w, T=200, B=2)
    d["b"] = torch.full_like(d["b"], float("-inf"))
    d["A_log"] = torch.full_like(d["A_log"], float("-inf"))
    y = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]), silu=True)
    q = y[:, :, :w.Hk * w.K].reshape(2, 200, w.Hk, w.K)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    S0 = to_np(d["S0"])
    ro = np.einsum("bthk,bhkv->bthv", np.repeat(qn, w.H // w.Hk, axis=2), S0) * 0.25
    t = {n: d[n].to(DEV) for n in ("x", "w", "a", "b", "A_log", "dt_bias", "S0")}
    for f in (1, 2):
        gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, f)
        try:
            o, sf = gpu.gdn_prefill(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                                    Hk=w.Hk, K=w.K, H=w.H, V=w.V, initial_state=t["S0"], scale=0.25)
            torch.cuda.synchronize()
        finally:
            gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, 0)
        assert torch.equal(sf.cpu(), d["S0"]), f"form {f}: the state changed"
        assert_close(to_np(o), ro, BF16, f"frozen gates, form {f} o")
