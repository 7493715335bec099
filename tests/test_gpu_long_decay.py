"""Whole-tensor parity at the prefill, GQA and packed workloads' full sizes
(every (sequence, head) unit), and long sequences with weak or no decay,
against the fp64 oracle.

The bf16 path rounds the state to a bf16 MFMA operand at every chunk (the
products K h and Q h); the workload gates decay fast, which hides any drift
that rounding could accumulate. Here A_log = -6 (exp(A_log) ~ 0.0025, so
alpha = exp(g) ~ 0.998 per token) and A_log = -inf (g = 0 exactly: no decay,
the state keeps everything it was written) run over 4096 and 16384 tokens, on
the whole-prefill entry and on the per-step chain, for every setting of the
scan schedule knob, each compared with the oracle's conv -> gates -> timestep
recurrence over every (sequence, head) unit. Measured errors go to
$GDN_PARITY_LOG when it is set.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16 = torch.bfloat16

# scan schedules of the bf16 path (GDN_TUNE_SCAN_FORM, GDN_TUNE_SCAN_TILES):
# automatic; column groups of one and two tiles; whole units (two tiles per wave)
SCHEDULES = [(0, 0), (1, 1), (1, 2), (2, 0)]


def _oracle(d):
    B, T, C = d["x"].shape
    Hk, K, H, V = d["Hk"], d["K"], d["H"], d["V"]
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    y = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]), cu_seqlens=cu, silu=True)
    q = y[:, :, :Hk * K].reshape(B, T, Hk, K)
    k = y[:, :, Hk * K:2 * Hk * K].reshape(B, T, Hk, K)
    v = y[:, :, 2 * Hk * K:].reshape(B, T, H, V)
    del y
    g, beta = oracle.gate_prepare(to_np(d["a"]), to_np(d["b"]), to_np(d["A_log"]),
                                  to_np(d["dt_bias"]))
    S0 = None if d["S0"] is None else to_np(d["S0"])
    return oracle.gated_delta_rule(q, k, v, g, beta, S0=S0, cu_seqlens=cu)


def _run(gdn, d, entry):
    t = {n: d[n].to(DEV) for n in ("x", "w", "a", "b", "A_log", "dt_bias")}
    S0 = None if d["S0"] is None else d["S0"].to(DEV)
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(DEV)
    dims = dict(Hk=d["Hk"], K=d["K"], H=d["H"], V=d["V"])
    if entry == "prefill":
        o, sf = gdn.gdn_prefill(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                                initial_state=S0, cu_seqlens=cu, **dims)
    else:
        o, sf = gdn.prefill_chain(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                                  initial_state=S0, cu_seqlens=cu, **dims)
    torch.cuda.synchronize()
    return to_np(o), to_np(sf)


def _check_all(gdn, d, what):
    ro, rs = _oracle(d)
    for sched in SCHEDULES:
        gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, sched[0])
        gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, sched[1])
        try:
            for entry in ("prefill", "chain"):
                o, sf = _run(gdn, d, entry)
                tag = f"{what} {entry} schedule={sched}"
                assert_close(o, ro, BF16, f"{tag} o")
                assert_close(sf, rs, BF16, f"{tag} state")
        finally:
            gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, 0)
            gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, 0)


def test_prefill_full_all_heads(gpu):
    # the benchmarked workload, whole o and final state (all 64 (sequence, head) units)
    d = wl.prefill_inputs(wl.WORKLOADS["prefill"])
    ro, rs = _oracle(d)
    o, sf = _run(gpu, d, "prefill")
    assert_close(o, ro, BF16, "prefill full o")
    assert_close(sf, rs, BF16, "prefill full state")


@pytest.mark.parametrize("name", ["gqa", "varlen"])
def test_prefill_full_all_units(gpu, name):
    # the long GQA and packed workloads, whole o and final state: every
    # (sequence, head) unit against the oracle, on the whole-prefill entry
    # and the per-step chain (the automatic scan schedule)
    d = wl.prefill_inputs(wl.WORKLOADS[name])
    print(f"full-size parity, every unit: {name}", flush=True)
    ro, rs = _oracle(d)
    for entry in ("prefill", "chain"):
        o, sf = _run(gpu, d, entry)
        assert_close(o, ro, BF16, f"{name} full {entry} o")
        assert_close(sf, rs, BF16, f"{name} full {entry} state")


@pytest.mark.parametrize("A_log", [-6.0, float("-inf")], ids=["weak", "none"])
def test_long_weak_decay_prefill_shape(gpu, A_log):
    # the prefill workload's shape (B=4, H=16, T=4096) with alpha ~ 0.998 or exactly 1
    d = wl.prefill_inputs(wl.WORKLOADS["prefill"])
    d["A_log"] = torch.full_like(d["A_log"], A_log)
    _check_all(gpu, d, f"T=4096 A_log={A_log}")


@pytest.mark.parametrize("A_log", [-6.0, float("-inf")], ids=["weak", "none"])
def test_long_weak_decay_16k(gpu, A_log):
    # one sequence of 16384 tokens (256 chunks), GQA heads as the long-prefill workload
    d = wl.prefill_inputs(wl.WORKLOADS["gqa"], T=16384)
    d["A_log"] = torch.full_like(d["A_log"], A_log)
    _check_all(gpu, d, f"T=16384 A_log={A_log}")

