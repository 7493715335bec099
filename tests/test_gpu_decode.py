"""Parity of gdn_recurrent_decode (HIP) with the oracle's Gated DeltaProduct
decode (prepare + M-step recurrence), over several carried steps."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _case(n, M, H, G, P, N, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    state = torch.randn(n, H, N, P, generator=gen) * 0.02
    steps = []
    for s in range(3):
        x = torch.randn(n, xl, generator=gen).to(dtype)
        ba = torch.randn(n, bl, generator=gen).to(dtype)
        steps.append((x, ba))
    return A_log, dt_bias, state, steps


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("M,H,G,P,N", [(1, 4, 2, 64, 64), (2, 4, 2, 128, 128), (3, 6, 3, 64, 128),
                                       (2, 8, 8, 128, 64), (4, 2, 1, 128, 128)])
def test_decode_small(gpu, dtype, M, H, G, P, N):
    n = 5
    A_log, dt_bias, state, steps = _case(n, M, H, G, P, N, dtype, seed=M * 100 + P + N)
    sg = state.to(DEV).contiguous()
    sr = to_np(state)
    for x, ba in steps:
        o = gpu.gdn_recurrent_decode(x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV), sg,
                                     M, H, G, P, N, scale=0.5)
        torch.cuda.synchronize()
        ro, sr = oracle.gdp_decode(to_np(x), to_np(ba), to_np(A_log), to_np(dt_bias), sr,
                                   M, H, G, P, N, scale=0.5)
        assert_close(to_np(o), ro, dtype, "decode o")
        assert_close(to_np(sg), sr, dtype, "decode state")


def test_decode_strided_rows(gpu):
    # x and ba as slices of wider rows (the ba slice of an input projection)
    n, M, H, G, P, N = 7, 2, 4, 2, 128, 128
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    gen = torch.Generator().manual_seed(1)
    xw = torch.randn(n, xl + 64, generator=gen).to(torch.bfloat16)
    baw = torch.randn(n, bl + 40, generator=gen).to(torch.bfloat16)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    state = torch.randn(n, H, N, P, generator=gen) * 0.02
    sg = state.to(DEV)
    xg, bag = xw.to(DEV), baw.to(DEV)
    o = gpu.gdn_recurrent_decode(xg[:, 64:], bag[:, 8:8 + bl], A_log.to(DEV), dt_bias.to(DEV), sg,
                                 M, H, G, P, N)
    torch.cuda.synchronize()
    ro, rs = oracle.gdp_decode(to_np(xw[:, 64:]), to_np(baw[:, 8:8 + bl]), to_np(A_log),
                               to_np(dt_bias), to_np(state), M, H, G, P, N)
    assert_close(to_np(o), ro, torch.bfloat16, "strided o")
    assert_close(to_np(sg), rs, torch.bfloat16, "strided state")


def test_decode_deterministic(gpu):
    n, M, H, G, P, N = 16, 2, 8, 4, 128, 128
    A_log, dt_bias, state, steps = _case(n, M, H, G, P, N, torch.bfloat16, seed=3)
    outs = []
    for _ in range(2):
        sg = state.to(DEV).contiguous()
        os_ = [gpu.gdn_recurrent_decode(x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV),
                                        sg, M, H, G, P, N) for x, ba in steps]
        torch.cuda.synchronize()
        outs.append((torch.stack(os_), sg.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_prefill_state_hands_over_to_decode(gpu):
    # prefill(T) -> final state -> one decode token (M = 1) == prefill(T + 1)'s last output
    T, H, K, V = 130, 4, 128, 128
    d = wl.chunk_inputs(B=1, T=T + 1, H=H, Hk=H, K=K, V=V, dtype=torch.float32, decay="weak",
                        s0_std=0.02, seed=17)
    q, k, v = (d[n].to(DEV) for n in ("q", "k", "v"))
    g, beta = d["g"].to(DEV), d["beta"].to(DEV)
    S0 = d["S0"].to(DEV)
    o_full, _ = gpu.gdn_chunk_fwd(q, k, v, g, beta, initial_state=S0)
    o_pre, s_pre = gpu.gdn_chunk_fwd(q[:, :T], k[:, :T], v[:, :T], g[:, :T].contiguous(),
                                     beta[:, :T].contiguous(), initial_state=S0)
    # decode row for token T with M = 1, G = H groups: v | k | q; ba = b | a chosen so
    # that sigmoid(b) = beta_T and -exp(A_log) softplus(a + dt_bias) = g_T
    bt = d["beta"][0, T].double()
    gt = d["g"][0, T].double()
    b = torch.log(bt / (1 - bt))
    A_log = torch.zeros(H)
    dt_bias = torch.zeros(H)
    a = torch.log(torch.expm1(-gt))                   # softplus(a) = -g
    x = torch.cat([d["v"][0, T].reshape(-1), d["k"][0, T].reshape(-1), d["q"][0, T].reshape(-1)])
    ba = torch.cat([b, a]).float()
    o_dec = gpu.gdn_recurrent_decode(x[None].to(DEV), ba[None].to(DEV), A_log.to(DEV),
                                     dt_bias.to(DEV), s_pre, 1, H, H, V, K)
    torch.cuda.synchronize()
    assert_close(to_np(o_dec[0]), to_np(o_full[0, T]), torch.float32, "handoff")


def test_decode_full_size(gpu):
    """The decode workload at full size (n = 256, M = 2, H = 32, G = 16, P = N = 128,
    1000 steps) in the launch configuration the benchmark times; the oracle follows a
    sample of requests through all steps (requests are independent)."""
    w = wl.WORKLOADS["decode"]
    st = wl.decode_state_inputs(w)
    sample = [0, 1, 77, 128, 200, 255]
    sg = st["state"].to(DEV)
    A_log, dt_bias = st["A_log"].to(DEV), st["dt_bias"].to(DEV)
    sr = to_np(st["state"][sample])
    worst_o = 0.0
    for s in range(w.steps):
        x, ba = wl.decode_step_inputs(w, s)
        o = gpu.gdn_recurrent_decode(x.to(DEV, non_blocking=True), ba.to(DEV, non_blocking=True),
                                     A_log, dt_bias, sg, w.M, w.H, w.G, w.V, w.K)
        ro, sr = oracle.gdp_decode(to_np(x[sample]), to_np(ba[sample]), to_np(st["A_log"]),
                                   to_np(st["dt_bias"]), sr, w.M, w.H, w.G, w.V, w.K)
        if s % 100 == 0 or s == w.steps - 1:
            worst_o = max(worst_o, assert_close(to_np(o[sample]), ro, torch.bfloat16, f"step {s} o"))
    torch.cuda.synchronize()
    assert_close(to_np(sg[sample]), sr, torch.bfloat16, "final state")
    assert torch.isfinite(sg).all()
