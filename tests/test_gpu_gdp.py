"""GPU parity of the Gated DeltaProduct steps around the recurrent core:
gdn_decode_prepare (the five-tensor export), gdn_conv1d_update (the decode
short-conv update with -1 padding slots) and gdn_gdp_prefill_prepare (a GDP
prefill through the chunked forward), against the oracle and against the
library's own prefill conv / decode where the arithmetic is the same."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _gates(H, gen):
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    return A_log, dt_bias


# ------------------------------------------------------------ decode prepare

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("n,M,H,G,P,N", [(3, 3, 4, 2, 64, 128), (256, 2, 32, 16, 128, 128),
                                         (5, 1, 8, 8, 128, 64)])
def test_decode_prepare_layout_and_gates(gpu, dtype, n, M, H, G, P, N):
    gen = torch.Generator().manual_seed(n + M + P)
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    x = torch.randn(n, xl + 16, generator=gen).to(dtype)[:, 8:8 + xl]   # strided rows
    ba = torch.randn(n, bl + 3, generator=gen).to(dtype)[:, :bl]
    A_log, dt_bias = _gates(H, gen)
    q, k, v, beta, g = gpu.gdn_decode_prepare(x.to(DEV), ba.to(DEV), A_log.to(DEV),
                                              dt_bias.to(DEV), M, H, G, P, N)
    torch.cuda.synchronize()
    rq, rk, rv, rb, rg = oracle.gdp_decode_prepare(to_np(x), to_np(ba), to_np(A_log),
                                                   to_np(dt_bias), M, H, G, P, N)
    # plain copies: bit-identical
    np.testing.assert_array_equal(to_np(q), rq)
    np.testing.assert_array_equal(to_np(k), rk)
    np.testing.assert_array_equal(to_np(v), rv)
    # fp32 gates: within fp32 transcendental accuracy of the fp64 definition
    np.testing.assert_allclose(to_np(beta), rb, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(to_np(g), rg, rtol=2e-6, atol=1e-7)
    assert (to_np(g)[:, 1:] == 0).all()
    # the same formulas as the gate kernel: bit-identical
    gg, bg = gpu.gdn_gate_prepare(ba[:, M * H:].to(DEV), ba[:, :H].to(DEV), A_log.to(DEV),
                                  dt_bias.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(g[:, 0].cpu(), gg.cpu())
    assert torch.equal(beta[:, 0].cpu(), bg.cpu())


# ------------------------------------------------------- decode conv update

@pytest.mark.parametrize("dtype,C", [(torch.float32, 384), (torch.bfloat16, 14336)])
def test_conv_update_token_by_token_equals_prefill_conv(gpu, dtype, C):
    # One sequence fed a token at a time from a zero slot: bit-identical to the
    # prefill conv kernel (same arithmetic), and close to the oracle.
    T, S = 11, 4
    gen = torch.Generator().manual_seed(C)
    x = torch.randn(1, T, C, generator=gen).to(dtype).to(DEV)
    w = (torch.randn(C, 4, generator=gen) * 0.5).to(dtype).to(DEV)
    bias = (torch.randn(C, generator=gen) * 0.1).to(dtype).to(DEV)
    yref = gpu.gdn_conv1d_causal(x, w, bias=bias, silu=True)
    st = torch.zeros(S, 3, C, dtype=dtype, device=DEV)
    slot = torch.tensor([2], dtype=torch.int32, device=DEV)
    rst = np.zeros((S, 3, C))
    for t in range(T):
        y = gpu.gdn_conv1d_update(x[0, t:t + 1], st, slot, w, bias=bias, silu=True)
        torch.cuda.synchronize()
        assert torch.equal(y[0], yref[0, t]), f"token {t}"
        ry, rst = oracle.conv1d_update(to_np(x[0, t:t + 1]), rst, [2], to_np(w), bias=to_np(bias))
        assert_close(to_np(y), ry, dtype, "conv update")
    assert torch.equal(st[2], x[0, T - 3:])             # the window holds the last three inputs
    assert (st[[0, 1, 3]] == 0).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv_update_padding_slots(gpu, dtype):
    n, S, C = 6, 8, 512
    gen = torch.Generator().manual_seed(5)
    x = torch.randn(n, C, generator=gen).to(dtype)
    w = (torch.randn(C, 4, generator=gen) * 0.5).to(dtype)
    st0 = torch.randn(S, 3, C, generator=gen).to(dtype)
    slots = torch.tensor([3, -1, 0, 7, 9, 5], dtype=torch.int32)   # -1 padding, 9 outside the pool
    st = st0.to(DEV).clone()
    y = gpu.gdn_conv1d_update(x.to(DEV), st, slots.to(DEV), w.to(DEV), silu=True)
    torch.cuda.synchronize()
    ry, rst = oracle.conv1d_update(to_np(x), to_np(st0), slots.numpy(), to_np(w))
    assert (y[1] == 0).all() and (y[4] == 0).all()
    assert_close(to_np(y), ry, dtype, "conv update")
    live = [0, 2, 3, 5]
    assert_close(to_np(y)[live], ry[live], dtype, "conv update live rows")
    np.testing.assert_array_equal(to_np(st), rst)        # window moves are plain copies
    for s in (1, 2, 4, 6):                               # slots no request names
        assert torch.equal(st[s].cpu(), st0[s])


# ---------------------------------------------------- GDP prefill (interleave)

def _gdp_case(B, T, M, H, G, P, N, dtype, seed, s0=True):
    gen = torch.Generator().manual_seed(seed)
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    x = torch.randn(B, T, xl, generator=gen).to(dtype)
    ba = torch.randn(B, T, bl, generator=gen).to(dtype)
    A_log, dt_bias = _gates(H, gen)
    S0 = torch.randn(B, H, N, P, generator=gen) * 0.02 if s0 else None
    return x, ba, A_log, dt_bias, S0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,M,H,G,P,N", [(2, 100, 2, 4, 2, 64, 64), (1, 70, 3, 4, 4, 128, 128),
                                           (2, 33, 1, 2, 1, 64, 128)])
def test_gdp_prefill_matches_oracle(gpu, dtype, B, T, M, H, G, P, N):
    x, ba, A_log, dt_bias, S0 = _gdp_case(B, T, M, H, G, P, N, dtype, seed=T + M)
    o, sf = gpu.gdp_prefill(x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV), M, H, G, P, N,
                            initial_state=S0.to(DEV), scale=0.5)
    torch.cuda.synchronize()
    ro, rsf = oracle.gdp_prefill(to_np(x), to_np(ba), to_np(A_log), to_np(dt_bias), M, H, G, P, N,
                                 S0=to_np(S0), scale=0.5)
    assert_close(to_np(o), ro, dtype, "gdp prefill o")
    assert_close(to_np(sf), rsf, dtype, "gdp prefill state")


def test_gdp_prefill_prepare_layout(gpu):
    B, T, M, H, G, P, N = 2, 5, 3, 4, 2, 64, 128
    x, ba, A_log, dt_bias, _ = _gdp_case(B, T, M, H, G, P, N, torch.bfloat16, seed=9, s0=False)
    q, k, v, g, beta, cu = gpu.gdn_gdp_prefill_prepare(x.to(DEV), ba.to(DEV), A_log.to(DEV),
                                                       dt_bias.to(DEV), M, H, G, P, N)
    torch.cuda.synchronize()
    assert cu is None
    # each token row against the decode preparation of the same row (bit-identical copies and gates)
    for b in range(B):
        dq, dk, dv, dbeta, dg = gpu.gdn_decode_prepare(x[b].to(DEV), ba[b].to(DEV), A_log.to(DEV),
                                                       dt_bias.to(DEV), M, H, G, P, N)
        torch.cuda.synchronize()
        per = H // G
        for t in range(T):
            for m in range(M):
                p = t * M + m
                assert torch.equal(v[b, p], dv[t, m])
                assert torch.equal(k[b, p], dk[t, m, ::per])     # one key per group
                assert torch.equal(q[b, p], dq[t, m, ::per])
                assert torch.equal(g[b, p], dg[t, m])
                assert torch.equal(beta[b, p], dbeta[t, m])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gdp_prefill_packed(gpu, dtype):
    M, H, G, P, N = 2, 4, 2, 64, 64
    lens = [37, 1, 90]
    T = sum(lens)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    x, ba, A_log, dt_bias, _ = _gdp_case(1, T, M, H, G, P, N, dtype, seed=4, s0=False)
    o, sf = gpu.gdp_prefill(x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV), M, H, G, P, N,
                            cu_seqlens=cu.to(DEV))
    torch.cuda.synchronize()
    ro, rsf = oracle.gdp_prefill(to_np(x), to_np(ba), to_np(A_log), to_np(dt_bias), M, H, G, P, N,
                                 cu_seqlens=cu.numpy())
    assert_close(to_np(o), ro, dtype, "gdp prefill packed o")
    assert_close(to_np(sf), rsf, dtype, "gdp prefill packed state")


def test_gdp_prefill_hands_over_to_decode(gpu):
    # prefill(T) -> final state -> one decode token == prefill(T + 1)'s last output
    B, T, M, H, G, P, N = 2, 64, 2, 4, 2, 128, 128
    x, ba, A_log, dt_bias, S0 = _gdp_case(B, T + 1, M, H, G, P, N, torch.float32, seed=77)
    xg, bag, Ag, dg, Sg = x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV), S0.to(DEV)
    o_full, _ = gpu.gdp_prefill(xg, bag, Ag, dg, M, H, G, P, N, initial_state=Sg)
    _, st = gpu.gdp_prefill(xg[:, :T].contiguous(), bag[:, :T].contiguous(), Ag, dg, M, H, G, P, N,
                            initial_state=Sg)
    st = st.contiguous()
    od = gpu.gdn_recurrent_decode(xg[:, T].contiguous(), bag[:, T].contiguous(), Ag, dg, st,
                                  M, H, G, P, N)
    torch.cuda.synchronize()
    assert_close(to_np(od), to_np(o_full[:, T]), torch.float32, "gdp handover")
