"""gdn_chunk_fwd and gdn_recurrent_decode on seeded random shapes against the
fp64 oracle, within the dtype's bar.

Chunked forward: fp32 and bf16, head dims K and V in {64, 128}, 1 to 4 key
heads with 1, 2 or 4 value heads each, dense batches (1 to 3 rows, lengths on
or next to a chunk boundary or drawn up to 300) or up to six packed sequences
of 0 to 200 tokens, with or without an initial state, each decay regime,
scale 1 or 1/sqrt(K), with or without the L2 norm of q and k (without it,
q and k are normalised beforehand: the recurrence needs |k| <= ~1); the bf16
cases also run every scan schedule (forms and tiles) and must give the same
bits.
Decode: 1 to 9 requests, M = 1 to 4 Householder copies, G groups of 1, 2 or 4
value heads, P and N in {64, 128}, three steps on one state.
Conv1d: integer inputs (exact in both dtypes, so compared bit for bit), 1 to
3 rows of up to 300 tokens or up to eight packed sequences, 8 to 1024
channels, under a random launch configuration (tokens per thread, threads).
Gated DeltaProduct prefill: 1 or 2 rows of up to 150 tokens, M = 1 to 3,
with or without an initial state.
Shapes come from random.Random(seed); values from the workloads' generators."""
import math
import random

import pytest
import torch

import numpy as np

import oracle
import workloads as wl
from tests.helpers import assert_close, bf16_round, to_np
from tests.test_gpu_chunk import _gpu_chunk, _oracle_chunk

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _chunk_case(i):
    r = random.Random(4096 + i)
    dtype = torch.float32 if i % 2 == 0 else torch.bfloat16
    K, V = r.choice([64, 128]), r.choice([64, 128])
    Hk = r.randint(1, 4)
    H = Hk * r.choice([1, 2, 4])
    kw = dict(H=H, Hk=Hk, K=K, V=V, dtype=dtype, decay=r.choice(list(wl.DECAY_GMAX)),
              s0_std=0.02 if r.random() < 0.5 else 0.0, seed=500 + i)
    if r.random() < 0.5:
        lengths = [r.choice([0, 1, 2, 63, 64, 65, 128, 129, r.randint(1, 200)])
                   for _ in range(r.randint(1, 6))]
        if sum(lengths) == 0:
            lengths[-1] = 7
        d = wl.chunk_inputs(B=1, T=sum(lengths), lengths=lengths, **kw)
    else:
        d = wl.chunk_inputs(B=r.randint(1, 3), T=r.choice([1, 63, 64, 65, 127, 130, r.randint(1, 300)]),
                            **kw)
    scale = 1.0 if r.random() < 0.5 else 1.0 / math.sqrt(K)
    l2norm = r.random() < 0.8
    if not l2norm:
        # pre-normalised q and k: the recurrence is only stable for |k| <= ~1
        for n in ("q", "k"):
            t = d[n].float()
            d[n] = (t / t.norm(dim=-1, keepdim=True)).to(dtype)
    return d, scale, l2norm


@pytest.mark.parametrize("i", range(12))
def test_random_shape_chunk_fwd(gpu, i):
    d, scale, l2norm = _chunk_case(i)
    o, sf = _gpu_chunk(gpu, d, scale, l2norm)
    ro, rs = _oracle_chunk(d, scale, l2norm)
    assert_close(to_np(o), ro, d["dtype"], f"case {i} o")
    assert_close(to_np(sf), rs, d["dtype"], f"case {i} final state")
    if d["dtype"] == torch.bfloat16:
        # the other bf16 scan schedules give the same bits
        try:
            for form, tiles in ((1, 1), (1, 2), (2, 0), (2, 1)):
                gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, form)
                gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_TILES, tiles)
                o2, sf2 = _gpu_chunk(gpu, d, scale, l2norm)
                assert torch.equal(o2, o) and torch.equal(sf2, sf), (i, form, tiles)
        finally:
            gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, 0)
            gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_TILES, 0)


@pytest.mark.parametrize("i", range(48))
def test_random_shape_decode(gpu, i):
    r = random.Random(8192 + i)
    dtype = torch.float32 if i % 2 == 0 else torch.bfloat16
    n, M = r.randint(1, 9), r.randint(1, 4)
    G = r.randint(1, 4)
    H = G * r.choice([1, 2, 4])
    P, N = r.choice([64, 128]), r.choice([64, 128])
    scale = r.choice([1.0, 0.5])
    gen = torch.Generator().manual_seed(900 + i)
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    state = torch.randn(n, H, N, P, generator=gen) * 0.02
    sg, sr = state.to(DEV).contiguous(), to_np(state)
    for step in range(3):
        x = torch.randn(n, xl, generator=gen).to(dtype)
        ba = torch.randn(n, bl, generator=gen).to(dtype)
        o = gpu.gdn_recurrent_decode(x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV), sg,
                                     M, H, G, P, N, scale=scale)
        torch.cuda.synchronize()
        ro, sr = oracle.gdp_decode(to_np(x), to_np(ba), to_np(A_log), to_np(dt_bias), sr,
                                   M, H, G, P, N, scale=scale)
        assert_close(to_np(o), ro, dtype, f"case {i} step {step} o")
        assert_close(to_np(sg), sr, dtype, f"case {i} step {step} state")


@pytest.mark.parametrize("i", range(48))
def test_random_shape_conv_bit_exact(gpu, i):
    r = random.Random(12288 + i)
    dtype = torch.float32 if i % 2 == 0 else torch.bfloat16
    C = 8 * r.randint(1, 128)
    if r.random() < 0.5:
        lengths = [r.choice([0, 1, 2, 3, 4, r.randint(1, 150)]) for _ in range(r.randint(1, 8))]
        if sum(lengths) == 0:
            lengths[0] = 3
        d = wl.integer_conv_inputs(B=1, T=sum(lengths), C=C, dtype=dtype, lengths=lengths, seed=i)
    else:
        d = wl.integer_conv_inputs(B=r.randint(1, 3), T=r.randint(1, 300), C=C, dtype=dtype, seed=i)
    cu = d.get("cu_seqlens")
    run, threads = r.choice([0, 8, 16, 32]), r.choice([0, 64, 128, 256])
    try:
        gpu.gdn_tune_set(gpu.GDN_TUNE_CONV_RUN, run)
        gpu.gdn_tune_set(gpu.GDN_TUNE_CONV_THREADS, threads)
        y = gpu.gdn_conv1d_causal(d["x"].to(DEV), d["w"].to(DEV),
                                  cu_seqlens=None if cu is None else cu.to(DEV), silu=False)
        torch.cuda.synchronize()
    finally:
        gpu.gdn_tune_set(gpu.GDN_TUNE_CONV_RUN, 0)
        gpu.gdn_tune_set(gpu.GDN_TUNE_CONV_THREADS, 0)
    ref = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]),
                               cu_seqlens=None if cu is None else cu.numpy(), silu=False)
    if dtype == torch.bfloat16:
        ref = bf16_round(ref)
    np.testing.assert_array_equal(to_np(y), ref, err_msg=f"case {i}: C={C} run={run} threads={threads}")


@pytest.mark.parametrize("i", range(24))
def test_random_shape_gdp_prefill(gpu, i):
    r = random.Random(16384 + i)
    dtype = torch.float32 if i % 2 == 0 else torch.bfloat16
    B, T, M = r.randint(1, 2), r.randint(1, 150), r.randint(1, 3)
    G = r.randint(1, 3)
    H = G * r.choice([1, 2])
    P, N = r.choice([64, 128]), r.choice([64, 128])
    gen = torch.Generator().manual_seed(1300 + i)
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    x = torch.randn(B, T, xl, generator=gen).to(dtype)
    ba = torch.randn(B, T, bl, generator=gen).to(dtype)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    S0 = torch.randn(B, H, N, P, generator=gen) * 0.02 if r.random() < 0.5 else None
    o, sf = gpu.gdp_prefill(x.to(DEV), ba.to(DEV), A_log.to(DEV), dt_bias.to(DEV), M, H, G, P, N,
                            initial_state=None if S0 is None else S0.to(DEV), scale=0.5)
    torch.cuda.synchronize()
    ro, rsf = oracle.gdp_prefill(to_np(x), to_np(ba), to_np(A_log), to_np(dt_bias), M, H, G, P, N,
                                 S0=None if S0 is None else to_np(S0), scale=0.5)
    assert_close(to_np(o), ro, dtype, f"case {i} o")
    assert_close(to_np(sf), rsf, dtype, f"case {i} state")
