"""gdn_chunk_fwd_noalloc (the library's own fixed device workspace) against
gdn_chunk_fwd (a caller workspace): the same kernels on the same inputs, so
the outputs and final states must be equal bit for bit. Two calls in a row,
the second on a smaller input, check that the reused array's leftover
contents from the first call do not leak into the second; a packed call and
an fp32 call follow, and one call beyond the array's size is refused."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


def _inputs(**kw):
    d = wl.chunk_inputs(**kw)
    t = {n: (None if d[n] is None else d[n].to(DEV)) for n in ("q", "k", "v", "g", "beta", "S0",
                                                                 "cu_seqlens")}
    return d, t


def _both(gdn, d, t):
    ref_o, ref_s = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"],
                                     initial_state=t["S0"], cu_seqlens=t["cu_seqlens"])
    o = torch.full_like(ref_o, float("nan"))
    s = torch.full_like(ref_s, float("nan"))
    gdn.gdn_chunk_fwd_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], o,
                              initial_state=t["S0"], final_state=s, cu_seqlens=t["cu_seqlens"])
    torch.cuda.synchronize()
    return (o, s), (ref_o, ref_s)


def _equal(got, ref, what):
    assert torch.equal(got[0], ref[0]), f"{what}: o differs from gdn_chunk_fwd"
    assert torch.equal(got[1], ref[1]), f"{what}: final state differs from gdn_chunk_fwd"


def test_noalloc_equals_chunk_fwd_twice(gpu):
    print("noalloc: B=2 T=1000 H=4 then B=1 T=300 H=2, bf16", flush=True)
    d1, t1 = _inputs(B=2, T=1000, H=4, Hk=2, K=128, V=128, decay="weak", s0_std=0.05, seed=31)
    _equal(*_both(gpu, d1, t1), "first call")
    d2, t2 = _inputs(B=1, T=300, H=2, Hk=2, K=128, V=128, decay="strong", seed=32)
    _equal(*_both(gpu, d2, t2), "second, smaller call")


def test_noalloc_packed_and_fp32(gpu):
    print("noalloc: packed bf16 then fp32", flush=True)
    lens = [130, 1, 64, 257]
    d, t = _inputs(B=1, T=sum(lens), H=4, Hk=4, K=64, V=128, lengths=lens, seed=33)
    _equal(*_both(gpu, d, t), "packed")
    d, t = _inputs(B=1, T=200, H=2, Hk=2, K=64, V=64, dtype=torch.float32, seed=34)
    _equal(*_both(gpu, d, t), "fp32")


def test_noalloc_refuses_oversized(gpu):
    cap = gpu.gdn_chunk_fwd_noalloc_capacity()
    B, T, H = 1, 4096, 16
    while gpu.gdn_chunk_fwd_workspace_size(B, T, H, H, 64, 64, 0, torch.bfloat16) <= cap:
        T *= 2
    q = torch.zeros((B, T, H, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((B, T, H), device=DEV)
    o = torch.empty_like(q)
    with pytest.raises(gpu.GdnError, match="WORKSPACE"):
        gpu.gdn_chunk_fwd_noalloc(q, q, q, g, g, o)
