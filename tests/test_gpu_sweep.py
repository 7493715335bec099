"""A seeded sweep over random shapes, wider than the per-feature tests: 300
whole prefills and 300 chunked forwards, in blocks of 50 cases.

Whole prefill (bf16): head dims 64 / 128, 1 to 8 q/k heads with 1, 2 or 4
value heads each, dense batches of 1 to 6 rows or up to 40 packed sequences
of 0 to 400 tokens (lengths on and next to chunk boundaries among them), with
or without an initial state and a conv bias, scale 1 or 1/8. Every scan
schedule gives the bits of the per-step chain, and the chain is within the
bf16 bar of the oracle.

Chunked forward (fp32 and bf16, stage inputs drawn directly): the decay
regimes, with or without an initial state, scale or no normalisation. Every
schedule of the dtype gives the same bits, and the result is within the
dtype's bar of the oracle."""
import random

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import TOL, assert_close, to_np
from tests.test_gpu_prefill import _bias, _chain, _fused, _oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16, FP32 = torch.bfloat16, torch.float32
BLOCK = 50
SCHEDULES = {BF16: [(0, 0), (1, 1), (1, 2), (2, 0), (2, 1)], FP32: [(0, 0), (0, 1), (0, 4)]}


def _set(gdn, sched):
    gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, sched[0])
    gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, sched[1])


def _prefill_case(i):
    r = random.Random(777 + i)
    K, V = r.choice([64, 128]), r.choice([64, 128])
    Hk = r.choice([1, 2, 3, 4, 8])
    H = Hk * r.choice([1, 2, 4])
    w = wl.Workload(f"sweep-{i}", 2, BF16, H=H, Hk=Hk, K=K, V=V,
                    s0_std=0.02 if r.random() < 0.5 else 0.0)
    if r.random() < 0.5:
        lengths = [r.choice([0, 1, 2, 3, 4, 63, 64, 65, 127, 128, 129, 191, 192, 193, r.randint(1, 400)])
                   for _ in range(r.randint(1, 40))]
        if sum(lengths) == 0:
            lengths[0] = 7
        kw = dict(lengths=lengths)
    else:
        kw = dict(B=r.randint(1, 6),
                  T=r.choice([1, 2, 3, 63, 64, 65, 127, 128, 129, 255, 256, 257, r.randint(1, 700)]))
    d = wl.prefill_inputs(w, seed=5000 + i, **kw)
    bias = _bias(d["C"], seed=i) if r.random() < 0.5 else None
    return d, bias, r.choice([1.0, 0.125])


@pytest.mark.parametrize("block", range(6))
def test_sweep_prefill(gpu, block):
    print(f"prefill sweep, cases {block * BLOCK} .. {block * BLOCK + BLOCK - 1}", flush=True)
    worst = 0.0
    try:
        for i in range(block * BLOCK, (block + 1) * BLOCK):
            d, bias, scale = _prefill_case(i)
            ref = _chain(gpu, d, bias=bias, scale=scale)
            for sched in SCHEDULES[BF16]:
                _set(gpu, sched)
                o, sf = _fused(gpu, d, bias=bias, scale=scale)
                assert torch.equal(o, ref[0]) and torch.equal(sf, ref[1]), f"case {i}, schedule {sched}"
            _set(gpu, (0, 0))
            ro, rs = _oracle(d, bias=bias, scale=scale)
            worst = max(worst, assert_close(to_np(ref[0]), ro, BF16, f"prefill case {i} o"),
                        assert_close(to_np(ref[1]), rs, BF16, f"prefill case {i} state"))
    finally:
        _set(gpu, (0, 0))
    print(f"worst {worst:.2e}", flush=True)


def _chunk_case(i):
    r = random.Random(4242 + i)
    dtype = r.choice([BF16, FP32])
    K, V = r.choice([64, 128]), r.choice([64, 128])
    Hk = r.choice([1, 2, 3, 4])
    H = Hk * r.choice([1, 2, 4])
    common = dict(H=H, Hk=Hk, K=K, V=V, dtype=dtype, decay=r.choice(list(wl.DECAY_GMAX)),
                  s0_std=r.choice([0.0, 0.05]), seed=9000 + i)
    if r.random() < 0.5:
        lengths = [r.choice([0, 1, 2, 63, 64, 65, 128, 129, r.randint(1, 300)])
                   for _ in range(r.randint(1, 20))]
        if sum(lengths) == 0:
            lengths[0] = 3
        d = wl.chunk_inputs(B=1, T=sum(lengths), lengths=lengths, **common)
    else:
        d = wl.chunk_inputs(B=r.randint(1, 4), T=r.choice([1, 63, 64, 65, 127, 200, r.randint(1, 500)]),
                            **common)
    kw = r.choice([dict(), dict(scale=0.125), dict(qk_l2norm=False)])
    if "qk_l2norm" in kw:
        # without the kernel's normalisation, keys and queries of unit norm
        # keep the recurrence bounded
        for n in ("q", "k"):
            x = d[n].float()
            d[n] = (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(dtype)
    return d, kw


@pytest.mark.parametrize("block", range(6))
def test_sweep_chunk_fwd(gpu, block):
    print(f"chunked-forward sweep, cases {block * BLOCK} .. {block * BLOCK + BLOCK - 1}", flush=True)
    try:
        for i in range(block * BLOCK, (block + 1) * BLOCK):
            d, kw = _chunk_case(i)
            t = {n: (None if d[n] is None else d[n].to(DEV))
                 for n in ("q", "k", "v", "g", "beta", "S0", "cu_seqlens")}
            outs = []
            for sched in SCHEDULES[d["dtype"]]:
                _set(gpu, sched)
                o, sf = gpu.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["S0"],
                                          cu_seqlens=t["cu_seqlens"], **kw)
                outs.append((o, sf))
            _set(gpu, (0, 0))
            torch.cuda.synchronize()
            for sched, (o, sf) in zip(SCHEDULES[d["dtype"]][1:], outs[1:]):
                assert torch.equal(o, outs[0][0]) and torch.equal(sf, outs[0][1]), f"case {i}, schedule {sched}"
            cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
            ro, rs = oracle.gated_delta_rule(to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["g"]),
                                             to_np(d["beta"]), S0=None if d["S0"] is None else to_np(d["S0"]),
                                             cu_seqlens=cu, scale=kw.get("scale", 1.0),
                                             l2norm=kw.get("qk_l2norm", True))
            assert_close(to_np(outs[0][0]), ro, d["dtype"], f"chunk case {i} o")
            assert_close(to_np(outs[0][1]), rs, d["dtype"], f"chunk case {i} state")
    finally:
        _set(gpu, (0, 0))
