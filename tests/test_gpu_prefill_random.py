"""gdn_prefill on seeded random shapes: equal bit for bit to the four-step
chain (conv1d + SiLU, gates, chunk_prepare, chunk_scan) under every scan
schedule (column groups of one and two tiles, whole units), and within the
bf16 bar of the fp64 oracle on the first few.

The shapes come from a fixed seed: head dims K and V in {64, 128}, 1, 2 or 4
key heads with 1, 2 or 4 value heads each, either dense batches whose length
falls on or next to a chunk boundary, or up to six packed sequences of 0 to
200 tokens, with or without an initial state and a conv bias. The inputs
follow the prefill workload's distributions (seed 1000 + case)."""
import random

import pytest
import torch

import workloads as wl
from tests.helpers import assert_close, to_np
from tests.test_gpu_prefill import _bias, _chain, _equal, _fused, _oracle

pytestmark = pytest.mark.gpu
BF16 = torch.bfloat16
N_CASES = 12
ORACLE_CASES = 4


def _draw(i):
    r = random.Random(2024 + i)
    K, V = r.choice([64, 128]), r.choice([64, 128])
    Hk = r.choice([1, 2, 4])
    H = Hk * r.choice([1, 2, 4])
    w = wl.Workload(f"random-{i}", 2, BF16, H=H, Hk=Hk, K=K, V=V,
                    s0_std=0.02 if r.random() < 0.5 else 0.0)
    if r.random() < 0.5:
        lengths = [r.choice([0, 1, 2, 3, 63, 64, 65, 127, 128, 129, r.randint(1, 200)])
                   for _ in range(r.randint(1, 6))]
        if sum(lengths) == 0:
            lengths[0] = 5
        kw = dict(lengths=lengths)
    else:
        kw = dict(B=r.randint(1, 3), T=r.choice([1, 63, 64, 65, 128, 191, r.randint(1, 300)]))
    return w, kw, r.random() < 0.5


def _case(i):
    w, kw, use_bias = _draw(i)
    d = wl.prefill_inputs(w, seed=1000 + i, **kw)
    return d, (_bias(d["C"], seed=i) if use_bias else None)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_prefill_equals_chain(gpu, i):
    d, bias = _case(i)
    ref = _chain(gpu, d, bias=bias)
    try:
        for form, tiles in ((1, 1), (1, 2), (2, 0)):
            gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, form)
            gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_TILES, tiles)
            _equal(_fused(gpu, d, bias=bias), ref, f"case {i}, form {form}, {tiles} tile(s)")
    finally:
        gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, 0)
        gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_TILES, 0)


@pytest.mark.parametrize("i", range(ORACLE_CASES))
def test_random_shape_prefill_matches_oracle(gpu, i):
    d, bias = _case(i)
    o, sf = _fused(gpu, d, bias=bias)
    ro, rs = _oracle(d, bias=bias)
    assert_close(to_np(o), ro, BF16, f"case {i} o")
    assert_close(to_np(sf), rs, BF16, f"case {i} state")
