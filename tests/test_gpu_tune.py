"""Launch-configuration knobs (gdn_tune_set) change scheduling only: every
value gives the automatic setting's results bit for bit, on shapes that span
several tiles, a ragged tail and packed sequences."""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.fixture
def knobs(gpu):
    yield gpu
    for k in (gpu.GDN_TUNE_SCAN_TILES, gpu.GDN_TUNE_CONV_RUN, gpu.GDN_TUNE_CONV_THREADS,
              gpu.GDN_TUNE_SCAN_FORM):
        gpu.gdn_tune_set(k, 0)


CASES = {
    "prefill-321": (wl.WORKLOADS["prefill"], dict(T=321, B=2)),
    "varlen-edges": (wl.WORKLOADS["varlen"], dict(lengths=[1, 3, 64, 0, 65, 200, 17])),
    "tiny-fp32": (wl.WORKLOADS["tiny"], dict(T=200)),
}


def _inputs(case):
    w, kw = CASES[case]
    d = wl.prefill_inputs(w, **kw)
    t = {n: d[n].to(DEV) for n in ("x", "w", "a", "b", "A_log", "dt_bias")}
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(DEV)
    return w, t, cu


@pytest.mark.parametrize("case", list(CASES))
def test_scan_tiles_do_not_change_results(knobs, case):
    w, t, cu = _inputs(case)
    dims = dict(Hk=w.Hk, K=w.K, H=w.H, V=w.V)
    fwd = knobs.gdn_prefill if w.dtype == torch.bfloat16 else knobs.prefill_chain
    ref = fwd(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"], cu_seqlens=cu, **dims)
    values = [1, 2, 4] if w.dtype == torch.bfloat16 else [1, 4, 2]   # (2 / 4: falls back)
    for v in values:
        knobs.gdn_tune_set(knobs.GDN_TUNE_SCAN_TILES, v)
        got = fwd(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"], cu_seqlens=cu, **dims)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), (case, v)


@pytest.mark.parametrize("case", list(CASES))
def test_conv_shapes_do_not_change_results(knobs, case):
    w, t, cu = _inputs(case)
    ref = knobs.gdn_conv1d_causal(t["x"], t["w"], cu_seqlens=cu, silu=True)
    for run in (8, 16, 32):
        for nth in (64, 128, 256):
            knobs.gdn_tune_set(knobs.GDN_TUNE_CONV_RUN, run)
            knobs.gdn_tune_set(knobs.GDN_TUNE_CONV_THREADS, nth)
            got = knobs.gdn_conv1d_causal(t["x"], t["w"], cu_seqlens=cu, silu=True)
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (case, run, nth)
