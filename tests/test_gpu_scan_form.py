"""The two workgroup forms of the bf16 state scan (GDN_TUNE_SCAN_FORM):
column groups with role-split waves (1), and one workgroup per (sequence,
head) unit over all its value columns (2). The form only reschedules the
same arithmetic: both must give the same bits on every shape, and each is
checked against the fp64 oracle directly on the small shapes (head dims,
GQA, ragged and packed lengths, an initial state, scale, no normalisation)
and at the workloads' full sizes on sampled units. The whole prefill's scan
(which also convolves the value rows) has both forms too: each must equal
the conv1d -> gates -> chunk_fwd chain bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import assert_close, to_np

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")
BF16 = torch.bfloat16
# (form, tiles): column groups; whole units with four compute waves of two
# tiles and a copy wave; whole units with eight compute waves of one tile
FORMS = ((1, 0), (2, 0), (2, 1))


@pytest.fixture
def form(gpu):
    yield gpu
    gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, 0)
    gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_TILES, 0)


def _run(gdn, d, f, **kw):
    gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_FORM, f[0])
    gdn.gdn_tune_set(gdn.GDN_TUNE_SCAN_TILES, f[1])
    t = {n: (None if d[n] is None else d[n].to(DEV)) for n in ("q", "k", "v", "g", "beta", "S0", "cu_seqlens")}
    o, sf = gdn.gdn_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], initial_state=t["S0"],
                              cu_seqlens=t["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, sf


def _oracle(d, **kw):
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].numpy()
    return oracle.gated_delta_rule(to_np(d["q"]), to_np(d["k"]), to_np(d["v"]), to_np(d["g"]),
                                   to_np(d["beta"]), S0=None if d["S0"] is None else to_np(d["S0"]),
                                   cu_seqlens=cu, **kw)


SMALL = {
    "k128v128": dict(B=2, T=321, H=4, Hk=4, K=128, V=128),
    "k64v64": dict(B=2, T=200, H=2, Hk=2, K=64, V=64),
    "k64v128": dict(B=1, T=130, H=2, Hk=1, K=64, V=128),
    "k128v64": dict(B=1, T=257, H=4, Hk=2, K=128, V=64),
    "gqa-s0": dict(B=1, T=700, H=4, Hk=2, K=128, V=128, s0_std=0.05, decay="weak"),
    "one-token": dict(B=3, T=1, H=2, Hk=2, K=128, V=128, s0_std=0.1),
    "packed": dict(B=1, T=1 + 64 + 65 + 200 + 3, H=2, Hk=2, K=128, V=128,
                   lengths=[1, 64, 65, 200, 3], decay="weak"),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_forms_equal_and_match_oracle(form, case):
    kw = dict(SMALL[case])
    d = wl.chunk_inputs(dtype=BF16, seed=hash(case) % 1000, **kw)
    print(f"scan forms: {case}", flush=True)
    ref = _run(form, d, FORMS[0])
    ro, rs = _oracle(d)
    for f in FORMS:
        o, sf = _run(form, d, f)
        assert torch.equal(o, ref[0]) and torch.equal(sf, ref[1]), (case, f)
        assert_close(to_np(o), ro, BF16, f"{case} form={f} o")
        assert_close(to_np(sf), rs, BF16, f"{case} form={f} state")


def test_forms_scale_and_no_norm(form):
    d = wl.chunk_inputs(B=1, T=150, H=2, Hk=2, K=128, V=128, dtype=BF16, seed=5)
    # no normalisation: keys of unit norm so the recurrence stays bounded
    for n in ("q", "k"):
        x = d[n].float()
        d[n] = (x / x.norm(dim=-1, keepdim=True)).to(BF16)
    for kw in (dict(scale=128 ** -0.5), dict(qk_l2norm=False)):
        ref = _run(form, d, FORMS[0], **kw)
        ro, rs = _oracle(d, scale=kw.get("scale", 1.0), l2norm=kw.get("qk_l2norm", True))
        for f in FORMS[1:]:
            o, sf = _run(form, d, f, **kw)
            assert torch.equal(o, ref[0]) and torch.equal(sf, ref[1]), (kw, f)
            assert_close(to_np(o), ro, BF16, f"form={f} {kw} o")


@pytest.mark.parametrize("name", ["prefill", "gqa", "varlen"])
def test_forms_equal_full_size(form, name):
    # the workloads' full sizes through conv1d + gates + chunk_fwd: the forms
    # agree bit for bit (the chain itself is checked against the oracle at
    # these sizes in test_gpu_chunk.py)
    w = wl.WORKLOADS[name]
    d = wl.prefill_inputs(w)
    print(f"scan forms full size: {name}", flush=True)
    t = {n: d[n].to(DEV) for n in ("x", "w", "a", "b", "A_log", "dt_bias")}
    S0 = None if d["S0"] is None else d["S0"].to(DEV)
    cu = None if d["cu_seqlens"] is None else d["cu_seqlens"].to(DEV)
    outs = []
    for f in FORMS:
        form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, f[0])
        form.gdn_tune_set(form.GDN_TUNE_SCAN_TILES, f[1])
        o, sf = form.prefill_chain(t["x"], t["w"], t["a"], t["b"], t["A_log"], t["dt_bias"],
                                   Hk=w.Hk, K=w.K, H=w.H, V=w.V, initial_state=S0, cu_seqlens=cu)
        torch.cuda.synchronize()
        outs.append((o, sf))
    for i in range(1, len(FORMS)):
        assert torch.equal(outs[0][0], outs[i][0]), f"{name}: o differs, form {FORMS[i]}"
        assert torch.equal(outs[0][1], outs[i][1]), f"{name}: final state differs, form {FORMS[i]}"


# whole prefill (gdn_prefill): the scan also convolves the value rows; both
# forms must equal the conv1d -> gates -> chunk_fwd chain bit for bit
@pytest.mark.parametrize("case", ["prefill-321", "gqa-700", "varlen-edges", "k64-v128",
                                  "k128-v64", "k64-v64"])
def test_forms_whole_prefill_equal_chain(form, case):
    from tests.test_gpu_prefill import SMALL as PSMALL, _bias, _chain, _fused, _equal
    w, kw = PSMALL[case]
    d = wl.prefill_inputs(w, **kw)
    print(f"scan forms, whole prefill: {case}", flush=True)
    bias = _bias(d["C"])
    ref = _chain(form, d)
    refb = _chain(form, d, bias=bias, scale=0.125)
    for f in FORMS[:2]:
        form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, f[0])
        _equal(_fused(form, d), ref, f"{case} form={f}")
        _equal(_fused(form, d, bias=bias, scale=0.125), refb, f"{case} form={f} bias, scale")
        form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, 0)


@pytest.mark.parametrize("name", ["prefill", "gqa", "varlen"])
def test_forms_whole_prefill_full_size(form, name):
    from tests.test_gpu_prefill import _chain, _fused, _equal
    d = wl.prefill_inputs(wl.WORKLOADS[name])
    print(f"scan forms, whole prefill full size: {name}", flush=True)
    ref = _chain(form, d)
    for f in FORMS[:2]:
        form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, f[0])
        _equal(_fused(form, d), ref, f"{name} form={f}")
        form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, 0)


@pytest.mark.parametrize("n", [1000, 1100])
def test_forms_many_packed_sequences(form, n):
    # more (sequence, head) units than the whole-unit threshold; 1,000
    # sequences are started longest first (the order is a rank sort on the
    # device, ties by index), 1,100 in index order (past the sort's limit of
    # 1,024). Lengths 0..130 (zero-length sequences pass S0 through); every
    # unit is compared with the oracle, so an order that repeated or skipped a
    # unit would show.
    gen = np.random.default_rng(n)
    lengths = [int(x) for x in gen.integers(0, 131, n)]
    lengths[3] = 0
    lengths[7] = 130
    d = wl.chunk_inputs(B=1, T=sum(lengths), H=1, Hk=1, K=128, V=128, dtype=BF16,
                        lengths=lengths, s0_std=0.05, seed=n)
    print(f"scan forms: {n} packed sequences, {sum(lengths)} tokens", flush=True)
    ref = _run(form, d, FORMS[0])
    ro, rs = _oracle(d)
    for f in FORMS[1:]:
        o, sf = _run(form, d, f)
        assert torch.equal(o, ref[0]) and torch.equal(sf, ref[1]), (n, f)
    assert_close(to_np(ref[0]), ro, BF16, f"{n} packed o")
    assert_close(to_np(ref[1]), rs, BF16, f"{n} packed state")
    # the automatic choice (whole units from 512 units) gives the same bits
    o, sf = _run(form, d, (0, 0))
    assert torch.equal(o, ref[0]) and torch.equal(sf, ref[1])


def test_forms_without_final_state(form):
    # no final state requested: the scan skips its store; o is unchanged
    d = wl.chunk_inputs(B=2, T=200, H=4, Hk=2, K=128, V=128, dtype=BF16, s0_std=0.05, seed=11)
    ref = _run(form, d, FORMS[0])
    for f in FORMS:
        o, sf = _run(form, d, f, output_final_state=False)
        assert sf is None
        assert torch.equal(o, ref[0]), f


@pytest.mark.parametrize("n", [1000, 1100])
def test_forms_whole_prefill_many_packed_sequences(form, n):
    # the whole prefill over many short packed sequences (lengths 0..130, an
    # initial state): past the whole-unit threshold the automatic choice runs
    # the auxiliary-wave form, longest first for 1,000 sequences and in index
    # order for 1,100. Both forms and the automatic choice equal the
    # conv1d -> gates -> chunk_fwd chain bit for bit, and every unit matches
    # the oracle.
    from tests.test_gpu_prefill import _chain, _fused, _equal, _oracle as _poracle
    gen = np.random.default_rng(n + 1)
    lengths = [int(x) for x in gen.integers(0, 131, n)]
    lengths[5] = 0
    lengths[9] = 130
    w = wl.Workload(f"packed{n}", 4, BF16, H=1, Hk=1, K=128, V=128, s0_std=0.05)
    d = wl.prefill_inputs(w, lengths=lengths, seed=n)
    print(f"scan forms, whole prefill: {n} packed sequences, {sum(lengths)} tokens", flush=True)
    ref = _chain(form, d)
    for f in ((1, 0), (2, 0), (0, 0)):
        form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, f[0])
        _equal(_fused(form, d), ref, f"{n} packed form={f}")
    form.gdn_tune_set(form.GDN_TUNE_SCAN_FORM, 0)
    ro, rs = _poracle(d)
    assert_close(to_np(ref[0]), ro, BF16, f"{n} packed whole prefill o")
    assert_close(to_np(ref[1]), rs, BF16, f"{n} packed whole prefill state")
