"""Sizes past the int32 range: element offsets into x, o and the decode state
beyond 2^31, where an index product formed in 32 bits would wrap.

The whole prefill runs on two packed sequences, 1,060,000 tokens in all: x
holds 6.5e9 elements, o 2.2e9. The second sequence starts past x element 2^31
and its last outputs lie past o element 2^31. Three checks follow. The whole
prefill equals the per-step chain (conv1d -> gates -> chunked forward) bit for
bit over all of o and the final states, in both scan workgroup forms. Windows
of o at the end of each sequence, and at the token where x's offsets cross
2^31, match the oracle; so do both final states. Each window's oracle run
starts from a zero state some hundreds of tokens earlier. This is exact to far
below the bar: the test requires the decay over the skipped prefix, exp(sum of
g), to be under 1e-30. Each step's factor (I - beta k k^T) has norm at most 1,
so whatever the state held before the prefix reaches the window scaled by at
most that product. The decode runs on 4,200 requests, whose fp32 state holds
2.2e9 elements, and sampled requests match the oracle's step.
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
I32 = 2 ** 31

W_BIG = wl.Workload("past-int32", 2, BF16, H=16, Hk=16, K=128, V=128)
LENGTHS = [400_000, 660_000]      # packed: T = 1,060,000
PREFIX = 512                      # oracle warm-up tokens before each window
WINDOW = 320                      # checked tokens per window
HEADS = [0, 9, 15]


def _window_oracle(d, h, t0, t1, seq_start):
    """o over tokens [t0, t1) and the state after t1 for value head h, from the
    oracle run on [t0 - PREFIX, t1) from a zero state (the conv reads the three
    rows before that, within the sequence). Returns (o [L, V], S [K, V],
    decay of the skipped prefix)."""
    Hk, K, H, V = W_BIG.Hk, W_BIG.K, W_BIG.H, W_BIG.V
    hk = h // (H // Hk)
    s0 = t0 - PREFIX
    assert s0 - 3 >= seq_start
    rows = slice(s0 - 3, t1)
    ch = np.r_[hk * K:(hk + 1) * K, Hk * K + hk * K:Hk * K + (hk + 1) * K,
               2 * Hk * K + h * V:2 * Hk * K + (h + 1) * V]
    chd = torch.as_tensor(ch, device=DEV)
    x = to_np(d["x"][0, rows].index_select(1, chd))[None]
    w = to_np(d["w"].index_select(0, chd))
    y = oracle.conv1d_causal(x, w, silu=True)[:, 3:]           # rows s0 .. t1 - 1
    q = y[:, :, :K].reshape(1, -1, 1, K)
    k = y[:, :, K:2 * K].reshape(1, -1, 1, K)
    v = y[:, :, 2 * K:].reshape(1, -1, 1, V)
    a = to_np(d["a"][0, s0:t1, h:h + 1])[None]
    b = to_np(d["b"][0, s0:t1, h:h + 1])[None]
    g, beta = oracle.gate_prepare(a, b, to_np(d["A_log"][h:h + 1]), to_np(d["dt_bias"][h:h + 1]))
    o, S = oracle.gated_delta_rule(q, k, v, g, beta)
    decay = float(np.exp(g[0, :PREFIX, 0].sum()))
    return o[0, PREFIX:, 0], S[0, 0], decay


def _prefill(gdn, d):
    o, sf = gdn.gdn_prefill(d["x"], d["w"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                            Hk=W_BIG.Hk, K=W_BIG.K, H=W_BIG.H, V=W_BIG.V, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return o, sf


def test_prefill_past_int32_offsets(gpu):
    d = wl.device_prefill_inputs(W_BIG, DEV, lengths=LENGTHS, seed=7)
    T, C, H, V = d["T"], d["C"], W_BIG.H, W_BIG.V
    assert d["x"].numel() > 2 * I32 and T * H * V > I32
    print(f"past int32: T={T}, x {d['x'].numel():.3g} elements, o {T * H * V:.3g}", flush=True)
    o, sf = _prefill(gpu, d)
    # the per-step chain, bit for bit
    oc, sfc = gpu.prefill_chain(d["x"], d["w"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                Hk=W_BIG.Hk, K=W_BIG.K, H=H, V=V, cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o, oc), "whole prefill differs from the chain"
    assert torch.equal(sf, sfc), "final states differ from the chain"
    del oc, sfc
    # the whole-unit scan form, bit for bit
    gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, 2)
    try:
        ow, sfw = _prefill(gpu, d)
    finally:
        gpu.gdn_tune_set(gpu.GDN_TUNE_SCAN_FORM, 0)
    assert torch.equal(o, ow), "whole-unit form differs"
    assert torch.equal(sf, sfw), "whole-unit form's final states differ"
    del ow, sfw
    # oracle windows: the end of each sequence (and its final state), and the
    # token at which x's element offsets pass 2^31
    ends = np.cumsum(LENGTHS)
    t_cross = -(-I32 // C)
    windows = [(0, int(ends[0]) - WINDOW, int(ends[0]), 0),
               (1, int(ends[1]) - WINDOW, int(ends[1]), int(ends[0])),
               (0, t_cross - WINDOW // 2, t_cross + WINDOW // 2, 0)]
    assert windows[1][1] * C > I32 and (T - 1) * H * V > I32
    for seq, t0, t1, start in windows:
        for h in HEADS:
            ro, rs, decay = _window_oracle(d, h, t0, t1, start)
            assert decay < 1e-30, (seq, t0, h, decay)
            tag = f"seq {seq} tokens {t0}..{t1} head {h}"
            assert_close(to_np(o[0, t0:t1, h]), ro, BF16, f"{tag} o")
            if t1 == int(ends[seq]):
                assert_close(to_np(sf[seq, h]), rs, BF16, f"{tag} final state")
    assert torch.isfinite(o).all()


def test_decode_past_int32_state(gpu):
    w = wl.WORKLOADS["decode"]
    n = 4200
    M, H, G, P, N = w.M, w.H, w.G, w.V, w.K
    assert n * H * N * P > I32
    gen = torch.Generator(device=DEV)
    gen.manual_seed(8)
    state = torch.randn((n, H, N, P), generator=gen, device=DEV) * w.s0_std
    xl, bl = wl.decode_row_sizes(M, H, G, P, N)
    x = torch.randn((n, xl), generator=gen, device=DEV, dtype=BF16)
    ba = torch.randn((n, bl), generator=gen, device=DEV, dtype=BF16)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen, device=DEV))
    dt_bias = torch.randn(H, generator=gen, device=DEV) * 0.1
    sample = [0, 2100, n - 1]
    s0 = to_np(state[sample])
    print(f"decode past int32: n={n}, state {state.numel():.3g} elements", flush=True)
    o = gpu.gdn_recurrent_decode(x, ba, A_log, dt_bias, state, M, H, G, P, N)
    torch.cuda.synchronize()
    ro, rs = oracle.gdp_decode(to_np(x[sample]), to_np(ba[sample]), to_np(A_log), to_np(dt_bias),
                               s0, M, H, G, P, N)
    assert_close(to_np(o[sample]), ro, BF16, "decode o")
    assert_close(to_np(state[sample]), rs, BF16, "decode state")
