"""The benchmark's algorithmic bytes (CPU): each figure rebuilt here tensor
by tensor from the workload's shapes (every tensor of the method read or
written once), so a dropped tensor or a wrong element size in bench.py fails;
the whole prefill's two kernel shares add up to the step's bytes; the flop
count and the prefill workload's quoted figures are checked too."""
import pytest

import bench
import workloads as wl

MB = 1e6


def _prefill_shapes(name):
    w = wl.WORKLOADS[name]
    if w.n_seqs:
        # (the lengths are the workload's first draw)
        lens = wl.varlen_lengths(wl._gen(w.seed), w.n_seqs, w.max_len).tolist()
        tok = sum(lens)
        n_chunks = sum((x + 63) // 64 for x in lens)
        N = len(lens)
    else:
        tok = w.B * w.T
        n_chunks = w.B * ((w.T + 63) // 64)
        N = w.B
    return w, tok, n_chunks, N


@pytest.mark.parametrize("name", ["tiny", "prefill", "gqa", "varlen"])
def test_prefill_bytes_and_flops(name):
    w, tok, n_chunks, N = _prefill_shapes(name)
    es = 4 if name == "tiny" else 2
    H, Hk, K, V = w.H, w.Hk, w.K, w.V
    s0 = w.s0_std > 0
    acc = bench.accounting(tok, n_chunks, N, H, Hk, K, V, es, s0=s0)
    C = 2 * Hk * K + H * V
    q = k = tok * Hk * K * es
    v = o = tok * H * V * es
    g = beta = tok * H * 4
    a = b = tok * H * es
    x = tok * C * es
    taps = C * 4 * es
    state_out = N * H * K * V * 4
    state_in = state_out if s0 else 0
    assert acc["chunk_fwd"]["bytes"] == q + k + v + g + beta + o + state_out + state_in
    assert acc["prefill"]["bytes"] == x + a + b + taps + o + state_out + state_in
    assert acc["prefill_prepare"]["bytes"] + acc["prefill_scan"]["bytes"] == acc["prefill"]["bytes"]
    assert acc["conv1d"]["bytes"] == 2 * x + taps
    assert acc["chunk_scan"]["bytes"] == q + k + v + o + state_out + state_in
    # flops per token and head (chunk C = 64): 6 d^2 + 5 C d + 2/3 C^2 with
    # the intra-chunk products as lower triangles, 10 C d when dense
    per = 6 * K * K + 5 * 64 * K + 2 * 64 * 64 / 3
    per_dense = 6 * K * K + 10 * 64 * K + 2 * 64 * 64 / 3
    assert acc["chunk_fwd"]["flops"] == pytest.approx(tok * H * per)
    assert acc["chunk_fwd"]["flops_dense"] == pytest.approx(tok * H * per_dense)


def test_prefill_workload_figures():
    # the prefill workload's figures in MB / GFLOP, as the measurement is quoted
    w, tok, n_chunks, N = _prefill_shapes("prefill")
    acc = bench.accounting(tok, n_chunks, N, w.H, w.Hk, w.K, w.V)
    assert acc["chunk_fwd"]["bytes"] / MB == pytest.approx(274.73, abs=0.01)
    assert acc["prefill"]["bytes"] / MB == pytest.approx(273.73, abs=0.01)
    assert acc["prefill_scan"]["bytes"] / MB == pytest.approx(138.43, abs=0.01)
    assert acc["conv1d"]["bytes"] / MB == pytest.approx(402.70, abs=0.01)
    assert acc["chunk_fwd"]["flops"] / 1e9 == pytest.approx(37.22, abs=0.01)
    assert acc["chunk_fwd"]["flops_dense"] / 1e9 == pytest.approx(47.96, abs=0.01)


def test_decode_bytes():
    wd = wl.WORKLOADS["decode"]
    n, M, H, G, P, N = wd.n, wd.M, wd.H, wd.G, wd.V, wd.K
    state = n * H * N * P * 4
    x = n * (M * H * P + M * G * N + G * N) * 2
    ba = n * (M * H + H) * 2
    o = n * H * P * 2
    got = bench.decode_accounting(n, M, H, G, P, N)
    assert got == 2 * state + x + ba + o
    assert got / 1e9 == pytest.approx(1.0832, abs=1e-4)
