"""Parity of gdn_gate_prepare (HIP) with the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import to_np

pytestmark = pytest.mark.gpu


def _gates(gdn, a, b, A_log, dt_bias):
    dev = torch.device("cuda")
    g, beta = gdn.gdn_gate_prepare(a.to(dev), b.to(dev), A_log.to(dev), dt_bias.to(dev))
    torch.cuda.synchronize()
    return to_np(g), to_np(beta)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gates_random(gpu, dtype):
    gen = torch.Generator().manual_seed(9)
    R, H = 1000, 16
    a = (torch.randn(R, H, generator=gen) * 8).to(dtype)
    b = (torch.randn(R, H, generator=gen) * 8).to(dtype)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    g, beta = _gates(gpu, a, b, A_log, dt_bias)
    gr, br = oracle.gate_prepare(to_np(a), to_np(b), to_np(A_log), to_np(dt_bias))
    # fp32 transcendentals: a few ulp relative per element
    np.testing.assert_allclose(beta, br, rtol=2e-6, atol=1e-30)
    np.testing.assert_allclose(g, gr, rtol=4e-6, atol=1e-37)
    assert (g <= 0).all() and (beta >= 0).all() and (beta <= 1).all()


def test_gates_threshold_and_tails(gpu):
    # softplus switches to the identity strictly above 20; far tails stay finite
    xs = np.array([19.0, 19.999998, 20.0, 20.000002, 21.0, -20.0, -80.0, -100.0, -120.0,
                   0.0, 1e-3, 88.0, 1e4], np.float32)
    H = xs.size
    a = torch.from_numpy(xs)[None, :]
    b = torch.from_numpy(np.linspace(-100, 100, H).astype(np.float32))[None, :]
    zeros = torch.zeros(H)
    g, beta = _gates(gpu, a, b, zeros, zeros)
    gr, br = oracle.gate_prepare(to_np(a), to_np(b), np.zeros(H), np.zeros(H))
    # fp32 underflow: exp(-100) and below flush to (sub)normal tiny values or 0
    np.testing.assert_allclose(g, gr, rtol=4e-6, atol=1e-38)
    np.testing.assert_allclose(beta, br, rtol=2e-6, atol=1e-30)
    assert g[0, 3] == -np.float32(20.000002) and g[0, 4] == -21.0
    assert np.isfinite(g).all() and np.isfinite(beta).all()


def test_gates_strided_rows(gpu):
    # a and b as column slices of one wider projection row (non-contiguous rows)
    gen = torch.Generator().manual_seed(2)
    R, H = 300, 32
    ba = torch.randn(R, 3 * H, generator=gen).to(torch.bfloat16)
    dev = torch.device("cuda")
    bag = ba.to(dev)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    g, beta = gpu.gdn_gate_prepare(bag[:, 2 * H:], bag[:, :H], A_log.to(dev), dt_bias.to(dev))
    torch.cuda.synchronize()
    gr, br = oracle.gate_prepare(to_np(ba[:, 2 * H:]), to_np(ba[:, :H]), to_np(A_log), to_np(dt_bias))
    np.testing.assert_allclose(to_np(g), gr, rtol=4e-6)
    np.testing.assert_allclose(to_np(beta), br, rtol=2e-6)


@pytest.mark.parametrize("name", ["prefill", "gqa"])
def test_gates_full_size(gpu, name):
    d = wl.prefill_inputs(wl.WORKLOADS[name])
    g, beta = _gates(gpu, d["a"], d["b"], d["A_log"], d["dt_bias"])
    gr, br = oracle.gate_prepare(to_np(d["a"]), to_np(d["b"]), to_np(d["A_log"]), to_np(d["dt_bias"]))
    np.testing.assert_allclose(beta, br, rtol=2e-6, atol=1e-30)
    np.testing.assert_allclose(g, gr, rtol=4e-6, atol=1e-37)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gates_four_wide_and_one_wide_agree(gpu, dtype):
    # contiguous rows with H % 4 == 0 take four heads per thread; the same
    # values one element off a 4-element boundary take one per thread: the
    # results must be the same bits
    gen = torch.Generator().manual_seed(31)
    R, H = 517, 16
    wide_a = (torch.randn(R, H + 1, generator=gen) * 8).to(dtype)
    wide_b = (torch.randn(R, H + 1, generator=gen) * 8).to(dtype)
    A_log = torch.log(1 + 15 * torch.rand(H, generator=gen))
    dt_bias = torch.randn(H, generator=gen) * 0.1
    dev = torch.device("cuda")
    wa, wb = wide_a.to(dev), wide_b.to(dev)
    A, D = A_log.to(dev), dt_bias.to(dev)
    g1, b1 = gpu.gdn_gate_prepare(wa[:, 1:], wb[:, 1:], A, D)               # misaligned rows
    g4, b4 = gpu.gdn_gate_prepare(wa[:, 1:].contiguous(), wb[:, 1:].contiguous(), A, D)
    torch.cuda.synchronize()
    assert torch.equal(g1, g4) and torch.equal(b1, b4)
    gr, br = oracle.gate_prepare(to_np(wide_a[:, 1:]), to_np(wide_b[:, 1:]), to_np(A_log),
                                 to_np(dt_bias))
    np.testing.assert_allclose(to_np(g4), gr, rtol=4e-6, atol=1e-37)
    np.testing.assert_allclose(to_np(b4), br, rtol=2e-6, atol=1e-30)
