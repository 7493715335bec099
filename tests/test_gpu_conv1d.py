"""Parity of gdn_conv1d_causal (HIP) with the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.helpers import TOL, assert_close, bf16_round, to_np

pytestmark = pytest.mark.gpu


def _run(gdn, x, w, cu=None, silu=True, bias=None):
    dev = torch.device("cuda")
    xg = x.to(dev)
    y = gdn.gdn_conv1d_causal(xg, w.to(dev), bias=None if bias is None else bias.to(dev),
                              cu_seqlens=None if cu is None else cu.to(dev), silu=silu)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("B,T,C", [(1, 1, 8), (2, 37, 64), (3, 100, 384), (1, 300, 1024)])
def test_conv_integer_inputs_bit_exact(gpu, dtype, B, T, C):
    d = wl.integer_conv_inputs(B=B, T=T, C=C, dtype=dtype, seed=B * 1000 + T)
    y = _run(gpu, d["x"], d["w"], silu=False)
    ref = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]), silu=False)
    if dtype == torch.bfloat16:
        ref = bf16_round(ref)
    np.testing.assert_array_equal(to_np(y), ref)


@pytest.mark.parametrize("lengths", [[1], [5, 1, 64, 3, 1, 17], [1] * 40, [130, 2, 1, 999, 64, 65]])
def test_conv_varlen_bit_exact_no_leak(gpu, lengths):
    T = sum(lengths)
    d = wl.integer_conv_inputs(B=1, T=T, C=128, lengths=lengths, seed=len(lengths))
    y = _run(gpu, d["x"], d["w"], cu=d["cu_seqlens"], silu=False)
    ref = bf16_round(oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]),
                                          cu_seqlens=d["cu_seqlens"].numpy(), silu=False))
    np.testing.assert_array_equal(to_np(y), ref)


def test_conv_strided_views(gpu):
    # x and y as channel slices of wider buffers (token stride > C)
    dev = torch.device("cuda")
    d = wl.integer_conv_inputs(B=2, T=50, C=256, seed=3)
    big = torch.zeros(2, 50, 512, dtype=torch.bfloat16)
    big[:, :, 128:384] = d["x"]
    xg = big.to(dev)[:, :, 128:384]
    ybig = torch.full((2, 50, 320), 7.0, dtype=torch.bfloat16, device=dev)
    yv = ybig[:, :, 32:288]
    gpu.gdn_conv1d_causal(xg, d["w"].to(dev), y=yv, silu=False)
    torch.cuda.synchronize()
    ref = bf16_round(oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]), silu=False))
    np.testing.assert_array_equal(to_np(ybig[:, :, 32:288]), ref)
    assert (ybig[:, :, :32] == 7).all() and (ybig[:, :, 288:] == 7).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_conv_silu_bias_random(gpu, dtype):
    g = torch.Generator().manual_seed(5)
    x = (torch.randn(2, 77, 192, generator=g) * 2).to(dtype)
    w = (torch.randn(192, 4, generator=g) * 0.5).to(dtype)
    bias = torch.randn(192, generator=g).to(dtype)
    y = _run(gpu, x, w, bias=bias, silu=True)
    ref = oracle.conv1d_causal(to_np(x), to_np(w), bias=to_np(bias), silu=True)
    assert_close(to_np(y), ref, dtype, "conv silu+bias")


def test_conv_tiny_workload(gpu):
    w_ = wl.WORKLOADS["tiny"]
    d = wl.prefill_inputs(w_)
    y = _run(gpu, d["x"], d["w"])
    ref = oracle.conv1d_causal(to_np(d["x"]), to_np(d["w"]), silu=True)
    assert_close(to_np(y), ref, torch.float32, "tiny conv")


@pytest.mark.parametrize("name", ["prefill", "varlen", "gqa"])
def test_conv_full_size_workloads(gpu, name):
    # full-size launch; the oracle checks a sample of channels (the conv is per channel)
    w_ = wl.WORKLOADS[name]
    d = wl.prefill_inputs(w_)
    cu = d["cu_seqlens"]
    y = _run(gpu, d["x"], d["w"], cu=cu)
    C = d["C"]
    sel = np.unique(np.concatenate([np.arange(0, 64), np.arange(C // 2, C // 2 + 64),
                                    np.arange(C - 64, C)]))
    xs = to_np(d["x"][:, :, sel])
    ref = oracle.conv1d_causal(xs, to_np(d["w"][sel]),
                               cu_seqlens=None if cu is None else cu.numpy(), silu=True)
    assert_close(to_np(y[:, :, sel]), ref, torch.bfloat16, f"{name} conv")
    assert torch.isfinite(y).all()
