"""Seeded synthetic inputs for the gated-delta-rule workloads.

This module only draws random numbers (CPU ``torch.Generator``, fp32 draws,
one RNE cast to the workload dtype). It holds none of the method's arithmetic,
and it is the only code that the HIP path's tests and the fp64 oracle share:
both sides receive the very same host tensors from here.

Workloads (the dimensions of the five configurations the repository is
measured on; "std" below is the standard deviation):

* ``tiny``    fp32, B=1, H=Hk=2, T=128, K=V=64
* ``prefill`` bf16, B=4, H=Hk=16, T=4096, K=V=128
* ``gqa``     bf16, B=1, H=32 value heads over Hk=16 q/k heads, T=65536,
              K=V=128, initial state ~N(0, 0.02) fp32 [1, 32, 128, 128]
* ``varlen``  bf16, 64 sequences, lengths uniform in [1, 2048], packed,
              H=Hk=16, K=V=128
* ``decode``  bf16, n=256 requests, M=2 Householder copies, H=32, G=16,
              P=N=128, fp32 state ~N(0, 0.02), 1000 steps

Prefill draw order (seed 100 + workload number): [varlen: lengths], then conv
input x [B, T, C] ~N(0, 1) with C = 2*Hk*K + H*V in q|k|v channel order, conv
weight w [C, 4] ~N(0, 0.5), a [B, T, H] ~N(0, 1), b [B, T, H] ~N(0, 1),
A_log = log U[1, 16] [H], dt_bias ~N(0, 0.1) [H], [gqa: S0 ~N(0, 0.02)].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

BF16 = torch.bfloat16
FP32 = torch.float32


@dataclass(frozen=True)
class Workload:
    name: str
    number: int            # 1..5; seed = 100 + number
    dtype: torch.dtype
    H: int
    Hk: int = 0
    K: int = 128
    V: int = 128
    B: int = 1
    T: int = 0
    n_seqs: int = 0        # varlen: number of packed sequences
    max_len: int = 0       # varlen: lengths uniform in [1, max_len]
    s0_std: float = 0.0    # initial state std (0 = zero state)
    # decode
    n: int = 0
    M: int = 0
    G: int = 0
    steps: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 100 + self.number


WORKLOADS = {
    "tiny": Workload("tiny", 1, FP32, H=2, Hk=2, K=64, V=64, B=1, T=128),
    "prefill": Workload("prefill", 2, BF16, H=16, Hk=16, K=128, V=128, B=4, T=4096),
    "gqa": Workload("gqa", 3, BF16, H=32, Hk=16, K=128, V=128, B=1, T=65536, s0_std=0.02),
    "varlen": Workload("varlen", 4, BF16, H=16, Hk=16, K=128, V=128, n_seqs=64, max_len=2048),
    "decode": Workload("decode", 5, BF16, H=32, G=16, K=128, V=128, n=256, M=2, steps=1000,
                       s0_std=0.02),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(gen, shape, std=1.0, mean=0.0):
    t = torch.randn(shape, generator=gen, dtype=FP32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t


def _log_uniform(gen, shape, lo, hi):
    """log of U[lo, hi] (the distribution of A_log)."""
    u = torch.rand(shape, generator=gen, dtype=FP32)
    return torch.log(lo + (hi - lo) * u)


def varlen_lengths(gen, n_seqs: int, max_len: int) -> torch.Tensor:
    return torch.randint(1, max_len + 1, (n_seqs,), generator=gen, dtype=torch.int64)


def cu_from_lengths(lengths) -> torch.Tensor:
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    return cu.to(torch.int32)


def prefill_inputs(w: Workload, *, T: int | None = None, B: int | None = None,
                   n_seqs: int | None = None, max_len: int | None = None,
                   lengths=None, seed: int | None = None) -> dict:
    """Inputs of the prefill chain (conv1d -> gates -> chunked forward).

    Sizes default to the workload's; the keyword overrides give smaller
    instances with the same distributions. Returns CPU tensors:
    x [B,T,C] (dtype), w [C,4] (dtype), a, b [B,T,H] (dtype), A_log, dt_bias
    [H] fp32, S0 [N,H,K,V] fp32 or None, cu_seqlens int32 [N+1] or None.
    """
    gen = _gen(w.seed if seed is None else seed)
    cu = None
    if w.n_seqs or lengths is not None or n_seqs is not None:
        if lengths is None:
            lengths = varlen_lengths(gen, n_seqs or w.n_seqs, max_len or w.max_len)
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
        cu = cu_from_lengths(lengths)
        B_ = 1
        T_ = int(lengths.sum())
        N = int(lengths.numel())
    else:
        B_ = B or w.B
        T_ = T or w.T
        N = B_
    C = 2 * w.Hk * w.K + w.H * w.V
    x = _normal(gen, (B_, T_, C))
    cw = _normal(gen, (C, 4), std=0.5)
    a = _normal(gen, (B_, T_, w.H))
    b = _normal(gen, (B_, T_, w.H))
    A_log = _log_uniform(gen, (w.H,), 1.0, 16.0)
    dt_bias = _normal(gen, (w.H,), std=0.1)
    S0 = _normal(gen, (N, w.H, w.K, w.V), std=w.s0_std) if w.s0_std > 0 else None
    return dict(x=x.to(w.dtype), w=cw.to(w.dtype), a=a.to(w.dtype), b=b.to(w.dtype),
                A_log=A_log, dt_bias=dt_bias, S0=S0, cu_seqlens=cu,
                B=B_, T=T_, N=N, C=C, H=w.H, Hk=w.Hk, K=w.K, V=w.V, dtype=w.dtype)


def device_prefill_inputs(w: Workload, dev, *, B: int | None = None, T: int | None = None,
                          lengths=None, seed: int | None = None) -> dict:
    """Inputs of the prefill chain drawn on the device, for sizes too large to
    draw on the host: the distributions of prefill_inputs (the same shapes,
    stds and draw order) from a seeded device generator, so the values are
    the device RNG's, not the host draws'. Packed batches take `lengths` (or
    the workload's length draw, made on the host first). Returns device
    tensors x, w, a, b, A_log, dt_bias, S0 (or None), cu_seqlens (or None)
    and the sizes B, T, N, C."""
    seed_ = w.seed if seed is None else seed
    cu = None
    if lengths is None and w.n_seqs:
        lengths = varlen_lengths(_gen(seed_), w.n_seqs, w.max_len)
    if lengths is not None:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
        cu = cu_from_lengths(lengths).to(dev)
        B_, T_, N = 1, int(lengths.sum()), int(lengths.numel())
    else:
        B_ = B or w.B
        T_ = T or w.T
        N = B_
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed_)
    C = 2 * w.Hk * w.K + w.H * w.V
    dt = w.dtype
    d = {"x": torch.randn((B_, T_, C), generator=gen, device=dev, dtype=dt),
         "w": (torch.randn((C, 4), generator=gen, device=dev) * 0.5).to(dt),
         "a": torch.randn((B_, T_, w.H), generator=gen, device=dev, dtype=dt),
         "b": torch.randn((B_, T_, w.H), generator=gen, device=dev, dtype=dt),
         "A_log": torch.log(1 + 15 * torch.rand(w.H, generator=gen, device=dev)),
         "dt_bias": torch.randn(w.H, generator=gen, device=dev) * 0.1}
    d["S0"] = (torch.randn((N, w.H, w.K, w.V), generator=gen, device=dev) * w.s0_std
               if w.s0_std > 0 else None)
    d.update(cu_seqlens=cu, B=B_, T=T_, N=N, C=C)
    return d


# Log-decay regimes for stage-level tests of the chunked forward, where g and
# beta are drawn directly: g = -U[0, gmax] (gmax = 0 means no decay), beta ~ U(0, 1).
DECAY_GMAX = {"strong": 12.0, "weak": 0.05, "none": 0.0}


def chunk_inputs(*, B: int, T: int, H: int, Hk: int, K: int, V: int, dtype=BF16,
                 decay: str = "strong", s0_std: float = 0.0, lengths=None,
                 seed: int = 7) -> dict:
    """Direct inputs of the chunked forward (no conv, no gate formula).

    q, k [B,T,Hk,K], v [B,T,H,V] ~N(0,1) in ``dtype``; g = -U[0, gmax] and
    beta ~U(0,1) [B,T,H] fp32; optional S0 ~N(0, s0_std) fp32 [N,H,K,V];
    optional packed lengths (then B must be 1 and T = sum(lengths)).
    """
    gen = _gen(seed)
    cu = None
    N = B
    if lengths is not None:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
        cu = cu_from_lengths(lengths)
        assert B == 1 and T == int(lengths.sum())
        N = int(lengths.numel())
    q = _normal(gen, (B, T, Hk, K))
    k = _normal(gen, (B, T, Hk, K))
    v = _normal(gen, (B, T, H, V))
    gmax = DECAY_GMAX[decay]
    g = -gmax * torch.rand((B, T, H), generator=gen, dtype=FP32)
    beta = torch.rand((B, T, H), generator=gen, dtype=FP32)
    S0 = _normal(gen, (N, H, K, V), std=s0_std) if s0_std > 0 else None
    return dict(q=q.to(dtype), k=k.to(dtype), v=v.to(dtype), g=g, beta=beta, S0=S0,
                cu_seqlens=cu, B=B, T=T, N=N, H=H, Hk=Hk, K=K, V=V, dtype=dtype)


def decode_state_inputs(w: Workload, *, n: int | None = None, seed: int | None = None) -> dict:
    """A_log [H], dt_bias [H] and the fp32 state [n, H, N, P] ~N(0, s0_std)."""
    gen = _gen(w.seed if seed is None else seed)
    n_ = n or w.n
    A_log = _log_uniform(gen, (w.H,), 1.0, 16.0)
    dt_bias = _normal(gen, (w.H,), std=0.1)
    state = _normal(gen, (n_, w.H, w.K, w.V), std=w.s0_std)
    return dict(A_log=A_log, dt_bias=dt_bias, state=state)


def decode_row_sizes(M: int, H: int, G: int, P: int, N: int) -> tuple[int, int]:
    """Lengths of the post-conv x row (v | k | q) and of the ba row (b | a)."""
    return M * H * P + M * G * N + G * N, M * H + H


def decode_step_inputs(w: Workload, step: int, *, n: int | None = None,
                       seed_base: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """x [n, M*H*P + M*G*N + G*N] and ba [n, M*H + H], both ~N(0,1) in the
    workload dtype; the generator is reseeded to seed*1000 + step."""
    n_ = n or w.n
    base = (w.seed * 1000) if seed_base is None else seed_base
    gen = _gen(base + step)
    xl, bl = decode_row_sizes(w.M, w.H, w.G, w.V, w.K)
    x = _normal(gen, (n_, xl))
    ba = _normal(gen, (n_, bl))
    return x.to(w.dtype), ba.to(w.dtype)


def integer_conv_inputs(*, B: int, T: int, C: int, dtype=BF16, lengths=None, seed: int = 11,
                        sentinel: float = 100.0) -> dict:
    """Integer-valued conv inputs for bit-exact checks: x in [-8, 8], w in
    {-2..2}; with packed lengths, the last 3 tokens of every sequence hold the
    sentinel +-100 so that a tap leaking across a boundary is large."""
    gen = _gen(seed)
    x = torch.randint(-8, 9, (B, T, C), generator=gen).to(FP32)
    w = torch.randint(-2, 3, (C, 4), generator=gen).to(FP32)
    cu = None
    if lengths is not None:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
        cu = cu_from_lengths(lengths)
        assert B == 1 and T == int(lengths.sum())
        sign = torch.randint(0, 2, (T, C), generator=gen).to(FP32) * 2 - 1
        ends = cu[1:].to(torch.int64)
        for e in ends.tolist():
            lo = max(0, e - 3)
            x[0, lo:e] = sentinel * sign[lo:e]
    return dict(x=x.to(dtype), w=w.to(dtype), cu_seqlens=cu, B=B, T=T, C=C)


def ragged_lengths(n: int, max_len: int, seed: int = 5) -> torch.Tensor:
    return varlen_lengths(_gen(seed), n, max_len)
