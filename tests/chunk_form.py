"""Test-only fp64 numpy prototype of the chunked gated delta rule.

The "ZzCompute" entry (PyTorch Helion Hackathon gallery) evaluates the gated
delta rule in 64-step chunks: a WY recompute of the keys/values (item 4), a
sequential inter-chunk state scan (item 2) and a per-chunk output (item 3).
Its equations are cited there by number only, so they are derived here from
the per-timestep recurrence; the derivation is pinned by checking this
prototype against the oracle's timestep loop.

Per chunk (positions r = 1..L, entering state h of shape K x V, G_r the
inclusive cumulative sum of g inside the chunk, gamma_r = exp(G_r),
Gamma_rs = exp(G_r - G_s) for s <= r, 0 otherwise):

    A    = strict_lower(diag(beta) (K K^T o Gamma))
    T    = (I + A)^-1 diag(beta)
    U    = T (V - diag(gamma) K h)                 (the corrected values)
    O    = scale * (diag(gamma) Q h + (Q K^T o Gamma) U)
    h'   = gamma_L h + (diag(gamma_L / gamma) K)^T U

This is test infrastructure; it shares nothing with the HIP library.
"""
from __future__ import annotations

import numpy as np


def _l2(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


def chunk_step(h, Kc, Qc, Vc, gc, bc, scale=1.0):
    """One chunk. Kc, Qc: [L, K]; Vc: [L, V]; gc, bc: [L]; h: [K, V].
    Returns (O [L, V], h_next [K, V], T [L, L])."""
    L = Kc.shape[0]
    G = np.cumsum(gc)
    diff = G[:, None] - G[None, :]
    lower_incl = np.tril(np.ones((L, L), dtype=bool))
    Gam = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
    A = np.tril(bc[:, None] * (Kc @ Kc.T) * Gam, -1)
    T = np.linalg.solve(np.eye(L) + A, np.diag(bc))
    gam = np.exp(G)
    U = T @ (Vc - gam[:, None] * (Kc @ h))
    O = scale * (gam[:, None] * (Qc @ h) + ((Qc @ Kc.T) * Gam) @ U)
    d = np.exp(G[-1] - G)
    h_next = gam[-1] * h + (d[:, None] * Kc).T @ U
    return O, h_next, T


def chunked_gated_delta_rule(q, k, v, g, beta, S0=None, cu_seqlens=None, scale=1.0,
                             l2norm=True, chunk=64):
    """Same signature and layouts as the oracle's gated_delta_rule."""
    q, k, v, g, beta = (np.asarray(t, np.float64) for t in (q, k, v, g, beta))
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    grp = H // Hk
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, np.int64)
        spans = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    else:
        spans = [(b, 0, T) for b in range(B)]
    N = len(spans)
    o = np.zeros((B, T, H, V))
    sf = np.zeros((N, H, K, V))
    if l2norm:
        q = _l2(q)
        k = _l2(k)
    for n, (b, t0, t1) in enumerate(spans):
        for h in range(H):
            hk = h // grp
            st = np.zeros((K, V)) if S0 is None else np.array(S0[n, h], np.float64)
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                O, st, _ = chunk_step(st, k[b, c0:c1, hk], q[b, c0:c1, hk], v[b, c0:c1, h],
                                      g[b, c0:c1, h], beta[b, c0:c1, h], scale)
                o[b, c0:c1, h] = O
            sf[n, h] = st
    return o, sf
