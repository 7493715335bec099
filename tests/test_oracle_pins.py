"""Pins of the fp64 oracle to facts outside the oracle itself.

Each test checks the oracle against something it does not share code with:
a library routine (numpy convolution, scipy's logistic function, a dense
linear solve), a closed form that follows from the recurrence, a worked
example derived by hand, brute force with explicit transition matrices, or a
value/shape the pages print (fixtures under tests/golden/). They are chosen
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.
"""
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests import chunk_form

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ------------------------------------------------------------------ conv1d

def test_conv_equals_numpy_causal_convolution():
    B, T, C, W = 2, 37, 5, 4
    x = RNG.standard_normal((B, T, C))
    w = RNG.standard_normal((C, W))
    y = oracle.conv1d_causal(x, w, silu=False)
    for b in range(B):
        for c in range(C):
            # np.convolve is the full convolution; its first T outputs are the causal
            # filter with x = 0 before t = 0. Reversing w makes w[W-1] the tap on x_t.
            ref = np.convolve(x[b, :, c], w[c, ::-1])[:T]
            np.testing.assert_allclose(y[b, :, c], ref, rtol=0, atol=1e-13)


def test_conv_impulse_response_and_tap_order():
    T, C, W = 12, 3, 4
    w = RNG.standard_normal((C, W))
    x = np.zeros((1, T, C))
    t0 = 5
    x[0, t0, 1] = 1.0
    y = oracle.conv1d_causal(x, w, silu=False)
    expect = np.zeros((T, C))
    for j in range(W):
        expect[t0 + j, 1] = w[1, W - 1 - j]
    np.testing.assert_array_equal(y[0], expect)


def test_conv_zero_padding_at_sequence_start():
    # x = 1 everywhere: y_t = sum of the taps that fall inside the sequence.
    T, C, W = 6, 2, 4
    w = np.array([[1.0, 10.0, 100.0, 1000.0], [2.0, 3.0, 5.0, 7.0]])
    y = oracle.conv1d_causal(np.ones((1, T, C)), w, silu=False)
    np.testing.assert_array_equal(y[0, :, 0], [1000, 1100, 1110, 1111, 1111, 1111])
    np.testing.assert_array_equal(y[0, :, 1], [7, 12, 15, 17, 17, 17])


def test_conv_silu_and_bias():
    B, T, C, W = 1, 20, 4, 4
    x = RNG.standard_normal((B, T, C)) * 3
    w = RNG.standard_normal((C, W))
    bias = RNG.standard_normal(C)
    z = oracle.conv1d_causal(x, w, silu=False) + bias
    y = oracle.conv1d_causal(x, w, bias=bias, silu=True)
    np.testing.assert_allclose(y, z * expit(z), rtol=1e-14, atol=1e-15)


def test_conv_varlen_is_per_sequence_conv():
    lengths = [1, 5, 2, 9, 1, 4]
    T, C, W = sum(lengths), 3, 4
    x = RNG.standard_normal((1, T, C))
    w = RNG.standard_normal((C, W))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    y = oracle.conv1d_causal(x, w, cu_seqlens=cu, silu=True)
    for i in range(len(lengths)):
        s, e = cu[i], cu[i + 1]
        ys = oracle.conv1d_causal(x[:, s:e], w, silu=True)
        np.testing.assert_array_equal(y[:, s:e], ys)


# ------------------------------------------------------------------- gates

def _golden_softplus():
    rows = []
    with open(os.path.join(GOLDEN, "softplus_threshold.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or line.split()[0] in ("threshold", "beta"):
                continue
            xs, ys = line.split()
            rows.append((float(xs), float(ys)))
    return rows


def test_softplus_golden_points_through_gate():
    # g = -exp(A_log) * softplus(a + dt_bias); with A_log = 0 and dt_bias = 0, g = -softplus(a).
    pts = _golden_softplus()
    a = np.array([[p[0] for p in pts]])
    H = a.shape[1]
    g, beta = oracle.gate_prepare(a, np.zeros_like(a), np.zeros(H), np.zeros(H))
    for (x, sp), gv in zip(pts, g[0]):
        assert -gv == pytest.approx(sp, rel=1e-15, abs=0), x
    np.testing.assert_array_equal(beta, 0.5)


def test_gates_against_library_functions():
    R, H = 50, 7
    a = RNG.standard_normal((R, H)) * 15
    b = RNG.standard_normal((R, H)) * 6
    A_log = np.log(RNG.uniform(1, 16, H))
    dt_bias = RNG.normal(0, 0.1, H)
    g, beta = oracle.gate_prepare(a, b, A_log, dt_bias)
    x = a + dt_bias
    sp = np.where(x > 20, x, np.logaddexp(0.0, x))
    np.testing.assert_allclose(beta, expit(b), rtol=1e-15)
    np.testing.assert_allclose(g, -np.exp(A_log) * sp, rtol=1e-14)
    assert (g <= 0).all() and (beta > 0).all() and (beta < 1).all()


def test_gate_extremes():
    a = np.array([[-745.0, -100.0, 25.0, 1e4]])
    b = np.array([[-800.0, 800.0, 0.0, -30.0]])
    g, beta = oracle.gate_prepare(a, b, np.zeros(4), np.zeros(4))
    assert np.isfinite(g).all() and np.isfinite(beta).all()
    assert beta[0, 0] == 0.0 and beta[0, 1] == 1.0
    assert g[0, 2] == -25.0 and g[0, 3] == -1e4
    assert g[0, 0] <= 0.0


# -------------------------------------------------------------- recurrence

def _run(q, k, v, g, beta, S0=None, **kw):
    return oracle.gated_delta_rule(q[None], k[None], v[None], g[None], beta[None],
                                   None if S0 is None else S0[None, None], **kw)


def test_hand_worked_example():
    # K = V = 2, S0 = 0, no normalisation. Derived by hand with
    # S_t = a_t S (I - b_t k k^T) + b_t v k^T (S is V x K), o_t = S_t q_t:
    # t1: k=e1, v=(2,4), b=1/2, a=1/2 -> S=[[1,0],[2,0]], q=e1 -> o=(1,2)
    # t2: k=e2, v=(6,2), b=1,   a=1   -> S=[[1,6],[2,2]], q=(1,1) -> o=(7,4)
    # t3: k=e1, v=(3,3), b=1/2, a=1/2 -> S k=(1,2); S(I-kk^T/2)=[[.5,6],[1,2]];
    #     x a -> [[.25,3],[.5,1]]; + v k^T/2 -> S=[[1.75,3],[2,1]], q=e2 -> o=(3,1)
    k = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 0.0]])[:, None, :]
    q = np.array([[1.0, 0.0], [1.0, 1.0], [0.0, 1.0]])[:, None, :]
    v = np.array([[2.0, 4.0], [6.0, 2.0], [3.0, 3.0]])[:, None, :]
    g = np.log(np.array([[0.5], [1.0], [0.5]]))
    beta = np.array([[0.5], [1.0], [0.5]])
    o, sf = _run(q, k, v, g, beta, l2norm=False)
    np.testing.assert_allclose(o[0, :, 0], [[1, 2], [7, 4], [3, 1]], rtol=0, atol=1e-15)
    # the stored final state is the K x V transpose of S
    np.testing.assert_allclose(sf[0, 0], np.array([[1.75, 3.0], [2.0, 1.0]]).T, atol=1e-15)


@pytest.mark.parametrize("K,V", [(8, 8), (6, 10), (12, 5)])
def test_pure_decay_when_beta_zero(K, V):
    # beta = 0: S_t = alpha_t S_{t-1}, so o_t = gamma_t S0 q_t with gamma_t = exp(sum g).
    T = 9
    q = RNG.standard_normal((T, 1, K))
    k = RNG.standard_normal((T, 1, K))
    v = RNG.standard_normal((T, 1, V))
    g = -RNG.uniform(0, 0.7, (T, 1))
    S0 = RNG.standard_normal((K, V))     # stored K x V
    o, sf = _run(q, k, v, g, np.zeros((T, 1)), S0, l2norm=False)
    gam = np.exp(np.cumsum(g[:, 0]))
    expect = gam[:, None] * (q[:, 0, :] @ S0)      # (S q) with S = S0^T
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sf[0, 0], gam[-1] * S0, rtol=1e-13)


def test_no_decay_no_write_keeps_initial_state():
    K, V, T = 7, 5, 6
    q = RNG.standard_normal((T, 1, K))
    S0 = RNG.standard_normal((K, V))
    o, sf = _run(q, RNG.standard_normal((T, 1, K)), RNG.standard_normal((T, 1, V)),
                 np.zeros((T, 1)), np.zeros((T, 1)), S0, l2norm=False)
    np.testing.assert_allclose(o[0, :, 0], q[:, 0, :] @ S0, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(sf[0, 0], S0)


@pytest.mark.parametrize("decay", [False, True])
def test_orthonormal_keys_give_gated_linear_attention(decay):
    # With orthonormal keys the erase term S_{t-1} k_t vanishes, so from S0 = 0:
    # o_t = sum_{s<=t} (gamma_t / gamma_s) beta_s (k_s . q_t) v_s.
    K, V, T = 16, 6, 12
    Qm, _ = np.linalg.qr(RNG.standard_normal((K, K)))
    k = Qm[:T][:, None, :]
    q = RNG.standard_normal((T, 1, K))
    v = RNG.standard_normal((T, 1, V))
    g = -RNG.uniform(0, 1.0, (T, 1)) if decay else np.zeros((T, 1))
    beta = RNG.uniform(0.1, 1.0, (T, 1))
    o, _ = _run(q, k, v, g, beta, l2norm=False)
    G = np.cumsum(g[:, 0])
    expect = np.zeros((T, V))
    for t in range(T):
        for s in range(t + 1):
            expect[t] += np.exp(G[t] - G[s]) * beta[s, 0] * (k[s, 0] @ q[t, 0]) * v[s, 0]
    np.testing.assert_allclose(o[0, :, 0], expect, rtol=1e-12, atol=1e-13)


def test_one_step_from_zero_state():
    # o_1 = beta_1 (k_1 . q_1) v_1 (alpha does not matter from S = 0).
    K, V = 9, 4
    q, k = RNG.standard_normal((1, 1, K)), RNG.standard_normal((1, 1, K))
    v = RNG.standard_normal((1, 1, V))
    o, _ = _run(q, k, v, np.array([[-0.3]]), np.array([[0.6]]), l2norm=False, scale=0.25)
    np.testing.assert_allclose(o[0, 0, 0], 0.25 * 0.6 * (k[0, 0] @ q[0, 0]) * v[0, 0], rtol=1e-14)


@pytest.mark.parametrize("K,V,T", [(4, 4, 8), (3, 5, 7), (6, 2, 8)])
def test_brute_force_transition_products(K, V, T):
    # Unrolled form in the K x V orientation h = S^T:
    #   h_t = M_t h_{t-1} + beta_t k_t v_t^T,   M_t = alpha_t (I - beta_t k_t k_t^T)
    #   h_T = (M_T...M_1) h_0 + sum_t (M_T...M_{t+1}) beta_t k_t v_t^T,  o_t = h_t^T q_t.
    q = RNG.standard_normal((T, 1, K))
    k = _unit(RNG.standard_normal((T, 1, K)))
    v = RNG.standard_normal((T, 1, V))
    g = -RNG.uniform(0, 1.2, (T, 1))
    beta = RNG.uniform(0, 1, (T, 1))
    h0 = RNG.standard_normal((K, V))
    o, sf = _run(q, k, v, g, beta, h0, l2norm=False)
    Ms = [np.exp(g[t, 0]) * (np.eye(K) - beta[t, 0] * np.outer(k[t, 0], k[t, 0])) for t in range(T)]
    for tt in range(1, T + 1):
        P = np.eye(K)
        for t in range(tt):
            P = Ms[t] @ P
        h = P @ h0
        for t in range(tt):
            R = np.eye(K)
            for s in range(t + 1, tt):
                R = Ms[s] @ R
            h = h + R @ (beta[t, 0] * np.outer(k[t, 0], v[t, 0]))
        np.testing.assert_allclose(o[0, tt - 1, 0], h.T @ q[tt - 1, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sf[0, 0], h, rtol=1e-11, atol=1e-12)


def test_l2_normalisation_is_applied():
    # o is invariant to positive rescaling of q_t and k_t (up to the eps) when l2norm is on,
    # and equals the un-normalised run on pre-normalised inputs.
    K, V, T = 8, 3, 10
    q = RNG.standard_normal((T, 1, K))
    k = RNG.standard_normal((T, 1, K))
    v = RNG.standard_normal((T, 1, V))
    g = -RNG.uniform(0, 0.5, (T, 1))
    beta = RNG.uniform(0, 1, (T, 1))
    o1, _ = _run(q, k, v, g, beta)
    o2, _ = _run(q * 7.0, k * 0.5, v, g, beta)
    np.testing.assert_allclose(o1, o2, rtol=1e-5, atol=1e-6)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    o3, _ = _run(qn, kn, v, g, beta, l2norm=False)
    np.testing.assert_allclose(o1, o3, rtol=1e-13, atol=1e-14)


def test_gqa_head_map_equals_explicit_repeat():
    # value head h reads q/k head h // (H / Hk): consecutive value heads share a group.
    B, T, H, Hk, K, V = 2, 9, 6, 2, 5, 3
    q = RNG.standard_normal((B, T, Hk, K))
    k = RNG.standard_normal((B, T, Hk, K))
    v = RNG.standard_normal((B, T, H, V))
    g = -RNG.uniform(0, 1, (B, T, H))
    beta = RNG.uniform(0, 1, (B, T, H))
    o, sf = oracle.gated_delta_rule(q, k, v, g, beta)
    rep = H // Hk
    o2, sf2 = oracle.gated_delta_rule(np.repeat(q, rep, axis=2), np.repeat(k, rep, axis=2),
                                      v, g, beta)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(sf, sf2)


def test_varlen_resets_state_per_sequence():
    lengths = [3, 1, 8, 5]
    T, H, K, V = sum(lengths), 2, 4, 3
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q = RNG.standard_normal((1, T, H, K))
    k = RNG.standard_normal((1, T, H, K))
    v = RNG.standard_normal((1, T, H, V))
    g = -RNG.uniform(0, 1, (1, T, H))
    beta = RNG.uniform(0, 1, (1, T, H))
    S0 = RNG.standard_normal((len(lengths), H, K, V))
    o, sf = oracle.gated_delta_rule(q, k, v, g, beta, S0=S0, cu_seqlens=cu)
    for i in range(len(lengths)):
        s, e = cu[i], cu[i + 1]
        oi, sfi = oracle.gated_delta_rule(q[:, s:e], k[:, s:e], v[:, s:e], g[:, s:e],
                                          beta[:, s:e], S0=S0[i:i + 1])
        np.testing.assert_array_equal(o[:, s:e], oi)
        np.testing.assert_array_equal(sf[i], sfi[0])


@pytest.mark.parametrize("T,chunk", [(1, 64), (63, 64), (65, 64), (200, 64), (130, 16)])
def test_chunked_form_equals_recurrence(T, chunk):
    # The chunked equations the GPU path evaluates reproduce the timestep loop.
    B, H, Hk, K, V = 1, 2, 1, 16, 12
    q = RNG.standard_normal((B, T, Hk, K))
    k = RNG.standard_normal((B, T, Hk, K))
    v = RNG.standard_normal((B, T, H, V))
    g = -RNG.uniform(0, 3.0, (B, T, H))
    beta = RNG.uniform(0, 1, (B, T, H))
    S0 = RNG.standard_normal((B, H, K, V)) * 0.1
    o, sf = oracle.gated_delta_rule(q, k, v, g, beta, S0=S0, scale=0.5)
    oc, sfc = chunk_form.chunked_gated_delta_rule(q, k, v, g, beta, S0=S0, scale=0.5,
                                                  chunk=chunk)
    scale_o = np.abs(o).max()
    assert np.abs(o - oc).max() <= 1e-12 * max(1.0, scale_o)
    assert np.abs(sf - sfc).max() <= 1e-12 * max(1.0, np.abs(sf).max())


def test_chunked_form_varlen():
    lengths = [70, 1, 64, 129]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, K, V = 2, 8, 8
    q = RNG.standard_normal((1, T, H, K))
    k = RNG.standard_normal((1, T, H, K))
    v = RNG.standard_normal((1, T, H, V))
    g = -RNG.uniform(0, 0.2, (1, T, H))
    beta = RNG.uniform(0, 1, (1, T, H))
    o, sf = oracle.gated_delta_rule(q, k, v, g, beta, cu_seqlens=cu)
    oc, sfc = chunk_form.chunked_gated_delta_rule(q, k, v, g, beta, cu_seqlens=cu)
    assert np.abs(o - oc).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(sf - sfc).max() <= 1e-12 * np.abs(sf).max()


# ------------------------------------------------------------------ decode

def _golden_layout():
    rows = {}
    with open(os.path.join(GOLDEN, "gdp_layout.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            p = line.split()
            rows[p[0]] = dict(zip(["n", "M", "H", "G", "P", "N", "x_row", "ba_row", "k_base",
                                   "q_base", "hpg"], map(int, p[1:])))
    return rows


def test_decode_layout_golden_and_prepare_split():
    import workloads
    for name, r in _golden_layout().items():
        n, M, H, G, P, N = r["n"], r["M"], r["H"], r["G"], r["P"], r["N"]
        assert workloads.decode_row_sizes(M, H, G, P, N) == (r["x_row"], r["ba_row"])
        if name != "small":
            continue
        x = RNG.standard_normal((n, r["x_row"]))
        ba = RNG.standard_normal((n, r["ba_row"]))
        A_log, dt_bias = np.log(RNG.uniform(1, 16, H)), RNG.normal(0, 0.1, H)
        q, k, v, beta, g = oracle.gdp_decode_prepare(x, ba, A_log, dt_bias, M, H, G, P, N)
        assert q.shape == (n, M, H, N) and k.shape == (n, M, H, N) and v.shape == (n, M, H, P)
        assert beta.shape == (n, M, H) and g.shape == (n, M, H)
        for m in range(M):
            for h in range(H):
                grp = h // r["hpg"]
                # plain copies of the row segments
                np.testing.assert_array_equal(v[:, m, h], x[:, (m * H + h) * P:(m * H + h + 1) * P])
                kb = r["k_base"] + (m * G + grp) * N
                np.testing.assert_array_equal(k[:, m, h], x[:, kb:kb + N])
                qb = r["q_base"] + grp * N
                if m == M - 1:      # query only on the last copy
                    np.testing.assert_array_equal(q[:, m, h], x[:, qb:qb + N])
                else:
                    assert (q[:, m, h] == 0).all()
                np.testing.assert_allclose(beta[:, m, h], expit(ba[:, m * H + h]), rtol=1e-15)
                if m == 0:          # the decay only on the first copy
                    xa = ba[:, M * H + h] + dt_bias[h]
                    sp = np.where(xa > 20, xa, np.logaddexp(0, xa))
                    np.testing.assert_allclose(g[:, 0, h], -np.exp(A_log[h]) * sp, rtol=1e-14)
                else:
                    assert (g[:, m, h] == 0).all()


def _decode_case(n, M, H, G, P, N, seed=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, M * H * P + M * G * N + G * N))
    ba = rng.standard_normal((n, M * H + H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt_bias = rng.normal(0, 0.1, H)
    st = rng.standard_normal((n, H, N, P)) * 0.1
    return x, ba, A_log, dt_bias, st


def test_decode_one_copy_from_zero_state():
    n, M, H, G, P, N = 3, 1, 4, 2, 5, 6
    x, ba, A_log, dt_bias, _ = _decode_case(n, M, H, G, P, N)
    o, st = oracle.gdp_decode(x, ba, A_log, dt_bias, np.zeros((n, H, N, P)), M, H, G, P, N,
                              l2norm=True)
    for r in range(n):
        for h in range(H):
            grp = h // (H // G)
            v = x[r, h * P:(h + 1) * P]
            k = x[r, H * P + grp * N: H * P + (grp + 1) * N]
            q = x[r, H * P + G * N + grp * N: H * P + G * N + (grp + 1) * N]
            kn = k / np.sqrt(k @ k + 1e-6)
            qn = q / np.sqrt(q @ q + 1e-6)
            b = expit(ba[r, h])
            np.testing.assert_allclose(o[r, h], b * (kn @ qn) * v, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(st[r, h], b * np.outer(kn, v), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("M", [2, 3])
def test_decode_brute_force(M):
    # Explicit K x K transitions over the M copies: decay only on copy 0, query on copy M-1.
    n, H, G, P, N = 2, 4, 2, 3, 5
    x, ba, A_log, dt_bias, st0 = _decode_case(n, M, H, G, P, N, seed=M)
    o, st = oracle.gdp_decode(x, ba, A_log, dt_bias, st0, M, H, G, P, N, scale=0.7)
    for r in range(n):
        for h in range(H):
            grp = h // (H // G)
            hmat = st0[r, h].copy()                   # N x P
            xa = ba[r, M * H + h] + dt_bias[h]
            alpha = np.exp(-np.exp(A_log[h]) * (xa if xa > 20 else np.log1p(np.exp(xa))))
            for m in range(M):
                kk = x[r, M * H * P + (m * G + grp) * N:M * H * P + (m * G + grp + 1) * N]
                kn = kk / np.sqrt(kk @ kk + 1e-6)
                vv = x[r, (m * H + h) * P:(m * H + h + 1) * P]
                b = expit(ba[r, m * H + h])
                a = alpha if m == 0 else 1.0
                hmat = a * (np.eye(N) - b * np.outer(kn, kn)) @ hmat + b * np.outer(kn, vv)
            qq = x[r, M * H * P + M * G * N + grp * N:M * H * P + M * G * N + (grp + 1) * N]
            qn = qq / np.sqrt(qq @ qq + 1e-6)
            np.testing.assert_allclose(o[r, h], 0.7 * hmat.T @ qn, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(st[r, h], hmat, rtol=1e-12, atol=1e-14)


def test_decode_second_copy_with_zero_beta_equals_one_copy():
    n, H, G, P, N = 3, 4, 4, 6, 6
    x2, ba2, A_log, dt_bias, st0 = _decode_case(n, 2, H, G, P, N)
    ba2[:, H:2 * H] = -np.inf        # beta of copy 1 = sigmoid(-inf) = 0 exactly
    o2, s2 = oracle.gdp_decode(x2, ba2, A_log, dt_bias, st0, 2, H, G, P, N)
    # the equivalent single-copy row: v and k of copy 0, the shared query; a unchanged
    x1 = np.concatenate([x2[:, :H * P], x2[:, 2 * H * P:2 * H * P + G * N],
                         x2[:, 2 * H * P + 2 * G * N:]], axis=1)
    ba1 = np.concatenate([ba2[:, :H], ba2[:, 2 * H:]], axis=1)
    o1, s1 = oracle.gdp_decode(x1, ba1, A_log, dt_bias, st0, 1, H, G, P, N)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s2, s1, rtol=1e-13, atol=1e-15)


# --------------------------------------------------- decode short-conv update

def test_conv_update_token_by_token_equals_prefill_conv():
    # Fed one token at a time from a zero window, the update is the prefill
    # convolution (same taps, zero padding at the start), here with a bias.
    rng = np.random.default_rng(11)
    T, C, W = 9, 12, 4
    x = rng.standard_normal((1, T, C))
    w = rng.standard_normal((C, W))
    bias = rng.standard_normal(C)
    ref = oracle.conv1d_causal(x, w, bias=bias, silu=True)[0]
    st = np.zeros((2, W - 1, C))
    for t in range(T):
        y, st = oracle.conv1d_update(x[0, t:t + 1], st, [1], w, bias=bias, silu=True)
        np.testing.assert_allclose(y[0], ref[t], rtol=1e-14, atol=1e-15)
    assert (st[0] == 0).all()                               # the other slot is untouched
    np.testing.assert_array_equal(st[1], x[0, T - (W - 1):])  # the window holds the last W-1 inputs


def test_conv_update_window_is_the_last_inputs_and_padding_zeroes():
    # Hand example, W = 4, one channel: y = w0 s0 + w1 s1 + w2 s2 + w3 x.
    w = np.array([[2.0, -1.0, 3.0, 0.5]])
    st = np.array([[[1.0], [2.0], [-4.0]], [[7.0], [8.0], [9.0]]])   # slots 0, 1
    y, st2 = oracle.conv1d_update(np.array([[6.0], [5.0]]), st, [0, -1], w, silu=False)
    assert y[0, 0] == 2 * 1 - 1 * 2 + 3 * (-4) + 0.5 * 6      # = -9
    assert y[1, 0] == 0.0                                   # padding request: zero row
    np.testing.assert_array_equal(st2[0, :, 0], [2.0, -4.0, 6.0])
    np.testing.assert_array_equal(st2[1], st[1])            # padding leaves every slot alone
    ys, _ = oracle.conv1d_update(np.array([[6.0]]), st, [0], w, silu=True)
    assert ys[0, 0] == pytest.approx(-9.0 / (1.0 + np.exp(9.0)), rel=1e-15)


# ------------------------------------------------ Gated DeltaProduct prefill

def _gdp_prefill_case(B, T, M, H, G, P, N, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, M * H * P + M * G * N + G * N))
    ba = rng.standard_normal((B, T, M * H + H))
    A_log = np.log(rng.uniform(1, 16, H))
    dt_bias = rng.normal(0, 0.1, H)
    S0 = rng.standard_normal((B, H, N, P)) * 0.05
    return x, ba, A_log, dt_bias, S0


def _interleave(x, ba, A_log, dt_bias, M, H, G, P, N):
    """The M*T-position sequence of the GDP prefill, built by explicit indexing
    (row t*M + m = copy m of token t; query on copy M-1, decay on copy 0)."""
    B, T, _ = x.shape
    q = np.zeros((B, M * T, G, N)); k = np.zeros((B, M * T, G, N)); v = np.zeros((B, M * T, H, P))
    g = np.zeros((B, M * T, H)); beta = np.zeros((B, M * T, H))
    kb, qb = M * H * P, M * H * P + M * G * N
    for t in range(T):
        for m in range(M):
            p = t * M + m
            v[:, p] = x[:, t, m * H * P:(m + 1) * H * P].reshape(B, H, P)
            k[:, p] = x[:, t, kb + m * G * N:kb + (m + 1) * G * N].reshape(B, G, N)
            if m == M - 1:
                q[:, p] = x[:, t, qb:qb + G * N].reshape(B, G, N)
            beta[:, p] = expit(ba[:, t, m * H:(m + 1) * H])
            if m == 0:
                xa = ba[:, t, M * H:] + dt_bias
                g[:, p] = -np.exp(A_log) * np.where(xa > 20, xa, np.logaddexp(0, xa))
    return q, k, v, g, beta


@pytest.mark.parametrize("M", [1, 2, 3])
def test_gdp_prefill_equals_recurrence_over_interleaved_sequence(M):
    # The token-by-token GDP layer is the gated delta rule (pinned above by
    # closed forms and brute force) over the interleaved M*T sequence, with
    # token t's output at position t*M + M-1 and the same final state.
    B, T, H, G, P, N = 2, 7, 4, 2, 5, 6
    x, ba, A_log, dt_bias, S0 = _gdp_prefill_case(B, T, M, H, G, P, N, seed=20 + M)
    o, sf = oracle.gdp_prefill(x, ba, A_log, dt_bias, M, H, G, P, N, S0=S0, scale=0.8)
    q, k, v, g, beta = _interleave(x, ba, A_log, dt_bias, M, H, G, P, N)
    o2, sf2 = oracle.gated_delta_rule(q, k, v, g, beta, S0=S0, scale=0.8)
    np.testing.assert_allclose(o, o2[:, M - 1::M], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sf, sf2, rtol=1e-12, atol=1e-14)
    # positions before the last copy carry a zero query: exactly zero output
    for m in range(M - 1):
        assert (o2[:, m::M] == 0).all()


def test_gdp_prefill_packed_sequences_reset_state():
    M, H, G, P, N = 2, 2, 1, 4, 4
    cu = [0, 3, 8]
    x, ba, A_log, dt_bias, _ = _gdp_prefill_case(1, 8, M, H, G, P, N, seed=31)
    o, sf = oracle.gdp_prefill(x, ba, A_log, dt_bias, M, H, G, P, N, cu_seqlens=cu)
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        o1, sf1 = oracle.gdp_prefill(x[:, a:b], ba[:, a:b], A_log, dt_bias, M, H, G, P, N)
        np.testing.assert_allclose(o[:, a:b], o1, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(sf[s], sf1[0], rtol=1e-13, atol=1e-15)


def test_softplus_golden_file_is_reproducible():
    # the fixture is written by a committed script (120-digit decimal
    # arithmetic, no floating-point library); re-running it gives the same bytes
    import subprocess
    import sys
    script = os.path.join(GOLDEN, "make_softplus_threshold.py")
    r = subprocess.run([sys.executable, script, "--check"], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_no_decay_gates_are_exact():
    # A_log = -inf gives g = -exp(-inf) * softplus(.) = -0 exactly: the
    # no-decay cases of the long-sequence parity tests rely on it
    g, beta = oracle.gate_prepare(np.array([[0.3, -5.0, 25.0]]), np.zeros((1, 3)),
                                  np.full(3, -np.inf), np.zeros(3))
    assert np.all(g == 0.0) and np.all(np.isfinite(g))
