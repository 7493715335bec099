"""fp64 CPU oracle for the gated-delta-rule forward (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are its only users. The product path (the HIP library and its
Python binding) never imports it, and it imports nothing from them.

Each function takes numpy arrays (any float dtype; converted exactly to
float64) and returns float64 numpy arrays. The arithmetic lives in oracle.c;
this file only marshals arguments. Sources, cited by title and section:

* "ZzCompute" (PyTorch Helion Hackathon gallery): item 1 "Causal Conv1d",
  items 2-4 (Gated DeltaNet chunk forward H / O, recompute W/U).
* Megatron-Core API docs, "core.ssm.ops.gdp.decode_prepare": introduction,
  "softplus", "gdp_decode_prepare_kernel", "gdp_decode_prepare".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, IEEE semantics, OpenMP) into _build/."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off",
               "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_get_threads.restype = ctypes.c_int
        lib.oracle_conv1d_causal.argtypes = [_dp, _dp, _dp, _dp, _ip] + [ctypes.c_int] * 6
        lib.oracle_gate_prepare.argtypes = [_dp] * 6 + [ctypes.c_int] * 2
        lib.oracle_gated_delta_rule.argtypes = (
            [_dp] * 8 + [_ip] + [ctypes.c_int] * 7 + [ctypes.c_double, ctypes.c_int])
        lib.oracle_gdp_decode_prepare.argtypes = [_dp] * 9 + [ctypes.c_int] * 6
        lib.oracle_conv1d_update.argtypes = [_dp, _dp, _ip, _dp, _dp, _dp] + [ctypes.c_int] * 5
        lib.oracle_gdp_prefill.argtypes = ([_dp] * 6 + [_ip] + [ctypes.c_int] * 8
                                           + [ctypes.c_double, ctypes.c_int])
        lib.oracle_gdp_decode.argtypes = (
            [_dp] * 6 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int])
        _lib = lib
        return lib


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, None, 0
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    return cu, cu.ctypes.data_as(_ip), int(cu.shape[0] - 1)


def conv1d_causal(x, w, bias=None, cu_seqlens=None, silu=True):
    """y[b,t,c] = act(sum_j w[c,j] * x[b, t-(W-1)+j, c] (+ bias[c])), taps before
    the token's own sequence start read zero. x: [B,T,C]; w: [C,W]."""
    lib = _load()
    x = _f64(x)
    w = _f64(w)
    B, T, C = x.shape
    W = w.shape[1]
    assert w.shape == (C, W)
    b = None if bias is None else _f64(bias)
    cu, cup, ns = _cu(cu_seqlens)
    if cu is not None:
        assert B == 1 and cu[0] == 0 and cu[-1] == T
    y = np.empty_like(x)
    lib.oracle_conv1d_causal(_ptr(x), _ptr(w), _ptr(b), _ptr(y), cup, ns, B, T, C, W, int(bool(silu)))
    return y


def gate_prepare(a, b, A_log, dt_bias):
    """beta = sigmoid(b); g = -exp(A_log) * softplus(a + dt_bias). a, b: [..., H]."""
    lib = _load()
    a = _f64(a)
    b = _f64(b)
    shape = a.shape
    H = shape[-1]
    R = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    A_log = _f64(A_log)
    dt_bias = _f64(dt_bias)
    assert b.shape == shape and A_log.shape == (H,) and dt_bias.shape == (H,)
    g = np.empty(shape, np.float64)
    beta = np.empty(shape, np.float64)
    lib.oracle_gate_prepare(_ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta), R, H)
    return g, beta


def gated_delta_rule(q, k, v, g, beta, S0=None, cu_seqlens=None, scale=1.0, l2norm=True,
                     return_state=True):
    """Per-timestep gated delta rule. q, k: [B,T,Hk,K]; v: [B,T,H,V]; g, beta: [B,T,H];
    S0: [N,H,K,V] or None. Returns (o [B,T,H,V], S_final [N,H,K,V])."""
    lib = _load()
    q, k, v, g, beta = (_f64(t) for t in (q, k, v, g, beta))
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    assert k.shape == q.shape and v.shape[:2] == (B, T) and g.shape == (B, T, H)
    assert beta.shape == (B, T, H) and H % Hk == 0
    cu, cup, ns = _cu(cu_seqlens)
    N = ns if cu is not None else B
    if cu is not None:
        assert B == 1 and cu[0] == 0 and cu[-1] == T
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None:
        assert s0.shape == (N, H, K, V)
    o = np.empty((B, T, H, V), np.float64)
    sf = np.empty((N, H, K, V), np.float64) if return_state else None
    lib.oracle_gated_delta_rule(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                _ptr(o), _ptr(sf), cup, ns, B, T, H, Hk, K, V,
                                float(scale), int(bool(l2norm)))
    return o, sf


def gdp_decode_prepare(x, ba, A_log, dt_bias, M, H, G, P, N):
    """Split/gate one decode step: returns (q [n,M,H,N], k [n,M,H,N], v [n,M,H,P],
    beta [n,M,H], g [n,M,H])."""
    lib = _load()
    x = _f64(x)
    ba = _f64(ba)
    n = x.shape[0]
    assert x.shape == (n, M * H * P + M * G * N + G * N) and ba.shape == (n, M * H + H)
    A_log = _f64(A_log)
    dt_bias = _f64(dt_bias)
    qo = np.empty((n, M, H, N))
    ko = np.empty((n, M, H, N))
    vo = np.empty((n, M, H, P))
    bo = np.empty((n, M, H))
    go = np.empty((n, M, H))
    lib.oracle_gdp_decode_prepare(_ptr(x), _ptr(ba), _ptr(A_log), _ptr(dt_bias), _ptr(qo),
                                  _ptr(ko), _ptr(vo), _ptr(bo), _ptr(go), n, M, H, G, P, N)
    return qo, ko, vo, bo, go


def gdp_decode(x, ba, A_log, dt_bias, state, M, H, G, P, N, scale=1.0, l2norm=True):
    """One decode token for n requests. state: [n,H,N,P] (not modified; the
    updated state is returned). Returns (o [n,H,P], new_state [n,H,N,P])."""
    lib = _load()
    x = _f64(x)
    ba = _f64(ba)
    n = x.shape[0]
    assert x.shape == (n, M * H * P + M * G * N + G * N) and ba.shape == (n, M * H + H)
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    assert st.shape == (n, H, N, P)
    A_log = _f64(A_log)
    dt_bias = _f64(dt_bias)
    o = np.empty((n, H, P))
    lib.oracle_gdp_decode(_ptr(x), _ptr(ba), _ptr(A_log), _ptr(dt_bias), _ptr(st), _ptr(o),
                          n, M, H, G, P, N, float(scale), int(bool(l2norm)))
    return o, st


def conv1d_update(x, conv_state, slot, w, bias=None, silu=True):
    """One decode token's short conv per request. x: [n, C]; conv_state:
    [S, W-1, C] (not modified; the updated state is returned); slot: [n] ints
    (outside [0, S): zero output, no update). Returns (y [n, C], new_state)."""
    lib = _load()
    x = _f64(x)
    w = _f64(w)
    n, C = x.shape
    W = w.shape[1]
    st = np.array(conv_state, dtype=np.float64, order="C", copy=True)
    assert st.shape[1:] == (W - 1, C) and w.shape == (C, W)
    sl = np.ascontiguousarray(np.asarray(slot, dtype=np.int32))
    assert sl.shape == (n,)
    b = None if bias is None else _f64(bias)
    y = np.empty((n, C), np.float64)
    lib.oracle_conv1d_update(_ptr(x), _ptr(st), sl.ctypes.data_as(_ip), _ptr(w), _ptr(b), _ptr(y),
                             n, st.shape[0], C, W, int(bool(silu)))
    return y, st


def gdp_prefill(x, ba, A_log, dt_bias, M, H, G, P, N, S0=None, cu_seqlens=None, scale=1.0,
                l2norm=True):
    """Gated DeltaProduct prefill, token by token. x: [B, T, row]; ba: [B, T, M*H+H];
    S0: [N_seq, H, N, P] or None. Returns (o [B, T, H, P], S_final)."""
    lib = _load()
    x = _f64(x)
    ba = _f64(ba)
    B, T, row = x.shape
    assert row == M * H * P + M * G * N + G * N and ba.shape == (B, T, M * H + H)
    cu, cup, ns = _cu(cu_seqlens)
    nseq = ns if cu is not None else B
    if cu is not None:
        assert B == 1 and cu[0] == 0 and cu[-1] == T
    st = np.zeros((nseq, H, N, P)) if S0 is None else np.array(S0, dtype=np.float64, order="C", copy=True)
    assert st.shape == (nseq, H, N, P)
    o = np.empty((B, T, H, P), np.float64)
    lib.oracle_gdp_prefill(_ptr(x), _ptr(ba), _ptr(_f64(A_log)), _ptr(_f64(dt_bias)), _ptr(st),
                           _ptr(o), cup, ns, B, T, M, H, G, P, N, float(scale), int(bool(l2norm)))
    return o, st
