"""The C-ABI boundary, without a GPU: the library loads, exports every entry
point that include/gdn.h declares, and rejects bad arguments with the
documented status codes (validation runs before any HIP call, so these calls
never touch a device; the pointers below are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "linear_attention_ssm_amd", "libgdn.so")

OK, EINVAL, EUNSUP, EWS, ELAUNCH = 0, 1, 2, 3, 4
FP32, BF16 = 0, 1
P = 0x10000          # fake, 16-byte aligned "device" addresses (never dereferenced)
P2 = 0x20000
P3 = 0x30000
P4 = 0x40000
P5 = 0x50000
P6 = 0x60000
WS = 0x100000        # 256-byte aligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libgdn.so is not built (run `python linear_attention_ssm_amd/build.py`)")
    L = ctypes.CDLL(LIB)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.gdn_status_string.argtypes = [i32]
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_conv1d_causal.argtypes = [vp, i64, i64, vp, vp, vp, i64, i64, vp, i32] + [i32] * 6 + [vp]
    L.gdn_gate_prepare.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, i32, i32, i32, vp]
    L.gdn_chunk_fwd_workspace_size.argtypes = [i32] * 8
    L.gdn_chunk_fwd_workspace_size.restype = sz
    L.gdn_chunk_fwd.argtypes = ([vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, i32] + [i32] * 6
                                + [f32, i32, i32, vp, sz, vp])
    L.gdn_recurrent_decode.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp] + [i32] * 6 + [f32, i32, i32, vp]
    L.gdn_chunk_prepare.argtypes = [vp, vp, i64, vp, vp, vp, i32] + [i32] * 5 + [f32, i32, i32, vp, sz, vp]
    L.gdn_chunk_scan.argtypes = [vp, vp, i64, vp, i64, vp, vp, vp, vp, i32] + [i32] * 7 + [vp, sz, vp]
    L.gdn_decode_prepare.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, vp] + [i32] * 7 + [vp]
    L.gdn_conv1d_update.argtypes = [vp, i64, vp, vp, vp, vp, vp, i64] + [i32] * 6 + [vp]
    L.gdn_gdp_prefill_prepare.argtypes = ([vp, i64, vp, i64, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp]
                                          + [i32] * 8 + [vp])
    L.gdn_tune_set.argtypes = [i32, i32]
    L.gdn_tune_get.argtypes = [i32]
    L.gdn_prefill_workspace_size.argtypes = [i32] * 8
    L.gdn_prefill_workspace_size.restype = sz
    L.gdn_prefill.argtypes = ([vp, i64, vp, vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, i32]
                              + [i32] * 6 + [f32, i32, i32, vp, sz, vp])
    L.gdn_prefill_prepare.argtypes = ([vp, i64, vp, vp, vp, i64, vp, i64, vp, vp, vp, i32] + [i32] * 6
                                      + [f32, i32, i32, vp, sz, vp])
    L.gdn_prefill_scan.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, i32] + [i32] * 6 + [i32, vp, sz, vp]
    L.gdn_chunk_fwd_noalloc.argtypes = ([vp, vp, i64, vp, i64, vp, vp, vp, vp, vp, vp, i32] + [i32] * 6
                                        + [f32, i32, i32, vp])
    L.gdn_chunk_fwd_noalloc_capacity.argtypes = []
    L.gdn_chunk_fwd_noalloc_capacity.restype = sz
    return L


def test_header_declares_the_operations():
    fns = declared_functions()
    for name in ("gdn_conv1d_causal", "gdn_gate_prepare", "gdn_chunk_fwd", "gdn_chunk_prepare",
                 "gdn_chunk_scan", "gdn_chunk_fwd_workspace_size", "gdn_recurrent_decode",
                 "gdn_decode_prepare", "gdn_conv1d_update", "gdn_gdp_prefill_prepare",
                 "gdn_status_string"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gdn_[a-z0-9_]+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    for code, name in [(OK, b"GDN_OK"), (EINVAL, b"GDN_EINVAL"), (EUNSUP, b"GDN_EUNSUPPORTED"),
                       (EWS, b"GDN_EWORKSPACE"), (ELAUNCH, b"GDN_ELAUNCH")]:
        assert lib.gdn_status_string(code).startswith(name)
    assert lib.gdn_status_string(99) is not None


def conv(lib, **kw):
    a = dict(x=P, xsb=4096 * 6144, xst=6144, w=P2, bias=None, y=P3, ysb=4096 * 6144, yst=6144,
             cu=None, n_seqs=0, B=4, T=4096, C=6144, W=4, silu=1, dtype=BF16, stream=None)
    a.update(kw)
    return lib.gdn_conv1d_causal(a["x"], a["xsb"], a["xst"], a["w"], a["bias"], a["y"], a["ysb"],
                                 a["yst"], a["cu"], a["n_seqs"], a["B"], a["T"], a["C"], a["W"],
                                 a["silu"], a["dtype"], a["stream"])


def test_conv_validation(lib):
    assert conv(lib, x=None) == EINVAL
    assert conv(lib, w=None) == EINVAL
    assert conv(lib, y=None) == EINVAL
    assert conv(lib, y=P) == EINVAL                     # aliasing
    assert conv(lib, B=0) == EINVAL
    assert conv(lib, T=-1) == EINVAL
    assert conv(lib, C=0) == EINVAL
    assert conv(lib, silu=2) == EINVAL
    assert conv(lib, xst=100) == EINVAL                 # rows overlap
    assert conv(lib, cu=P4, n_seqs=3) == EINVAL         # packed needs B == 1
    assert conv(lib, cu=P4, n_seqs=0, B=1) == EINVAL
    assert conv(lib, W=3) == EUNSUP
    assert conv(lib, dtype=7) == EUNSUP
    assert conv(lib, C=6140, xst=6144, yst=6144) == EUNSUP   # C not a multiple of 8 bf16
    assert conv(lib, x=P + 2) == EUNSUP                 # misaligned base
    assert conv(lib, xst=6148, xsb=4096 * 6148) == EUNSUP    # row stride not 16-byte aligned
    assert conv(lib, T=0) == OK                         # empty input: nothing to launch


def gate(lib, **kw):
    a = dict(a=P, asr=16, b=P2, bsr=16, A_log=P3, dt=P4, g=P5, beta=P6, R=10, H=16, dtype=BF16)
    a.update(kw)
    return lib.gdn_gate_prepare(a["a"], a["asr"], a["b"], a["bsr"], a["A_log"], a["dt"], a["g"],
                                a["beta"], a["R"], a["H"], a["dtype"], None)


def test_gate_validation(lib):
    for key in ("a", "b", "A_log", "dt", "g", "beta"):
        assert gate(lib, **{key: None}) == EINVAL
    assert gate(lib, H=0) == EINVAL
    assert gate(lib, R=-1) == EINVAL
    assert gate(lib, asr=8) == EINVAL
    assert gate(lib, beta=P5) == EINVAL                 # g and beta alias
    assert gate(lib, dtype=5) == EUNSUP
    assert gate(lib, R=0) == OK


def chunk(lib, **kw):
    a = dict(q=P, k=P + 4096, qks=6144, v=P + 8192, vs=6144, g=P2, beta=P3, S0=None, Sf=P4, o=P5,
             cu=None, n=0, B=4, T=4096, H=16, Hk=16, K=128, V=128, scale=1.0, l2=1, dtype=BF16,
             ws=WS, wsb=1 << 40)
    a.update(kw)
    return lib.gdn_chunk_fwd(a["q"], a["k"], a["qks"], a["v"], a["vs"], a["g"], a["beta"], a["S0"],
                             a["Sf"], a["o"], a["cu"], a["n"], a["B"], a["T"], a["H"], a["Hk"], a["K"],
                             a["V"], a["scale"], a["l2"], a["dtype"], a["ws"], a["wsb"], None)


def test_chunk_validation(lib):
    for key in ("q", "k", "v", "g", "beta", "o", "ws"):
        assert chunk(lib, **{key: None}) == EINVAL
    assert chunk(lib, H=16, Hk=3) == EINVAL             # H % Hk
    assert chunk(lib, B=0) == EINVAL
    assert chunk(lib, l2=3) == EINVAL
    assert chunk(lib, cu=P6, n=4) == EINVAL             # packed needs B == 1
    assert chunk(lib, qks=100) == EINVAL                # q/k rows shorter than Hk*K
    assert chunk(lib, vs=100) == EINVAL
    assert chunk(lib, o=P) == EINVAL                    # o aliases q
    assert chunk(lib, Sf=P5) == EINVAL                  # final state aliases o
    assert chunk(lib, K=96) == EUNSUP
    assert chunk(lib, V=256) == EUNSUP
    assert chunk(lib, dtype=3) == EUNSUP
    assert chunk(lib, q=P + 2) == EUNSUP
    assert chunk(lib, ws=WS + 16) == EUNSUP             # workspace must be 256-byte aligned
    assert chunk(lib, qks=6148) == EUNSUP
    assert chunk(lib, qks=1 << 24) == EUNSUP            # 64 rows overflow 32-bit offsets
    assert chunk(lib, vs=1 << 24) == EUNSUP
    need = lib.gdn_chunk_fwd_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16)
    assert chunk(lib, wsb=need - 1) == EWS


def test_chunk_phase_validation(lib):
    need = lib.gdn_chunk_fwd_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16)
    prep = lambda **kw: lib.gdn_chunk_prepare(
        kw.get("q", P), kw.get("k", P + 4096), kw.get("qks", 6144), kw.get("g", P2), kw.get("beta", P3),
        None, 0, 4, 4096, kw.get("H", 16), kw.get("Hk", 16), kw.get("K", 128), 1.0, 1, BF16,
        kw.get("ws", WS), kw.get("wsb", need), None)
    scan = lambda **kw: lib.gdn_chunk_scan(
        kw.get("q", P), kw.get("k", P + 4096), 6144, kw.get("v", P + 8192), kw.get("vs", 6144), None,
        kw.get("Sf", P4), kw.get("o", P5), None, 0, 4, 4096, 16, 16, 128, kw.get("V", 128), BF16,
        kw.get("ws", WS), kw.get("wsb", need), None)
    assert prep(g=None) == EINVAL and prep(beta=None) == EINVAL and prep(ws=None) == EINVAL
    assert prep(H=16, Hk=5) == EINVAL and prep(K=32) == EUNSUP and prep(wsb=need - 1) == EWS
    assert prep(qks=1 << 40) == EUNSUP                    # 64 rows would overflow 32-bit offsets
    assert scan(v=None) == EINVAL and scan(o=None) == EINVAL and scan(o=P) == EINVAL
    assert scan(V=96) == EUNSUP and scan(vs=100) == EINVAL and scan(wsb=need - 1) == EWS


def test_chunk_workspace_size(lib):
    # offsets (one 256-byte block) + one record per (chunk, value head): T and P as 6
    # MFMA fragments each (64 lanes x 16 B bf16 / 32 B fp32) + 4 x 64 fp32 row factors
    rec_bf16 = 2 * 6 * 64 * 16 + 4 * 64 * 4
    rec_fp32 = 2 * 6 * 64 * 32 + 4 * 64 * 4
    tiles, H = 4 * 64, 16
    need = lib.gdn_chunk_fwd_workspace_size(4, 4096, H, H, 128, 128, 0, BF16)
    assert need == 256 + tiles * H * rec_bf16
    assert lib.gdn_chunk_fwd_workspace_size(4, 4096, H, H, 128, 128, 0, FP32) == 256 + tiles * H * rec_fp32
    # packed: an upper bound on the chunk count, sum(ceil(len/64)) <= (T + 63 n) / 64
    packed = lib.gdn_chunk_fwd_workspace_size(1, 1000, 4, 4, 64, 64, 10, BF16)
    tiles_ub = (1000 + 63 * 10) // 64
    assert packed >= tiles_ub * 4 * rec_bf16
    assert lib.gdn_chunk_fwd_workspace_size(0, 10, 4, 4, 64, 64, 0, BF16) == 0


def prefill(lib, **kw):
    B, T, H, Hk, K, V = kw.get("B", 4), 4096, kw.get("H", 16), kw.get("Hk", 16), kw.get("K", 128), kw.get("V", 128)
    C = 2 * Hk * K + H * V
    need = lib.gdn_prefill_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16)
    a = dict(x=P, xs=C, w=P2, bias=None, a=P3, as_=H, b=P3 + 64, bs=H, A_log=P4, dt=P4 + 64,
             S0=None, Sf=P5, o=P6, cu=None, n=0, scale=1.0, l2=1, dtype=BF16, ws=WS, wsb=need)
    a.update(kw)
    return lib.gdn_prefill(a["x"], a["xs"], a["w"], a["bias"], a["a"], a["as_"], a["b"], a["bs"],
                           a["A_log"], a["dt"], a["S0"], a["Sf"], a["o"], a["cu"], a["n"], B, T, H,
                           Hk, K, V, a["scale"], a["l2"], a["dtype"], a["ws"], a["wsb"], None)


def test_prefill_validation(lib):
    for key in ("x", "w", "a", "b", "A_log", "dt", "o", "ws"):
        assert prefill(lib, **{key: None}) == EINVAL, key
    assert prefill(lib, H=16, Hk=3) == EINVAL            # H % Hk
    assert prefill(lib, B=0) == EINVAL
    assert prefill(lib, l2=2) == EINVAL
    assert prefill(lib, cu=P6 + 4096, n=4) == EINVAL     # packed needs B == 1
    assert prefill(lib, xs=6143) == EINVAL               # rows shorter than 2 Hk K + H V
    assert prefill(lib, as_=8) == EINVAL and prefill(lib, bs=15) == EINVAL
    assert prefill(lib, o=P) == EINVAL                   # o aliases x
    assert prefill(lib, Sf=P6) == EINVAL                 # final state aliases o
    assert prefill(lib, dtype=FP32) == EUNSUP            # bf16 only
    assert prefill(lib, K=96) == EUNSUP and prefill(lib, V=32) == EUNSUP
    assert prefill(lib, x=P + 2) == EUNSUP and prefill(lib, w=P2 + 8) == EUNSUP
    assert prefill(lib, bias=P2 + 8) == EUNSUP and prefill(lib, o=P6 + 4) == EUNSUP
    assert prefill(lib, xs=6148) == EUNSUP               # rows must stay 16-byte aligned
    assert prefill(lib, xs=1 << 40) == EUNSUP            # 64 rows overflow 32-bit offsets
    assert prefill(lib, ws=WS + 16) == EUNSUP
    need = lib.gdn_prefill_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16)
    assert prefill(lib, wsb=need - 1) == EWS


def test_prefill_phase_validation(lib):
    need = lib.gdn_prefill_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16)
    prep = lambda **kw: lib.gdn_prefill_prepare(
        kw.get("x", P), kw.get("xs", 6144), kw.get("w", P2), None, kw.get("a", P3), kw.get("as_", 16),
        kw.get("b", P3 + 64), 16, kw.get("A_log", P4), P4 + 64, None, 0, 4, 4096, 16, kw.get("Hk", 16),
        kw.get("K", 128), 128, 1.0, kw.get("l2", 1), kw.get("dtype", BF16), kw.get("ws", WS),
        kw.get("wsb", need), None)
    scan = lambda **kw: lib.gdn_prefill_scan(
        kw.get("x", P), kw.get("xs", 6144), kw.get("w", P2), None, None, kw.get("Sf", P5),
        kw.get("o", P6), None, 0, 4, 4096, 16, 16, 128, kw.get("V", 128), kw.get("dtype", BF16),
        kw.get("ws", WS), kw.get("wsb", need), None)
    assert prep(x=None) == EINVAL and prep(w=None) == EINVAL and prep(xs=100) == EINVAL
    assert prep(a=None) == EINVAL and prep(A_log=None) == EINVAL and prep(ws=None) == EINVAL
    assert prep(Hk=5) == EINVAL and prep(K=32) == EUNSUP and prep(dtype=FP32) == EUNSUP
    assert prep(x=P + 2) == EUNSUP and prep(wsb=need - 1) == EWS
    assert prep(as_=8) == EINVAL and prep(l2=2) == EINVAL
    assert scan(o=None) == EINVAL and scan(o=P) == EINVAL and scan(Sf=P6) == EINVAL
    assert scan(V=96) == EUNSUP and scan(wsb=need - 1) == EWS and scan(w=None) == EINVAL


def test_tune_knobs(lib):
    SCAN, RUN, THREADS, FORM = 0, 1, 2, 3
    try:
        for knob, good, bad in ((SCAN, (1, 2, 4, 0), (3, -1, 8)), (RUN, (8, 16, 32, 0), (4, 64)),
                                (THREADS, (64, 128, 256, 0), (32, 512)), (FORM, (1, 2, 0), (3, -1))):
            for v in good:
                assert lib.gdn_tune_set(knob, v) == OK and lib.gdn_tune_get(knob) == v
            lib.gdn_tune_set(knob, good[0])
            for v in bad:   # rejected values change nothing
                assert lib.gdn_tune_set(knob, v) == EINVAL and lib.gdn_tune_get(knob) == good[0]
        assert lib.gdn_tune_set(4, 0) == EINVAL and lib.gdn_tune_get(4) == -1
        assert lib.gdn_tune_get(-1) == -1
    finally:
        for knob in (SCAN, RUN, THREADS, FORM):
            lib.gdn_tune_set(knob, 0)


def test_prefill_workspace_size(lib):
    # the chunked forward's workspace, then per (chunk, key head) a block of the
    # convolved q and k rows: 2 x 64 rows x K bf16
    chunk = lib.gdn_chunk_fwd_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16)
    blocks = 4 * 64 * 16 * (2 * 64 * 128 * 2)
    assert lib.gdn_prefill_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16) == chunk + blocks
    # packed: the same upper bound on the chunk count as the records
    packed_chunk = lib.gdn_chunk_fwd_workspace_size(1, 1000, 4, 2, 64, 64, 10, BF16)
    packed = lib.gdn_prefill_workspace_size(1, 1000, 4, 2, 64, 64, 10, BF16)
    tiles_ub = (1000 + 63 * 10) // 64
    assert packed == (packed_chunk + 255) // 256 * 256 + tiles_ub * 2 * (2 * 64 * 64 * 2)
    assert lib.gdn_prefill_workspace_size(4, 4096, 16, 16, 128, 128, 0, FP32) == 0
    assert lib.gdn_prefill_workspace_size(0, 10, 4, 4, 64, 64, 0, BF16) == 0


def decode(lib, **kw):
    M, H, G, Pd, N = 2, 32, 16, 128, 128
    a = dict(x=P, xs=M * H * Pd + M * G * N + G * N, ba=P2, bas=M * H + H, A_log=P3, dt=P4,
             state=P5, o=P6, n=256, M=M, H=H, G=G, P=Pd, N=N, scale=1.0, l2=1, dtype=BF16)
    a.update(kw)
    return lib.gdn_recurrent_decode(a["x"], a["xs"], a["ba"], a["bas"], a["A_log"], a["dt"],
                                    a["state"], a["o"], a["n"], a["M"], a["H"], a["G"], a["P"],
                                    a["N"], a["scale"], a["l2"], a["dtype"], None)


def test_decode_validation(lib):
    for key in ("x", "ba", "A_log", "dt", "state", "o"):
        assert decode(lib, **{key: None}) == EINVAL
    assert decode(lib, G=5) == EINVAL                   # H % G
    assert decode(lib, M=0) == EINVAL
    assert decode(lib, n=-1) == EINVAL
    assert decode(lib, xs=100) == EINVAL
    assert decode(lib, bas=10) == EINVAL
    assert decode(lib, o=P5) == EINVAL                  # o aliases state
    assert decode(lib, M=5, xs=10 ** 6, bas=1000) == EUNSUP
    assert decode(lib, P=96) == EUNSUP
    assert decode(lib, state=P5 + 4) == EUNSUP
    assert decode(lib, n=0) == OK


def test_binding_fails_loudly_on_cpu_tensors():
    import torch
    import linear_attention_ssm_amd as gdn
    x = torch.zeros(1, 4, 8, dtype=torch.bfloat16)
    w = torch.zeros(8, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        gdn.gdn_conv1d_causal(x, w, y=torch.zeros_like(x))


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "linear_attention_ssm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


ROW5 = 2 * 32 * 128 + 2 * 16 * 128 + 16 * 128   # decode workload row (M=2, H=32, G=16, P=N=128)


def dprep(lib, **kw):
    a = dict(x=P, xs=ROW5, ba=P2, bas=96, A_log=P3, dt=P4, q=P5, k=P6, v=0x70000, beta=0x80000,
             g=0x90000, n=256, M=2, H=32, G=16, Pd=128, N=128, dtype=BF16)
    a.update(kw)
    return lib.gdn_decode_prepare(a["x"], a["xs"], a["ba"], a["bas"], a["A_log"], a["dt"], a["q"],
                                  a["k"], a["v"], a["beta"], a["g"], a["n"], a["M"], a["H"],
                                  a["G"], a["Pd"], a["N"], a["dtype"], None)


def test_decode_prepare_validation(lib):
    for key in ("x", "ba", "A_log", "dt", "q", "k", "v", "beta", "g"):
        assert dprep(lib, **{key: None}) == EINVAL
    assert dprep(lib, n=-1) == EINVAL
    assert dprep(lib, M=0) == EINVAL
    assert dprep(lib, G=5) == EINVAL                    # H % G
    assert dprep(lib, k=P5) == EINVAL                   # q and k alias
    assert dprep(lib, g=0x80000) == EINVAL              # beta and g alias
    assert dprep(lib, xs=ROW5 - 8) == EINVAL            # row stride shorter than a row
    assert dprep(lib, bas=95) == EINVAL
    assert dprep(lib, Pd=96) == EUNSUP
    assert dprep(lib, N=32) == EUNSUP
    assert dprep(lib, dtype=3) == EUNSUP
    assert dprep(lib, x=P + 2) == EUNSUP                # misaligned
    assert dprep(lib, xs=ROW5 + 4) == EUNSUP            # row stride not 16-byte aligned
    assert dprep(lib, q=P5 + 8) == EUNSUP
    assert dprep(lib, n=0) == OK


def cupd(lib, **kw):
    a = dict(x=P, xs=6144, st=P2, slot=P3, w=P4, bias=None, y=P5, ys=6144, n=8, n_slots=16, C=6144,
             W=4, silu=1, dtype=BF16)
    a.update(kw)
    return lib.gdn_conv1d_update(a["x"], a["xs"], a["st"], a["slot"], a["w"], a["bias"], a["y"],
                                 a["ys"], a["n"], a["n_slots"], a["C"], a["W"], a["silu"], a["dtype"],
                                 None)


def test_conv_update_validation(lib):
    for key in ("x", "st", "slot", "w", "y"):
        assert cupd(lib, **{key: None}) == EINVAL
    assert cupd(lib, n=-1) == EINVAL
    assert cupd(lib, n_slots=0) == EINVAL
    assert cupd(lib, C=0) == EINVAL
    assert cupd(lib, silu=3) == EINVAL
    assert cupd(lib, y=P) == EINVAL                     # y aliases x
    assert cupd(lib, y=P2) == EINVAL                    # y aliases the state
    assert cupd(lib, xs=100) == EINVAL
    assert cupd(lib, W=3) == EUNSUP
    assert cupd(lib, dtype=9) == EUNSUP
    assert cupd(lib, C=6140, xs=6144, ys=6144) == EUNSUP
    assert cupd(lib, st=P2 + 4) == EUNSUP
    assert cupd(lib, bias=P6 + 2) == EUNSUP
    assert cupd(lib, n=0, x=None, y=None, slot=None) == OK


def gprep(lib, **kw):
    a = dict(x=P, xs=ROW5, ba=P2, bas=96, A_log=P3, dt=P4, cu=None, n_seqs=0, cu_out=None, q=P5,
             k=P6, v=0x70000, g=0x80000, beta=0x90000, B=2, T=64, M=2, H=32, G=16, Pd=128, N=128,
             dtype=BF16)
    a.update(kw)
    return lib.gdn_gdp_prefill_prepare(a["x"], a["xs"], a["ba"], a["bas"], a["A_log"], a["dt"],
                                       a["cu"], a["n_seqs"], a["cu_out"], a["q"], a["k"], a["v"],
                                       a["g"], a["beta"], a["B"], a["T"], a["M"], a["H"], a["G"],
                                       a["Pd"], a["N"], a["dtype"], None)


def test_gdp_prefill_prepare_validation(lib):
    for key in ("x", "ba", "A_log", "dt", "q", "k", "v", "g", "beta"):
        assert gprep(lib, **{key: None}) == EINVAL
    assert gprep(lib, B=0) == EINVAL
    assert gprep(lib, T=-1) == EINVAL
    assert gprep(lib, M=0) == EINVAL
    assert gprep(lib, G=3) == EINVAL
    assert gprep(lib, cu=0xA0000, n_seqs=2) == EINVAL   # packed needs B == 1
    assert gprep(lib, cu_out=0xB0000) == EINVAL          # cu_out without cu_seqlens
    assert gprep(lib, v=P5) == EINVAL                    # q and v alias
    assert gprep(lib, xs=ROW5 - 1) == EINVAL
    assert gprep(lib, Pd=100) == EUNSUP
    assert gprep(lib, x=P + 4) == EUNSUP
    assert gprep(lib, T=0, x=None, ba=None, q=None, k=None, v=None, g=None, beta=None) == OK
    assert gprep(lib, B=1, cu=0xA0000, n_seqs=2, cu_out=0xB0000, T=0) == OK


def test_token_strides_of_length_one_dims(lib):
    """A length-1 dimension may carry any stride (a view of [B, 1, ...] can
    report a token stride shorter than a row): the binding takes the token
    stride from the batch stride when each batch row has one token."""
    import torch

    import linear_attention_ssm_amd as gdn
    y = torch.zeros(3, 1, 6144, dtype=torch.bfloat16)
    q = y[:, :, :64].view(3, 1, 1, 64)             # strides (6144, 64, 64, 1)
    assert gdn._even_batches(q)
    assert gdn._tstride(q, 64) == 6144             # = batch stride
    x = torch.zeros(2, 5, 8)
    assert gdn._tstride(x, 8) == 8 and gdn._even_batches(x)
    lone = torch.zeros(1, 1, 1, 64).as_strided((1, 1, 1, 64), (64, 1, 64, 1))
    assert gdn._tstride(lone, 64) == 64            # at least a row
    uneven = torch.zeros(2, 10, 8)[:, :5]          # batch stride 80, token stride 8, T = 5
    assert not gdn._even_batches(uneven)


def _raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_binding_checks_every_supplied_tensor():
    """Every tensor the caller supplies, outputs included, is checked for
    shape, dtype and layout before any pointer reaches the library (a wrong
    output shape would otherwise send the kernels out of bounds). CPU
    tensors: the checks run before the device check."""
    import torch

    import linear_attention_ssm_amd as gdn
    bf, f32 = torch.bfloat16, torch.float32
    B, T, Hk, K, H, V = 2, 70, 2, 64, 4, 64
    C = 2 * Hk * K + H * V
    z = torch.zeros
    # conv1d: y shape and layout, taps per channel, bias length
    x = z(B, T, C, dtype=bf)
    w = z(C, 4, dtype=bf)
    _raises(lambda: gdn.gdn_conv1d_causal(x, w, y=z(B, T, C - 8, dtype=bf)), "y must have shape")
    _raises(lambda: gdn.gdn_conv1d_causal(x, w, y=z(B, T, C, dtype=f32)), "y must be")
    _raises(lambda: gdn.gdn_conv1d_causal(x, w, y=z(B, C, T, dtype=bf).transpose(1, 2)),
            "contiguous channel")
    _raises(lambda: gdn.gdn_conv1d_causal(x, z(C - 8, 4, dtype=bf), y=z(B, T, C, dtype=bf)), "w must be")
    _raises(lambda: gdn.gdn_conv1d_causal(x, w, y=z(B, T, C, dtype=bf), bias=z(C + 8, dtype=bf)),
            "bias must have shape")
    # gates: per-head parameters
    a = z(B, T, H, dtype=bf)
    _raises(lambda: gdn.gdn_gate_prepare(a, a, z(H + 1), z(H)), "A_log must have shape")
    _raises(lambda: gdn.gdn_gate_prepare(a, a, z(H), z(H, dtype=torch.float64)), "dt_bias must be")
    # chunked forward: o and the states
    q = z(B, T, Hk, K, dtype=bf)
    v = z(B, T, H, V, dtype=bf)
    g = z(B, T, H)
    ok_o = z(B, T, H, V, dtype=bf)
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=z(B, T, H, V + 64, dtype=bf)), "o must have shape")
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=z(B, T, H, V, dtype=f32)), "o must be")
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=z(B, T, V, H, dtype=bf).transpose(2, 3)),
            "o must be contiguous")
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=ok_o, final_state=z(B, H, V, V + 64)),
            "final_state must have shape")
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=ok_o, final_state=z(B, H, K, V, dtype=bf)),
            "final_state must be")
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=ok_o, initial_state=z(B + 1, H, K, V)),
            "initial_state must have shape")
    # the phases: the scan's o and k; the prepare's gates
    _raises(lambda: gdn.gdn_chunk_scan(q, q, v, z(B, T, H, V - 8, dtype=bf), z(16, dtype=torch.uint8)),
            "o must have shape")
    _raises(lambda: gdn.gdn_chunk_scan(q, z(B, T, Hk, K + 64, dtype=bf), v, ok_o, z(16, dtype=torch.uint8)),
            "k must be")
    _raises(lambda: gdn.gdn_chunk_scan(q, z(B, T, Hk, K), v, ok_o, z(16, dtype=torch.uint8)),
            "q and k")
    _raises(lambda: gdn.gdn_chunk_prepare(q, q, g, z(B, T, H + 1), z(16, dtype=torch.uint8)),
            "beta must have shape")
    # whole prefill: o and the final state
    xp = z(B, T, C, dtype=bf)
    AL = z(H)
    _raises(lambda: gdn.gdn_prefill(xp, w, a, a, AL, AL, Hk=Hk, K=K, H=H, V=V,
                                    o=z(B, T, H, V, dtype=f32)), "o must be")
    _raises(lambda: gdn.gdn_prefill(xp, w, a, a, AL, AL, Hk=Hk, K=K, H=H, V=V, o=ok_o,
                                    final_state=z(B, H, K, 2 * V)), "final_state must have shape")
    _raises(lambda: gdn.gdn_prefill(xp, w, a, a, z(H + 2), AL, Hk=Hk, K=K, H=H, V=V), "A_log must have shape")
    # decode: o, the state, the parameters and the row lengths
    M, G, P, N, n = 2, 2, 64, 64, 3
    row = M * H * P + M * G * N + G * N
    xd = z(n, row, dtype=bf)
    ba = z(n, M * H + H, dtype=bf)
    st = z(n, H, N, P)
    _raises(lambda: gdn.gdn_recurrent_decode(xd, ba, AL, AL, st, M, H, G, P, N, o=z(n, H, P + 8, dtype=bf)),
            "o must have shape")
    _raises(lambda: gdn.gdn_recurrent_decode(xd, ba, z(H - 1), AL, st, M, H, G, P, N), "A_log must have shape")
    _raises(lambda: gdn.gdn_recurrent_decode(xd, ba, AL, AL, z(n, H, P, N + 64), M, H, G, P, N),
            "state must have shape")
    _raises(lambda: gdn.gdn_recurrent_decode(xd[:, :row - 8], ba, AL, AL, st, M, H, G, P, N), "x rows")
    _raises(lambda: gdn.gdn_recurrent_decode(xd, ba[:, :-1], AL, AL, st, M, H, G, P, N), "ba rows")
    _raises(lambda: gdn.gdn_decode_prepare(xd, ba, AL, z(H + 1), M, H, G, P, N), "dt_bias must have shape")
    # decode conv update: y, taps, bias
    Cu = 128
    cst = z(4, 3, Cu, dtype=bf)
    slot = z(n, dtype=torch.int32)
    xu = z(n, Cu, dtype=bf)
    wu = z(Cu, 4, dtype=bf)
    _raises(lambda: gdn.gdn_conv1d_update(xu, cst, slot, wu, y=z(n, Cu - 8, dtype=bf)), "y must have shape")
    _raises(lambda: gdn.gdn_conv1d_update(xu, cst, slot, z(Cu, 4)), "w must be")
    _raises(lambda: gdn.gdn_conv1d_update(xu, cst, slot, wu, bias=z(Cu - 8, dtype=bf)), "bias must have shape")
    # GDP interleave: row lengths, parameters
    xg = z(1, 5, row, dtype=bf)
    bg = z(1, 5, M * H + H, dtype=bf)
    _raises(lambda: gdn.gdn_gdp_prefill_prepare(xg[:, :, :row - 8], bg, AL, AL, M, H, G, P, N), "x rows")
    _raises(lambda: gdn.gdn_gdp_prefill_prepare(xg, bg, z(H, dtype=bf), AL, M, H, G, P, N), "A_log must be")
    # correct shapes on the CPU: the device check still refuses them
    _raises(lambda: gdn.gdn_chunk_fwd(q, q, v, g, g, o=ok_o), "GPU")


def test_noalloc_validation(lib):
    """gdn_chunk_fwd_noalloc: the checks of gdn_chunk_fwd, and a workspace
    that would exceed the library's fixed array refused before any HIP call."""
    cap = lib.gdn_chunk_fwd_noalloc_capacity()
    assert cap == 64 << 20
    call = lambda **kw: lib.gdn_chunk_fwd_noalloc(
        kw.get("q", P), kw.get("k", P + 4096), kw.get("qks", 6144), kw.get("v", P + 8192), 6144,
        kw.get("g", P2), kw.get("beta", P3), None, kw.get("Sf", P4), kw.get("o", P5), None, 0,
        kw.get("B", 4), kw.get("T", 4096), 16, 16, 128, 128, 1.0, 1, kw.get("dtype", BF16), None)
    assert call(q=None) == EINVAL and call(o=None) == EINVAL and call(o=P) == EINVAL
    assert call(g=None) == EINVAL and call(Sf=P5) == EINVAL
    assert call(dtype=3) == EUNSUP and call(q=P + 2) == EUNSUP
    # the prefill workload fits; eight times its batch does not
    assert lib.gdn_chunk_fwd_workspace_size(4, 4096, 16, 16, 128, 128, 0, BF16) <= cap
    assert lib.gdn_chunk_fwd_workspace_size(32, 4096, 16, 16, 128, 128, 0, BF16) > cap
    assert call(B=32) == EWS
