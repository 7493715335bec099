"""MI355X-native gated-delta-rule forward: Python binding of libgdn.so.

The functions below carry the names of the C entry points in include/gdn.h and
only marshal arguments: tensor -> device pointer, strides, dtype code, the
current HIP stream. Every step of the computation runs in the library's HIP
kernels; there is no fallback. Importing this package fails if libgdn.so has
not been built (``python linear_attention_ssm_amd/build.py``), and every call
fails on tensors that are not on a GPU.

PyTorch is used for device memory (allocating outputs and workspaces) and for
the current stream only.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "GdnError", "LIB_PATH", "gdn_status_string", "gdn_conv1d_causal", "gdn_gate_prepare",
    "gdn_chunk_fwd_workspace_size", "gdn_chunk_fwd", "gdn_chunk_prepare", "gdn_chunk_scan",
    "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_noalloc_capacity",
    "gdn_prefill_workspace_size", "gdn_prefill", "gdn_prefill_prepare", "gdn_prefill_scan",
    "gdn_tune_set", "gdn_tune_get", "GDN_TUNE_SCAN_TILES", "GDN_TUNE_CONV_RUN",
    "GDN_TUNE_CONV_THREADS", "GDN_TUNE_SCAN_FORM",
    "gdn_recurrent_decode", "gdn_decode_prepare", "gdn_conv1d_update", "gdn_gdp_prefill_prepare",
    "gdp_prefill", "prefill_chain", "split_qkv",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_FP32, GDN_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: GDN_FP32, torch.bfloat16: GDN_BF16}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python linear_attention_ssm_amd/build.py` "
        "(the HIP library is the only implementation; there is no fallback)")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_lib.gdn_status_string.argtypes = [_i32]
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_conv1d_causal.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _vp, _i32,
                                   _i32, _i32, _i32, _i32, _i32, _i32, _vp]
_lib.gdn_conv1d_causal.restype = _i32
_lib.gdn_gate_prepare.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
_lib.gdn_gate_prepare.restype = _i32
_lib.gdn_chunk_fwd_workspace_size.argtypes = [_i32] * 8
_lib.gdn_chunk_fwd_workspace_size.restype = _sz
_lib.gdn_chunk_fwd.argtypes = ([_vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32]
                               + [_i32] * 6 + [_f32, _i32, _i32, _vp, _sz, _vp])
_lib.gdn_chunk_fwd.restype = _i32
_lib.gdn_chunk_fwd_noalloc.argtypes = ([_vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32]
                                       + [_i32] * 6 + [_f32, _i32, _i32, _vp])
_lib.gdn_chunk_fwd_noalloc.restype = _i32
_lib.gdn_chunk_fwd_noalloc_capacity.argtypes = []
_lib.gdn_chunk_fwd_noalloc_capacity.restype = _sz
_lib.gdn_tune_set.argtypes = [_i32, _i32]
_lib.gdn_tune_set.restype = _i32
_lib.gdn_tune_get.argtypes = [_i32]
_lib.gdn_tune_get.restype = _i32
_lib.gdn_prefill_workspace_size.argtypes = [_i32] * 8
_lib.gdn_prefill_workspace_size.restype = _sz
_lib.gdn_prefill.argtypes = ([_vp, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp,
                              _vp, _i32] + [_i32] * 6 + [_f32, _i32, _i32, _vp, _sz, _vp])
_lib.gdn_prefill.restype = _i32
_lib.gdn_prefill_prepare.argtypes = ([_vp, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32]
                                     + [_i32] * 6 + [_f32, _i32, _i32, _vp, _sz, _vp])
_lib.gdn_prefill_prepare.restype = _i32
_lib.gdn_prefill_scan.argtypes = ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32] + [_i32] * 6
                                  + [_i32, _vp, _sz, _vp])
_lib.gdn_prefill_scan.restype = _i32
_lib.gdn_chunk_prepare.argtypes = ([_vp, _vp, _i64, _vp, _vp, _vp, _i32] + [_i32] * 5
                                   + [_f32, _i32, _i32, _vp, _sz, _vp])
_lib.gdn_chunk_prepare.restype = _i32
_lib.gdn_chunk_scan.argtypes = ([_vp, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _i32] + [_i32] * 7
                                + [_vp, _sz, _vp])
_lib.gdn_chunk_scan.restype = _i32
_lib.gdn_recurrent_decode.argtypes = ([_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp]
                                      + [_i32] * 6 + [_f32, _i32, _i32, _vp])
_lib.gdn_recurrent_decode.restype = _i32
_lib.gdn_decode_prepare.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp] + [_i32] * 7 + [_vp]
_lib.gdn_decode_prepare.restype = _i32
_lib.gdn_conv1d_update.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64] + [_i32] * 6 + [_vp]
_lib.gdn_conv1d_update.restype = _i32
_lib.gdn_gdp_prefill_prepare.argtypes = ([_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _vp, _vp,
                                          _vp, _vp, _vp] + [_i32] * 8 + [_vp])
_lib.gdn_gdp_prefill_prepare.restype = _i32


class GdnError(RuntimeError):
    """A non-zero gdn_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {gdn_status_string(status)}")


def gdn_status_string(status: int) -> str:
    return _lib.gdn_status_string(int(status)).decode()


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise GdnError(rc, where)


def _dev(t: torch.Tensor, name: str) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor on the GPU")
    return t.data_ptr()


def _opt(t, name):
    return None if t is None else _dev(t, name)


def _need(t, name: str, shape, dtype: torch.dtype, contiguous: bool = True) -> None:
    """Shape, dtype and layout of a tensor the caller supplies (checked before
    any pointer reaches the library: the kernels assume exactly this layout)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_params(H: int, **params) -> None:
    """Per-head fp32 gate parameters (A_log, dt_bias): contiguous [H]."""
    for name, t in params.items():
        _need(t, name, (H,), torch.float32)


def _same_device(*tensors) -> None:
    devs = {t.device for t in tensors if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")


def _code(dt: torch.dtype) -> int:
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt} (float32 or bfloat16)")
    return _DTYPE_CODE[dt]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _tstride(t: torch.Tensor, row: int) -> int:
    """Token stride of a [B, T, ...] tensor as the library takes it (batch b,
    token t at (b T + t) * stride). A length-1 dimension may carry any stride:
    with one token per batch row the batch stride is the token stride, and a
    lone row gets any stride at least a row long."""
    B, T = t.shape[:2]
    if T == 1 and B > 1:
        return t.stride(0)
    if T <= 1:
        return max(t.stride(1), row)
    return t.stride(1)


def _even_batches(t: torch.Tensor) -> bool:
    B, T = t.shape[:2]
    return B <= 1 or T <= 1 or t.stride(0) == T * t.stride(1)


# --------------------------------------------------------------------- conv1d

def gdn_conv1d_causal(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor | None = None,
                      bias: torch.Tensor | None = None, cu_seqlens: torch.Tensor | None = None,
                      silu: bool = True) -> torch.Tensor:
    """Depthwise causal conv1d (W = 4) with optional SiLU. x: [B, T, C] with
    the channel dim contiguous; w: [C, 4]; cu_seqlens: int32 [N+1] for packed
    sequences (B == 1). Returns y [B, T, C] (allocated if not given)."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [B, T, C] with a contiguous channel dim")
    B, T, C = x.shape
    if w.dim() != 2 or w.shape[0] != C:
        raise ValueError(f"w must be [C, W] with C = {C}")
    _need(w, "w", (C, w.shape[1]), x.dtype)
    if bias is not None:
        _need(bias, "bias", (C,), x.dtype)
    if y is None:
        y = torch.empty((B, T, C), dtype=x.dtype, device=x.device)
    _need(y, "y", (B, T, C), x.dtype, contiguous=False)
    if y.stride(2) != 1:
        raise ValueError("y must have a contiguous channel dim")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
    _same_device(x, w, y, bias, cu_seqlens)
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    # (one token per row: its token stride is never used, and a length-1
    # dimension may carry any stride)
    xt, yt = (x.stride(1), y.stride(1)) if T > 1 else (C, C)
    rc = _lib.gdn_conv1d_causal(_dev(x, "x"), x.stride(0), xt, _dev(w, "w"),
                                _opt(bias, "bias"), _dev(y, "y"), y.stride(0), yt,
                                _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, C, w.shape[1],
                                int(bool(silu)), _code(x.dtype), _stream(x.device))
    _check(rc, "gdn_conv1d_causal")
    return y


# ---------------------------------------------------------------------- gates

def gdn_gate_prepare(a: torch.Tensor, b: torch.Tensor, A_log: torch.Tensor,
                     dt_bias: torch.Tensor, g: torch.Tensor | None = None,
                     beta: torch.Tensor | None = None):
    """beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias). a, b: [..., H]
    (rows may be strided, the head dim contiguous). Returns fp32 (g, beta) of
    a's shape."""
    if a.shape != b.shape or a.dtype != b.dtype:
        raise ValueError("a and b must have the same shape and dtype")
    H = a.shape[-1]
    a2 = a.reshape(-1, H) if a.dim() != 2 else a
    b2 = b.reshape(-1, H) if b.dim() != 2 else b
    if a2.stride(-1) != 1 or b2.stride(-1) != 1:
        raise ValueError("the head dim of a and b must be contiguous")
    R = a2.shape[0]
    if g is None:
        g = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    if beta is None:
        beta = torch.empty(a.shape, dtype=torch.float32, device=a.device)
    for t, n in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != R * H:
            raise ValueError(f"{n} must be a contiguous fp32 tensor with {R * H} elements")
    _need_params(H, A_log=A_log, dt_bias=dt_bias)
    _same_device(a, b, A_log, dt_bias, g, beta)
    rc = _lib.gdn_gate_prepare(_dev(a2, "a"), a2.stride(0), _dev(b2, "b"), b2.stride(0),
                               _dev(A_log, "A_log"), _dev(dt_bias, "dt_bias"), _dev(g, "g"),
                               _dev(beta, "beta"), R, H, _code(a.dtype), _stream(a.device))
    _check(rc, "gdn_gate_prepare")
    return g, beta


# ----------------------------------------------------------------- chunk fwd

def gdn_chunk_fwd_workspace_size(B: int, T: int, H: int, Hk: int, K: int, V: int,
                                 n_seqs: int, dtype: torch.dtype) -> int:
    return int(_lib.gdn_chunk_fwd_workspace_size(B, T, H, Hk, K, V, n_seqs, _code(dtype)))


def _token_rows(t: torch.Tensor, name: str, heads: int, d: int):
    """[B, T, heads, d] with contiguous (heads, d) and batch stride T * token stride."""
    if t.dim() != 4 or t.shape[2] != heads or t.shape[3] != d:
        raise ValueError(f"{name} must be [B, T, {heads}, {d}]")
    if t.stride(3) != 1 or (heads > 1 and t.stride(2) != d) or not _even_batches(t):
        raise ValueError(f"{name}: heads and head dim must be contiguous and batches evenly strided")
    return _tstride(t, heads * d)


def _chunk_outputs(like, B, T, N, H, K, V, initial_state, output_final_state, o, final_state):
    """The initial state (if any), and the output and final state, allocated
    when not given and checked when given: o contiguous [B, T, H, V] in the
    activation dtype, states contiguous fp32 [N, H, K, V]."""
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, K, V), torch.float32)
    if o is None:
        o = torch.empty((B, T, H, V), dtype=like.dtype, device=like.device)
    _need(o, "o", (B, T, H, V), like.dtype)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, K, V), dtype=torch.float32, device=like.device)
    if not output_final_state:
        final_state = None
    if final_state is not None:
        _need(final_state, "final_state", (N, H, K, V), torch.float32)
    return o, final_state


def gdn_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, initial_state: torch.Tensor | None = None,
                  output_final_state: bool = True, cu_seqlens: torch.Tensor | None = None,
                  scale: float = 1.0, qk_l2norm: bool = True,
                  workspace: torch.Tensor | None = None, o: torch.Tensor | None = None,
                  final_state: torch.Tensor | None = None):
    """Chunked gated delta rule. q, k: [B, T, Hk, K]; v: [B, T, H, V] (token
    rows may be strided views of the conv output); g, beta: fp32 [B, T, H];
    initial_state: fp32 [N, H, K, V] or None. Returns (o [B, T, H, V],
    final_state [N, H, K, V] or None)."""
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    st_qk = _token_rows(q, "q", Hk, K)
    if _token_rows(k, "k", Hk, K) != st_qk or k.shape != q.shape:
        raise ValueError("q and k must share shape and strides")
    st_v = _token_rows(v, "v", H, V)
    if v.shape[:2] != (B, T) or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must agree in batch, length and dtype")
    for t, n in ((g, "g"), (beta, "beta")):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != (B, T, H):
            raise ValueError(f"{n} must be a contiguous fp32 [B, T, H] tensor")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    N = n_seqs if cu_seqlens is not None else B
    o, final_state = _chunk_outputs(q, B, T, N, H, K, V, initial_state, output_final_state,
                                    o, final_state)
    ws_bytes = gdn_chunk_fwd_workspace_size(B, T, H, Hk, K, V, n_seqs, q.dtype)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    _same_device(q, k, v, g, beta, initial_state, final_state, o, cu_seqlens, workspace)
    rc = _lib.gdn_chunk_fwd(_dev(q, "q"), _dev(k, "k"), st_qk, _dev(v, "v"), st_v, _dev(g, "g"),
                            _dev(beta, "beta"), _opt(initial_state, "initial_state"),
                            _opt(final_state, "final_state"), _dev(o, "o"),
                            _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk, K, V,
                            float(scale), int(bool(qk_l2norm)), _code(q.dtype),
                            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                            _stream(q.device))
    _check(rc, "gdn_chunk_fwd")
    return o, final_state


def gdn_chunk_fwd_noalloc_capacity() -> int:
    """Bytes of the library's own device workspace used by gdn_chunk_fwd_noalloc."""
    return int(_lib.gdn_chunk_fwd_noalloc_capacity())


def gdn_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                          beta: torch.Tensor, o: torch.Tensor,
                          initial_state: torch.Tensor | None = None,
                          final_state: torch.Tensor | None = None,
                          cu_seqlens: torch.Tensor | None = None, scale: float = 1.0,
                          qk_l2norm: bool = True):
    """gdn_chunk_fwd with the library's own fixed device workspace: nothing is
    allocated, so the caller passes the outputs (o [B, T, H, V]; final_state
    [N, H, K, V] fp32 or None). Calls that overlap on one GPU race on the
    workspace. Returns (o, final_state)."""
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    st_qk = _token_rows(q, "q", Hk, K)
    if _token_rows(k, "k", Hk, K) != st_qk or k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape, strides and dtype")
    st_v = _token_rows(v, "v", H, V)
    if v.shape[:2] != (B, T) or v.dtype != q.dtype:
        raise ValueError("v must agree with q in batch, length and dtype")
    _need(g, "g", (B, T, H), torch.float32)
    _need(beta, "beta", (B, T, H), torch.float32)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    N = n_seqs if cu_seqlens is not None else B
    _chunk_outputs(q, B, T, N, H, K, V, initial_state, final_state is not None, o, final_state)
    _same_device(q, k, v, g, beta, o, initial_state, final_state, cu_seqlens)
    rc = _lib.gdn_chunk_fwd_noalloc(_dev(q, "q"), _dev(k, "k"), st_qk, _dev(v, "v"), st_v,
                                    _dev(g, "g"), _dev(beta, "beta"),
                                    _opt(initial_state, "initial_state"),
                                    _opt(final_state, "final_state"), _dev(o, "o"),
                                    _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk, K, V,
                                    float(scale), int(bool(qk_l2norm)), _code(q.dtype),
                                    _stream(q.device))
    _check(rc, "gdn_chunk_fwd_noalloc")
    return o, final_state


# launch-configuration knobs (C constants of the same names)
GDN_TUNE_SCAN_TILES, GDN_TUNE_CONV_RUN, GDN_TUNE_CONV_THREADS, GDN_TUNE_SCAN_FORM = 0, 1, 2, 3


def gdn_tune_set(knob: int, value: int) -> None:
    """Set a launch-configuration knob (0 = automatic); results do not change."""
    _check(_lib.gdn_tune_set(int(knob), int(value)), "gdn_tune_set")


def gdn_tune_get(knob: int) -> int:
    v = int(_lib.gdn_tune_get(int(knob)))
    if v < 0:
        raise ValueError(f"unknown knob {knob}")
    return v


def gdn_prefill_workspace_size(B: int, T: int, H: int, Hk: int, K: int, V: int,
                               n_seqs: int, dtype: torch.dtype = torch.bfloat16) -> int:
    return int(_lib.gdn_prefill_workspace_size(B, T, H, Hk, K, V, n_seqs, _code(dtype)))


def _prefill_args(x, w, a, b, A_log, dt_bias, Hk, K, H, V, bias, cu_seqlens):
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [B, T, C] with a contiguous channel dim")
    B, T, C = x.shape
    if C != 2 * Hk * K + H * V:
        raise ValueError(f"x has {C} channels, expected 2*Hk*K + H*V = {2 * Hk * K + H * V}")
    if not _even_batches(x):
        raise ValueError("x: batch rows must be evenly strided (stride(0) == T * stride(1))")
    if w.shape != (C, 4) or not w.is_contiguous() or w.dtype != x.dtype:
        raise ValueError("w must be a contiguous [C, 4] tensor of x's dtype")
    if bias is not None and (bias.shape != (C,) or bias.dtype != x.dtype or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [C] tensor of x's dtype")
    for t, n in ((a, "a"), (b, "b")):
        if t is None:
            continue
        if t.shape != (B, T, H) or t.dtype != x.dtype or t.stride(2) != 1 or not _even_batches(t):
            raise ValueError(f"{n} must be [B, T, H] of x's dtype, head dim contiguous, "
                             "batch rows evenly strided")
    for t, n in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        if t is not None:
            _need(t, n, (H,), torch.float32)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _same_device(x, w, a, b, A_log, dt_bias, bias, cu_seqlens)
    return B, T, n_seqs


def _prefill_outputs(x, B, T, n_seqs, cu_seqlens, H, K, V, initial_state, output_final_state,
                     o, final_state):
    N = n_seqs if cu_seqlens is not None else B
    return _chunk_outputs(x, B, T, N, H, K, V, initial_state, output_final_state, o, final_state)


def _prefill_ws(workspace, x, B, T, H, Hk, K, V, n_seqs):
    if workspace is None:
        ws_bytes = gdn_prefill_workspace_size(B, T, H, Hk, K, V, n_seqs, x.dtype)
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    return workspace


def gdn_prefill(x: torch.Tensor, w: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                A_log: torch.Tensor, dt_bias: torch.Tensor, *, Hk: int, K: int, H: int, V: int,
                bias: torch.Tensor | None = None, initial_state: torch.Tensor | None = None,
                output_final_state: bool = True, cu_seqlens: torch.Tensor | None = None,
                scale: float = 1.0, qk_l2norm: bool = True,
                workspace: torch.Tensor | None = None, o: torch.Tensor | None = None,
                final_state: torch.Tensor | None = None):
    """The whole prefill (conv1d + SiLU over q | k | v, gates, chunked forward)
    in two launches (gdn_prefill_prepare, gdn_prefill_scan). x: bf16 [B, T, C] rows before the convolution, C = 2 Hk
    K + H V, channel dim contiguous; w: [C, 4]; a, b: bf16 [B, T, H] (the head
    dim contiguous, rows evenly strided). Returns (o [B, T, H, V],
    final_state [N, H, K, V] or None), equal bit for bit to prefill_chain."""
    B, T, n_seqs = _prefill_args(x, w, a, b, A_log, dt_bias, Hk, K, H, V, bias, cu_seqlens)
    o, final_state = _prefill_outputs(x, B, T, n_seqs, cu_seqlens, H, K, V, initial_state,
                                      output_final_state, o, final_state)
    workspace = _prefill_ws(workspace, x, B, T, H, Hk, K, V, n_seqs)
    rc = _lib.gdn_prefill(_dev(x, "x"), _tstride(x, x.shape[2]), _dev(w, "w"), _opt(bias, "bias"),
                          _dev(a, "a"), _tstride(a, H), _dev(b, "b"), _tstride(b, H),
                          _dev(A_log, "A_log"), _dev(dt_bias, "dt_bias"),
                          _opt(initial_state, "initial_state"), _opt(final_state, "final_state"),
                          _dev(o, "o"), _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk, K, V,
                          float(scale), int(bool(qk_l2norm)), _code(x.dtype),
                          _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                          _stream(x.device))
    _check(rc, "gdn_prefill")
    return o, final_state


def gdn_prefill_prepare(x, w, a, b, A_log, dt_bias, workspace, *, Hk, K, H, V, bias=None,
                        cu_seqlens=None, scale=1.0, qk_l2norm=True):
    """Phase 1 of gdn_prefill (q/k convolution, gates, per-chunk solve) into `workspace`."""
    B, T, n_seqs = _prefill_args(x, w, a, b, A_log, dt_bias, Hk, K, H, V, bias, cu_seqlens)
    rc = _lib.gdn_prefill_prepare(_dev(x, "x"), _tstride(x, x.shape[2]), _dev(w, "w"),
                                  _opt(bias, "bias"), _dev(a, "a"), _tstride(a, H), _dev(b, "b"),
                                  _tstride(b, H),
                                  _dev(A_log, "A_log"), _dev(dt_bias, "dt_bias"),
                                  _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk, K, V,
                                  float(scale), int(bool(qk_l2norm)), _code(x.dtype),
                                  _dev(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(), _stream(x.device))
    _check(rc, "gdn_prefill_prepare")


def gdn_prefill_scan(x, w, workspace, *, Hk, K, H, V, bias=None, initial_state=None,
                     output_final_state=True, cu_seqlens=None, o=None, final_state=None):
    """Phase 2 of gdn_prefill (value convolution and the state scan). Returns (o, final_state)."""
    B, T, n_seqs = _prefill_args(x, w, None, None, None, None, Hk, K, H, V, bias, cu_seqlens)
    o, final_state = _prefill_outputs(x, B, T, n_seqs, cu_seqlens, H, K, V, initial_state,
                                      output_final_state, o, final_state)
    rc = _lib.gdn_prefill_scan(_dev(x, "x"), _tstride(x, x.shape[2]), _dev(w, "w"), _opt(bias, "bias"),
                               _opt(initial_state, "initial_state"), _opt(final_state, "final_state"),
                               _dev(o, "o"), _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk,
                               K, V, _code(x.dtype), _dev(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(), _stream(x.device))
    _check(rc, "gdn_prefill_scan")
    return o, final_state


def gdn_chunk_prepare(q, k, g, beta, workspace, cu_seqlens=None, scale=1.0, qk_l2norm=True,
                      H: int | None = None):
    """Phase 1 of gdn_chunk_fwd (per-chunk WY solve) into `workspace`."""
    B, T, Hk, K = q.shape
    H = g.shape[2] if H is None else H
    st_qk = _token_rows(q, "q", Hk, K)
    if _token_rows(k, "k", Hk, K) != st_qk or k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape, strides and dtype")
    _need(g, "g", (B, T, H), torch.float32)
    _need(beta, "beta", (B, T, H), torch.float32)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    _same_device(q, k, g, beta, cu_seqlens, workspace)
    rc = _lib.gdn_chunk_prepare(_dev(q, "q"), _dev(k, "k"), st_qk, _dev(g, "g"), _dev(beta, "beta"),
                                _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk, K,
                                float(scale), int(bool(qk_l2norm)), _code(q.dtype),
                                _dev(workspace, "workspace"),
                                workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(rc, "gdn_chunk_prepare")


def gdn_chunk_scan(q, k, v, o, workspace, initial_state=None, final_state=None, cu_seqlens=None):
    """Phase 2 of gdn_chunk_fwd (state scan + outputs) from a prepared workspace."""
    B, T, Hk, K = q.shape
    H, V = v.shape[2], v.shape[3]
    st_qk = _token_rows(q, "q", Hk, K)
    if _token_rows(k, "k", Hk, K) != st_qk or k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must share shape, strides and dtype")
    st_v = _token_rows(v, "v", H, V)
    if v.shape[:2] != (B, T) or v.dtype != q.dtype:
        raise ValueError("v must agree with q in batch, length and dtype")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    N = n_seqs if cu_seqlens is not None else B
    _chunk_outputs(q, B, T, N, H, K, V, initial_state, final_state is not None, o, final_state)
    _same_device(q, k, v, o, initial_state, final_state, cu_seqlens, workspace)
    rc = _lib.gdn_chunk_scan(_dev(q, "q"), _dev(k, "k"), st_qk, _dev(v, "v"), st_v,
                             _opt(initial_state, "initial_state"), _opt(final_state, "final_state"),
                             _dev(o, "o"), _opt(cu_seqlens, "cu_seqlens"), n_seqs, B, T, H, Hk, K, V,
                             _code(q.dtype), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(rc, "gdn_chunk_scan")
    return o


# -------------------------------------------------------------------- decode

def _decode_rows(x, ba, M, H, G, P, N) -> None:
    """x [n, >= M*H*P + M*G*N + G*N] and ba [n, >= M*H + H] rows of one dtype,
    the last dim contiguous (rows may be strided)."""
    n = x.shape[0]
    if x.dim() != 2 or ba.dim() != 2 or ba.shape[0] != n:
        raise ValueError("x and ba must be [n, row]")
    if x.stride(-1) != 1 or ba.stride(-1) != 1 or ba.dtype != x.dtype:
        raise ValueError("x and ba must be [n, row] with contiguous rows of one dtype")
    if x.shape[1] < M * H * P + M * G * N + G * N:
        raise ValueError(f"x rows must hold M*H*P + M*G*N + G*N = {M * H * P + M * G * N + G * N} "
                         f"elements, got {x.shape[1]}")
    if ba.shape[1] < M * H + H:
        raise ValueError(f"ba rows must hold M*H + H = {M * H + H} elements, got {ba.shape[1]}")


def gdn_recurrent_decode(x: torch.Tensor, ba: torch.Tensor, A_log: torch.Tensor,
                         dt_bias: torch.Tensor, state: torch.Tensor, M: int, H: int, G: int,
                         P: int, N: int, o: torch.Tensor | None = None, scale: float = 1.0,
                         qk_l2norm: bool = True) -> torch.Tensor:
    """One decode token for n requests. x: [n, M*H*P + M*G*N + G*N] (v | k | q);
    ba: [n, M*H + H] (b | a), rows may be strided; state: fp32 [n, H, N, P],
    updated in place. Returns o [n, H, P] in x's dtype."""
    if x.dim() == 3:
        x = x.reshape(x.shape[0], x.shape[-1])
    if ba.dim() == 3:
        ba = ba.reshape(ba.shape[0], ba.shape[-1])
    n = x.shape[0]
    _decode_rows(x, ba, M, H, G, P, N)
    _need(state, "state", (n, H, N, P), torch.float32)
    _need_params(H, A_log=A_log, dt_bias=dt_bias)
    if o is None:
        o = torch.empty((n, H, P), dtype=x.dtype, device=x.device)
    _need(o, "o", (n, H, P), x.dtype)
    _same_device(x, ba, A_log, dt_bias, state, o)
    rc = _lib.gdn_recurrent_decode(_dev(x, "x"), x.stride(0), _dev(ba, "ba"), ba.stride(0),
                                   _dev(A_log, "A_log"), _dev(dt_bias, "dt_bias"),
                                   _dev(state, "state"), _dev(o, "o"), n, M, H, G, P, N,
                                   float(scale), int(bool(qk_l2norm)), _code(x.dtype),
                                   _stream(x.device))
    _check(rc, "gdn_recurrent_decode")
    return o


def gdn_decode_prepare(x: torch.Tensor, ba: torch.Tensor, A_log: torch.Tensor,
                       dt_bias: torch.Tensor, M: int, H: int, G: int, P: int, N: int,
                       out: tuple | None = None):
    """The five tensors of one decode step: returns (q [n,M,H,N], k [n,M,H,N],
    v [n,M,H,P] in x's dtype, beta [n,M,H], g [n,M,H] fp32). `out` may hold
    preallocated contiguous (q, k, v, beta, g)."""
    if x.dim() == 3:
        x = x.reshape(x.shape[0], x.shape[-1])
    if ba.dim() == 3:
        ba = ba.reshape(ba.shape[0], ba.shape[-1])
    n = x.shape[0]
    _decode_rows(x, ba, M, H, G, P, N)
    _need_params(H, A_log=A_log, dt_bias=dt_bias)
    dev = x.device
    if out is None:
        q = torch.empty((n, M, H, N), dtype=x.dtype, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((n, M, H, P), dtype=x.dtype, device=dev)
        beta = torch.empty((n, M, H), dtype=torch.float32, device=dev)
        g = torch.empty_like(beta)
    else:
        q, k, v, beta, g = out
        for t, shp, dt in ((q, (n, M, H, N), x.dtype), (k, (n, M, H, N), x.dtype),
                           (v, (n, M, H, P), x.dtype), (beta, (n, M, H), torch.float32),
                           (g, (n, M, H), torch.float32)):
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"output tensors must be contiguous {shp} {dt}")
    _same_device(x, ba, A_log, dt_bias, q, k, v, beta, g)
    rc = _lib.gdn_decode_prepare(_dev(x, "x"), x.stride(0), _dev(ba, "ba"), ba.stride(0),
                                 _dev(A_log, "A_log"), _dev(dt_bias, "dt_bias"), _dev(q, "q"),
                                 _dev(k, "k"), _dev(v, "v"), _dev(beta, "beta"), _dev(g, "g"),
                                 n, M, H, G, P, N, _code(x.dtype), _stream(dev))
    _check(rc, "gdn_decode_prepare")
    return q, k, v, beta, g


def gdn_conv1d_update(x: torch.Tensor, conv_state: torch.Tensor, slot: torch.Tensor,
                      w: torch.Tensor, bias: torch.Tensor | None = None,
                      y: torch.Tensor | None = None, silu: bool = True) -> torch.Tensor:
    """Short-conv update of one decode token per request. x: [n, C] (rows may be
    strided); conv_state: [S, W-1, C] contiguous, updated in place; slot: int32
    [n] (-1 = padding: zero output, no update). Returns y [n, C]."""
    n, C = x.shape
    S, Wm1, Cs = conv_state.shape
    if x.stride(-1) != 1 or Cs != C or not conv_state.is_contiguous() or conv_state.dtype != x.dtype:
        raise ValueError("conv_state must be a contiguous [S, W-1, C] tensor of x's dtype")
    if slot.dtype != torch.int32 or slot.numel() != n:
        raise ValueError("slot must be int32 [n]")
    _need(w, "w", (C, Wm1 + 1), x.dtype)
    if bias is not None:
        _need(bias, "bias", (C,), x.dtype)
    if y is None:
        y = torch.empty((n, C), dtype=x.dtype, device=x.device)
    _need(y, "y", (n, C), x.dtype, contiguous=False)
    if y.stride(-1) != 1:
        raise ValueError("y must be [n, C] with contiguous rows")
    _same_device(x, conv_state, slot, w, bias, y)
    rc = _lib.gdn_conv1d_update(_dev(x, "x"), x.stride(0), _dev(conv_state, "conv_state"),
                                _dev(slot, "slot"), _dev(w, "w"), _opt(bias, "bias"), _dev(y, "y"),
                                y.stride(0), n, S, C, Wm1 + 1, int(bool(silu)), _code(x.dtype),
                                _stream(x.device))
    _check(rc, "gdn_conv1d_update")
    return y


def gdn_gdp_prefill_prepare(x: torch.Tensor, ba: torch.Tensor, A_log: torch.Tensor,
                            dt_bias: torch.Tensor, M: int, H: int, G: int, P: int, N: int,
                            cu_seqlens: torch.Tensor | None = None, out: tuple | None = None):
    """Interleave a Gated DeltaProduct prefill into an M*T-token gated delta
    rule. x: [B, T, M*H*P + M*G*N + G*N], ba: [B, T, M*H + H] (token rows may
    be strided, batches evenly strided). Returns (q [B, M*T, G, N], k, v
    [B, M*T, H, P], g [B, M*T, H], beta, cu_out or None)."""
    B, T, row = x.shape
    if x.stride(-1) != 1 or ba.stride(-1) != 1 or ba.shape[:2] != (B, T) or ba.dtype != x.dtype:
        raise ValueError("x and ba must be [B, T, row] with contiguous rows of one dtype")
    if row < M * H * P + M * G * N + G * N or ba.shape[2] < M * H + H:
        raise ValueError("x rows must hold M*H*P + M*G*N + G*N elements and ba rows M*H + H")
    _need_params(H, A_log=A_log, dt_bias=dt_bias)
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", (cu_seqlens.numel(),), torch.int32)
    for t, name in ((x, "x"), (ba, "ba")):
        if not _even_batches(t):
            raise ValueError(f"{name}: batches must be evenly strided")
    dev = x.device
    if out is None:
        q = torch.empty((B, M * T, G, N), dtype=x.dtype, device=dev)
        k = torch.empty_like(q)
        v = torch.empty((B, M * T, H, P), dtype=x.dtype, device=dev)
        g = torch.empty((B, M * T, H), dtype=torch.float32, device=dev)
        beta = torch.empty_like(g)
    else:
        q, k, v, g, beta = out
        for t, shp, dt in ((q, (B, M * T, G, N), x.dtype), (k, (B, M * T, G, N), x.dtype),
                           (v, (B, M * T, H, P), x.dtype), (g, (B, M * T, H), torch.float32),
                           (beta, (B, M * T, H), torch.float32)):
            if tuple(t.shape) != shp or t.dtype != dt or not t.is_contiguous():
                raise ValueError(f"output tensors must be contiguous {shp} {dt}")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    cu_out = None if cu_seqlens is None else torch.empty_like(cu_seqlens)
    _same_device(x, ba, A_log, dt_bias, cu_seqlens, q, k, v, g, beta)
    rc = _lib.gdn_gdp_prefill_prepare(_dev(x, "x"), _tstride(x, row), _dev(ba, "ba"),
                                      _tstride(ba, ba.shape[2]),
                                      _dev(A_log, "A_log"), _dev(dt_bias, "dt_bias"),
                                      _opt(cu_seqlens, "cu_seqlens"), n_seqs, _opt(cu_out, "cu_out"),
                                      _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(g, "g"),
                                      _dev(beta, "beta"), B, T, M, H, G, P, N, _code(x.dtype),
                                      _stream(dev))
    _check(rc, "gdn_gdp_prefill_prepare")
    return q, k, v, g, beta, cu_out


def gdp_prefill(x, ba, A_log, dt_bias, M, H, G, P, N, initial_state=None, cu_seqlens=None,
                scale=1.0, qk_l2norm=True, workspace=None):
    """A Gated DeltaProduct prefill: the interleave above, then gdn_chunk_fwd
    over the M*T positions. Returns (o [B, T, H, P] -- a view of rows t*M + M-1
    of the interleaved output --, final_state [N_seq, H, N, P])."""
    q, k, v, g, beta, cu2 = gdn_gdp_prefill_prepare(x, ba, A_log, dt_bias, M, H, G, P, N, cu_seqlens)
    o2, fs = gdn_chunk_fwd(q, k, v, g, beta, initial_state=initial_state, cu_seqlens=cu2,
                           scale=scale, qk_l2norm=qk_l2norm, workspace=workspace)
    return o2[:, M - 1::M], fs


# ------------------------------------------------------------ prefill chain

def split_qkv(y: torch.Tensor, Hk: int, K: int, H: int, V: int):
    """Zero-copy q, k, v views of the conv output y [B, T, 2*Hk*K + H*V]
    (channel order q | k | v)."""
    B, T, C = y.shape
    if C != 2 * Hk * K + H * V:
        raise ValueError("channel count does not match q | k | v")
    q = y[:, :, :Hk * K].unflatten(2, (Hk, K))
    k = y[:, :, Hk * K:2 * Hk * K].unflatten(2, (Hk, K))
    v = y[:, :, 2 * Hk * K:].unflatten(2, (H, V))
    return q, k, v


def prefill_chain(x, w, a, b, A_log, dt_bias, *, Hk, K, H, V, initial_state=None,
                  cu_seqlens=None, scale=1.0, qk_l2norm=True, bufs: dict | None = None):
    """conv1d + SiLU -> q|k|v views -> gates -> chunked forward. Returns
    (o, final_state). `bufs` may hold preallocated 'y', 'g', 'beta', 'o',
    'final_state' and 'workspace' tensors."""
    bufs = {} if bufs is None else bufs
    y = gdn_conv1d_causal(x, w, y=bufs.get("y"), cu_seqlens=cu_seqlens, silu=True)
    q, k, v = split_qkv(y, Hk, K, H, V)
    g, beta = gdn_gate_prepare(a, b, A_log, dt_bias, g=bufs.get("g"), beta=bufs.get("beta"))
    return gdn_chunk_fwd(q, k, v, g, beta, initial_state=initial_state, cu_seqlens=cu_seqlens,
                         scale=scale, qk_l2norm=qk_l2norm, workspace=bufs.get("workspace"),
                         o=bufs.get("o"), final_state=bufs.get("final_state"))
