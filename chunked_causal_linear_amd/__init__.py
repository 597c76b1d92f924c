"""Chunked causal linear attention on MI355X: thin Python binding over liblasp.so.

Only argument marshalling lives here; every step runs in the HIP library.  torch
tensors serve as device buffers and torch's current stream is the HIP stream.
The binding raises if the library is missing: there is no fallback path.

  fwd(Q, K, V, chunk, ...) -> (O, M_out, state_cache)
  bwd(Q, K, V, dO, chunk, ...) -> (dQ, dK, dV, dM_in)
  fwd_bidir / bwd_bidir: the unmasked (bidirectional) form, bf16, no decay
  fwd_gated / bwd_gated: per-token, per-key-channel gates (log-gates in, their
                         gradient out), chunk 64

Semantics, layouts and error codes are those of include/lasp.h ("Linear Attention
Sequence Parallelism", arXiv 2404.02882, Sec. 3.2, Algorithms 2 and 3).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "bwd", "fwd_bidir", "bwd_bidir", "fwd_gated", "bwd_gated", "LaspError", "lib",
           "Shape", "LASP_FP32", "LASP_BF16", "state_cache_bytes", "fwd_workspace_bytes",
           "bwd_workspace_bytes", "gated_state_cache_bytes", "gated_fwd_workspace_bytes",
           "gated_bwd_workspace_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblasp.so")
LASP_FP32, LASP_BF16 = 0, 1
_lib = None


class LaspError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: status %d (%s)" % (what, status, _status_string(status)))


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "N", "d", "chunk", "nseq")]


def lib():
    """The loaded liblasp.so (ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("liblasp.so is not built (run __graft_entry__.build() or "
                              "python -m chunked_causal_linear_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        SP = ctypes.POINTER(Shape)
        L.lasp_state_cache_bytes.argtypes = [SP, ctypes.c_int]
        L.lasp_state_cache_bytes.restype = S
        for f in (L.lasp_fwd_workspace_bytes, L.lasp_bwd_workspace_bytes):
            f.argtypes = [SP, ctypes.c_int, ctypes.c_int]
            f.restype = S
        L.lasp_fwd.argtypes = [SP, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, S, P]
        L.lasp_fwd.restype = ctypes.c_int
        L.lasp_bwd.argtypes = [SP, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.lasp_bwd.restype = ctypes.c_int
        L.lasp_fwd_ex.argtypes = L.lasp_fwd.argtypes + [P]
        L.lasp_fwd_ex.restype = ctypes.c_int
        L.lasp_bwd_ex.argtypes = L.lasp_bwd.argtypes + [P]
        L.lasp_bwd_ex.restype = ctypes.c_int
        L.lasp_fwd_bidir.argtypes = [SP, ctypes.c_int, P, P, P, P, P, P, P, P, P, S, P]
        L.lasp_fwd_bidir.restype = ctypes.c_int
        L.lasp_bwd_bidir.argtypes = [SP, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.lasp_bwd_bidir.restype = ctypes.c_int
        L.lasp_gated_state_cache_bytes.argtypes = [SP, ctypes.c_int]
        L.lasp_gated_state_cache_bytes.restype = S
        for f in (L.lasp_gated_fwd_workspace_bytes, L.lasp_gated_bwd_workspace_bytes):
            f.argtypes = [SP, ctypes.c_int, ctypes.c_int]
            f.restype = S
        L.lasp_fwd_gated.argtypes = [SP, ctypes.c_int, P, P, P, P, P, P, P, P, P, P, S, P]
        L.lasp_fwd_gated.restype = ctypes.c_int
        L.lasp_bwd_gated.argtypes = [SP, ctypes.c_int] + [P] * 15 + [S, P]
        L.lasp_bwd_gated.restype = ctypes.c_int
        L.lasp_fwd_gated_ex.argtypes = L.lasp_fwd_gated.argtypes + [P]
        L.lasp_fwd_gated_ex.restype = ctypes.c_int
        L.lasp_bwd_gated_ex.argtypes = L.lasp_bwd_gated.argtypes + [P]
        L.lasp_bwd_gated_ex.restype = ctypes.c_int
        L.lasp_status_string.argtypes = [ctypes.c_int]
        L.lasp_status_string.restype = ctypes.c_char_p
        L.lasp_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _status_string(st):
    try:
        return lib().lasp_status_string(int(st)).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return LASP_BF16
    if t.dtype == torch.float32:
        return LASP_FP32
    raise TypeError("Q/K/V must be bfloat16 or float32, got %s" % t.dtype)


def _shape(Q, chunk, cu_seqlens):
    B, H, N, d = Q.shape
    nseq = 0 if cu_seqlens is None else int(cu_seqlens.numel()) - 1
    return Shape(B, H, N, d, int(chunk), nseq)


def state_cache_bytes(shape: Shape, dtype: int) -> int:
    return int(lib().lasp_state_cache_bytes(ctypes.byref(shape), dtype))


def fwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_fwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def bwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_bwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, device, dtype=None, shape=None):
    if t is None:
        return
    if t.device != device:
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd(Q, K, V, chunk, decay=None, cu_seqlens=None, M_in=None, *, want_m_out=True,
        want_state_cache=True, out=None, workspace=None, events=None):
    """Forward pass.  Q, K, V: [B, H, N, d] bf16 or fp32 CUDA tensors.
    decay: float32 [H] CUDA tensor or None.  cu_seqlens: int32 [nseq+1] CUDA tensor
    or None.  M_in: float32 [S, H, d, d] or None.  Returns (O, M_out, state_cache)
    (M_out / state_cache are None when not requested).  events: optional ctypes
    array of 4 hipEvent_t handles for per-kernel timing (see lasp_fwd_ex)."""
    import torch
    dev = Q.device
    S_ = _shape(Q, chunk, cu_seqlens)
    dt = _dtype_code(Q)
    nS = S_.nseq if S_.nseq else S_.B
    st_shape = (nS, S_.H, S_.d, S_.d)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_dev(n, t, dev, Q.dtype, Q.shape)
    _check_dev("decay", decay, dev, torch.float32, (S_.H,))
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    _check_dev("M_in", M_in, dev, torch.float32, st_shape)
    O = torch.empty_like(Q) if out is None else out
    M_out = torch.empty(st_shape, dtype=torch.float32, device=dev) if want_m_out else None
    cache = None
    if want_state_cache:
        cache = torch.empty(max(1, state_cache_bytes(S_, dt)), dtype=torch.uint8, device=dev)
    nws = fwd_workspace_bytes(S_, dt, cache is not None)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    rc = lib().lasp_fwd_ex(ctypes.byref(S_), dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(decay),
                           _ptr(cu_seqlens), _ptr(M_in), _ptr(O), _ptr(M_out), _ptr(cache),
                           _ptr(workspace), nws, _stream(dev), events)
    if rc != 0:
        raise LaspError(rc, "lasp_fwd")
    return O, M_out, cache


def bwd(Q, K, V, dO, chunk, decay=None, cu_seqlens=None, M_in=None, dM_out=None,
        state_cache=None, *, want_dm_in=True, workspace=None, events=None):
    """Backward pass for l = <dO, O> + <dM_out, M_out>.  state_cache: the buffer
    fwd returned for the same inputs, or None (states are recomputed).
    Returns (dQ, dK, dV, dM_in)."""
    import torch
    dev = Q.device
    S_ = _shape(Q, chunk, cu_seqlens)
    dt = _dtype_code(Q)
    nS = S_.nseq if S_.nseq else S_.B
    st_shape = (nS, S_.H, S_.d, S_.d)
    for n, t in (("Q", Q), ("K", K), ("V", V), ("dO", dO)):
        _check_dev(n, t, dev, Q.dtype, Q.shape)
    _check_dev("decay", decay, dev, torch.float32, (S_.H,))
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    _check_dev("M_in", M_in, dev, torch.float32, st_shape)
    _check_dev("dM_out", dM_out, dev, torch.float32, st_shape)
    if state_cache is not None:
        _check_dev("state_cache", state_cache, dev, torch.uint8)
        if state_cache.numel() < state_cache_bytes(S_, dt):
            raise ValueError("state_cache is smaller than lasp_state_cache_bytes()")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dM_in = torch.empty(st_shape, dtype=torch.float32, device=dev) if want_dm_in else None
    nws = bwd_workspace_bytes(S_, dt, state_cache is not None)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    rc = lib().lasp_bwd_ex(ctypes.byref(S_), dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(dO),
                           _ptr(decay), _ptr(cu_seqlens), _ptr(M_in), _ptr(dM_out),
                           _ptr(state_cache), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dM_in),
                           _ptr(workspace), nws, _stream(dev), events)
    if rc != 0:
        raise LaspError(rc, "lasp_bwd")
    return dQ, dK, dV, dM_in


def fwd_bidir(Q, K, V, chunk=256, cu_seqlens=None, M_in=None, *, want_m_out=True,
              want_state_cache=True, workspace=None):
    """Unmasked (bidirectional) forward, bf16: O = Q (M_in + sum_i k_i^T v_i) per
    sequence and head (lasp_fwd_bidir).  chunk only sets the work split.
    Returns (O, M_out, state_cache)."""
    import torch
    dev = Q.device
    S_ = _shape(Q, chunk, cu_seqlens)
    dt = _dtype_code(Q)
    nS = S_.nseq if S_.nseq else S_.B
    st_shape = (nS, S_.H, S_.d, S_.d)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_dev(n, t, dev, Q.dtype, Q.shape)
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    _check_dev("M_in", M_in, dev, torch.float32, st_shape)
    O = torch.empty_like(Q)
    M_out = torch.empty(st_shape, dtype=torch.float32, device=dev) if want_m_out else None
    cache = None
    if want_state_cache:
        cache = torch.empty(max(1, state_cache_bytes(S_, dt)), dtype=torch.uint8, device=dev)
    nws = fwd_workspace_bytes(S_, dt, cache is not None)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    rc = lib().lasp_fwd_bidir(ctypes.byref(S_), dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(cu_seqlens),
                              _ptr(M_in), _ptr(O), _ptr(M_out), _ptr(cache), _ptr(workspace), nws,
                              _stream(dev))
    if rc != 0:
        raise LaspError(rc, "lasp_fwd_bidir")
    return O, M_out, cache


def bwd_bidir(Q, K, V, dO, chunk=256, cu_seqlens=None, M_in=None, dM_out=None,
              state_cache=None, *, want_dm_in=True, workspace=None):
    """Unmasked (bidirectional) backward for l = <dO, O> + <dM_out, M_out>
    (lasp_bwd_bidir).  Returns (dQ, dK, dV, dM_in)."""
    import torch
    dev = Q.device
    S_ = _shape(Q, chunk, cu_seqlens)
    dt = _dtype_code(Q)
    nS = S_.nseq if S_.nseq else S_.B
    st_shape = (nS, S_.H, S_.d, S_.d)
    for n, t in (("Q", Q), ("K", K), ("V", V), ("dO", dO)):
        _check_dev(n, t, dev, Q.dtype, Q.shape)
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    _check_dev("M_in", M_in, dev, torch.float32, st_shape)
    _check_dev("dM_out", dM_out, dev, torch.float32, st_shape)
    if state_cache is not None:
        _check_dev("state_cache", state_cache, dev, torch.uint8)
        if state_cache.numel() < state_cache_bytes(S_, dt):
            raise ValueError("state_cache is smaller than lasp_state_cache_bytes()")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dM_in = torch.empty(st_shape, dtype=torch.float32, device=dev) if want_dm_in else None
    nws = bwd_workspace_bytes(S_, dt, state_cache is not None)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    rc = lib().lasp_bwd_bidir(ctypes.byref(S_), dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(dO),
                              _ptr(cu_seqlens), _ptr(M_in), _ptr(dM_out), _ptr(state_cache),
                              _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dM_in), _ptr(workspace), nws,
                              _stream(dev))
    if rc != 0:
        raise LaspError(rc, "lasp_bwd_bidir")
    return dQ, dK, dV, dM_in


def gated_state_cache_bytes(shape: Shape, dtype: int) -> int:
    return int(lib().lasp_gated_state_cache_bytes(ctypes.byref(shape), dtype))


def gated_fwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_gated_fwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def gated_bwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_gated_bwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def fwd_gated(Q, K, V, log_g, chunk=64, cu_seqlens=None, M_in=None, *, want_m_out=True,
              want_state_cache=True, workspace=None, events=None):
    """Gated forward (lasp_fwd_gated): kv_p = Diag(g_p) kv_{p-1} + k_p^T v_p,
    o_p = q_p kv_p, with log_g = log g as a float32 [B, H, N, d] tensor.
    Returns (O, M_out, state_cache)."""
    import torch
    dev = Q.device
    S_ = _shape(Q, chunk, cu_seqlens)
    dt = _dtype_code(Q)
    nS = S_.nseq if S_.nseq else S_.B
    st_shape = (nS, S_.H, S_.d, S_.d)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_dev(n, t, dev, Q.dtype, Q.shape)
    _check_dev("log_g", log_g, dev, torch.float32, Q.shape)
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    _check_dev("M_in", M_in, dev, torch.float32, st_shape)
    O = torch.empty_like(Q)
    M_out = torch.empty(st_shape, dtype=torch.float32, device=dev) if want_m_out else None
    cache = None
    if want_state_cache:
        cache = torch.empty(max(1, gated_state_cache_bytes(S_, dt)), dtype=torch.uint8, device=dev)
    nws = gated_fwd_workspace_bytes(S_, dt, cache is not None)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    rc = lib().lasp_fwd_gated_ex(ctypes.byref(S_), dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(log_g),
                                 _ptr(cu_seqlens), _ptr(M_in), _ptr(O), _ptr(M_out), _ptr(cache),
                                 _ptr(workspace), nws, _stream(dev), events)
    if rc != 0:
        raise LaspError(rc, "lasp_fwd_gated")
    return O, M_out, cache


def bwd_gated(Q, K, V, log_g, dO, chunk=64, cu_seqlens=None, M_in=None, dM_out=None,
              state_cache=None, *, want_dm_in=True, workspace=None, events=None):
    """Gated backward for l = <dO, O> + <dM_out, M_out> (lasp_bwd_gated).
    Returns (dQ, dK, dV, dlog_g, dM_in)."""
    import torch
    dev = Q.device
    S_ = _shape(Q, chunk, cu_seqlens)
    dt = _dtype_code(Q)
    nS = S_.nseq if S_.nseq else S_.B
    st_shape = (nS, S_.H, S_.d, S_.d)
    for n, t in (("Q", Q), ("K", K), ("V", V), ("dO", dO)):
        _check_dev(n, t, dev, Q.dtype, Q.shape)
    _check_dev("log_g", log_g, dev, torch.float32, Q.shape)
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    _check_dev("M_in", M_in, dev, torch.float32, st_shape)
    _check_dev("dM_out", dM_out, dev, torch.float32, st_shape)
    if state_cache is not None:
        _check_dev("state_cache", state_cache, dev, torch.uint8)
        if state_cache.numel() < gated_state_cache_bytes(S_, dt):
            raise ValueError("state_cache is smaller than lasp_gated_state_cache_bytes()")
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dLG = torch.empty_like(log_g)
    dM_in = torch.empty(st_shape, dtype=torch.float32, device=dev) if want_dm_in else None
    nws = gated_bwd_workspace_bytes(S_, dt, state_cache is not None)
    if workspace is None or workspace.numel() < nws:
        workspace = torch.empty(max(1, nws), dtype=torch.uint8, device=dev)
    rc = lib().lasp_bwd_gated_ex(ctypes.byref(S_), dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(log_g),
                                 _ptr(dO), _ptr(cu_seqlens), _ptr(M_in), _ptr(dM_out),
                                 _ptr(state_cache), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dLG),
                                 _ptr(dM_in), _ptr(workspace), nws, _stream(dev), events)
    if rc != 0:
        raise LaspError(rc, "lasp_bwd_gated")
    return dQ, dK, dV, dLG, dM_in
