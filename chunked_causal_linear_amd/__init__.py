"""Chunked causal linear attention on MI355X: thin Python binding over liblasp.so.

Only argument marshalling lives here; every step runs in the HIP library.  torch
tensors serve as device buffers and torch's current stream is the HIP stream.
The binding raises if the library is missing: there is no fallback path.

  fwd(Q, K, V, chunk, ...) -> (O, M_out, state_cache)
  bwd(Q, K, V, dO, chunk, ...) -> (dQ, dK, dV, dM_in)
  fwd_bidir / bwd_bidir: the unmasked (bidirectional) form, no decay
  fwd_gated / bwd_gated: per-token, per-key-channel gates (log-gates in, their
                         gradient out); the kernels use 64-token chunks
  fwd_norm / bwd_norm: output rows normalised (Norm of LASP Eq. 2)
  autograd (submodule): lasp_attention, lasp_gated_attention and
                        lasp_bidir_attention as torch.autograd.Functions

Semantics, layouts and error codes are those of include/lasp.h ("Linear Attention
Sequence Parallelism", arXiv 2404.02882, Sec. 3.2, Algorithms 2 and 3).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fwd", "fwd_noalloc", "bwd", "fwd_norm", "bwd_norm", "fwd_bidir", "bwd_bidir", "fwd_gated", "bwd_gated", "LaspError", "lib",
           "Shape", "Sizes", "LASP_FP32", "LASP_BF16", "query_sizes", "state_cache_bytes",
           "fwd_workspace_bytes", "bwd_workspace_bytes", "gated_state_cache_bytes",
           "gated_fwd_workspace_bytes", "gated_bwd_workspace_bytes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblasp.so")
LASP_FP32, LASP_BF16 = 0, 1
FORM_CAUSAL, FORM_GATED, FORM_NORM = 0, 1, 2
_lib = None


class LaspError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: status %d (%s)" % (what, status, _status_string(status)))


class Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "H", "N", "d", "chunk", "nseq")]


class Sizes(ctypes.Structure):
    _fields_ = [("state_cache", ctypes.c_size_t), ("fwd_workspace", ctypes.c_size_t * 2),
                ("bwd_workspace", ctypes.c_size_t * 2), ("segment_chunks", ctypes.c_int)]


def lib():
    """The loaded liblasp.so (ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("liblasp.so is not built (run __graft_entry__.build() or "
                              "python -m chunked_causal_linear_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        SP = ctypes.POINTER(Shape)

        def sig(f, args, res=I):
            f.argtypes, f.restype = args, res

        sig(L.lasp_state_cache_bytes, [SP, I], S)
        sig(L.lasp_gated_state_cache_bytes, [SP, I], S)
        for f in (L.lasp_fwd_workspace_bytes, L.lasp_bwd_workspace_bytes,
                  L.lasp_gated_fwd_workspace_bytes, L.lasp_gated_bwd_workspace_bytes):
            sig(f, [SP, I, I], S)
        sig(L.lasp_query_sizes, [SP, I, I, I, ctypes.POINTER(Sizes)])
        # entry points: shape, dtype, pointers..., workspace_bytes, stream
        sig(L.lasp_fwd, [SP, I] + [P] * 10 + [S, P])
        sig(L.lasp_bwd, [SP, I] + [P] * 14 + [S, P])
        sig(L.lasp_fwd_bidir, [SP, I] + [P] * 9 + [S, P])
        sig(L.lasp_bwd_bidir, [SP, I] + [P] * 13 + [S, P])
        sig(L.lasp_fwd_gated, [SP, I] + [P] * 10 + [S, P])
        sig(L.lasp_bwd_gated, [SP, I] + [P] * 15 + [S, P])
        # _ex variants: + events, segment_chunks
        for n in ("fwd", "bwd", "fwd_bidir", "bwd_bidir", "fwd_gated", "bwd_gated"):
            base = getattr(L, "lasp_" + n)
            sig(getattr(L, "lasp_%s_ex" % n), base.argtypes + [P, I])
        sig(L.lasp_fwd_noalloc, [SP, I] + [P] * 9 + [P])
        sig(L.lasp_fwd_norm, [SP, I] + [P] * 11 + [S, P])
        sig(L.lasp_bwd_norm, [SP, I] + [P] * 16 + [S, P])
        sig(L.lasp_noalloc_scratch_bytes, [], S)
        sig(L.lasp_status_string, [I], ctypes.c_char_p)
        sig(L.lasp_version, [])
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


def query_sizes(shape: Shape, dtype: int, form: int = FORM_CAUSAL,
                segment_chunks: int = 0) -> Sizes:
    """All buffer sizes for a call (lasp_query_sizes)."""
    out = Sizes()
    rc = lib().lasp_query_sizes(ctypes.byref(shape), dtype, form, int(segment_chunks),
                                ctypes.byref(out))
    if rc != 0:
        raise LaspError(rc, "lasp_query_sizes")
    return out


def state_cache_bytes(shape: Shape, dtype: int) -> int:
    return int(lib().lasp_state_cache_bytes(ctypes.byref(shape), dtype))


def fwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_fwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def bwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_bwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def gated_state_cache_bytes(shape: Shape, dtype: int) -> int:
    return int(lib().lasp_gated_state_cache_bytes(ctypes.byref(shape), dtype))


def gated_fwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_gated_fwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


def gated_bwd_workspace_bytes(shape: Shape, dtype: int, with_cache: bool) -> int:
    return int(lib().lasp_gated_bwd_workspace_bytes(ctypes.byref(shape), dtype, int(with_cache)))


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


class _Call:
    """Validated arguments and sizes shared by every entry point: the token
    tensors (the layout of Q), the optional packed-batch table, the states, and
    the workspace / state-cache sizes for the call's form and segment length."""

    def __init__(self, Q, chunk, cu_seqlens, tokens, states, form, segment_chunks,
                 log_g=None, decay=None):
        import torch
        self.dev = Q.device
        if self.dev.type != "cuda":
            raise ValueError("tensors must be on a GPU (got %s)" % self.dev)
        self.S = _shape(Q, chunk, cu_seqlens)
        self.dt = _dtype_code(Q)
        nS = self.S.nseq if self.S.nseq else self.S.B
        self.st_shape = (nS, self.S.H, self.S.d, self.S.d)
        for n, t in tokens:
            _check_dev(n, t, self.dev, Q.dtype, Q.shape)
        _check_dev("log_g", log_g, self.dev, torch.float32, Q.shape)
        _check_dev("decay", decay, self.dev, torch.float32, (self.S.H,))
        _check_dev("cu_seqlens", cu_seqlens, self.dev, torch.int32)
        for n, t in states:
            _check_dev(n, t, self.dev, torch.float32, self.st_shape)
        self.seg = int(segment_chunks)
        self.sizes = query_sizes(self.S, self.dt, form, self.seg)

    def empty_state(self, want):
        import torch
        return torch.empty(self.st_shape, dtype=torch.float32, device=self.dev) if want else None

    def new_cache(self, want):
        import torch
        if not want:
            return None
        return torch.empty(max(1, self.sizes.state_cache), dtype=torch.uint8, device=self.dev)

    def check_cache(self, cache):
        import torch
        if cache is not None:
            _check_dev("state_cache", cache, self.dev, torch.uint8)
            if cache.numel() < self.sizes.state_cache:
                raise ValueError("state_cache is smaller than the call's state-cache size")

    def workspace(self, need, given):
        import torch
        if given is not None:
            _check_dev("workspace", given, self.dev, torch.uint8)
            if given.numel() >= need:
                return given
        return torch.empty(max(1, need), dtype=torch.uint8, device=self.dev)


def _run(name, c, args, ws, need, events):
    rc = getattr(lib(), name + "_ex")(ctypes.byref(c.S), c.dt, *args, _ptr(ws), need,
                                       _stream(c.dev), events, c.seg)
    if rc != 0:
        raise LaspError(rc, name)


def fwd(Q, K, V, chunk, decay=None, cu_seqlens=None, M_in=None, *, want_m_out=True,
        want_state_cache=True, out=None, workspace=None, events=None, segment_chunks=0):
    """Forward pass.  Q, K, V: [B, H, N, d] bf16 or fp32 CUDA tensors.
    decay: float32 [H] CUDA tensor or None.  cu_seqlens: int32 [nseq+1] CUDA tensor
    or None.  M_in: float32 [S, H, d, d] or None.  out: an optional preallocated O
    (Q's dtype, shape, device; contiguous).  Returns (O, M_out, state_cache)
    (M_out / state_cache are None when not requested).  events: optional ctypes
    array of 4 hipEvent_t handles for per-kernel timing; segment_chunks: 0 or an
    explicit segment length (see lasp_fwd_ex)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V), ("out", out)],
              [("M_in", M_in)], FORM_CAUSAL, segment_chunks, decay=decay)
    O = torch.empty_like(Q) if out is None else out
    M_out = c.empty_state(want_m_out)
    cache = c.new_cache(want_state_cache)
    need = c.sizes.fwd_workspace[cache is not None]
    ws = c.workspace(need, workspace)
    _run("lasp_fwd", c, [_ptr(Q), _ptr(K), _ptr(V), _ptr(decay), _ptr(cu_seqlens), _ptr(M_in),
                         _ptr(O), _ptr(M_out), _ptr(cache)], ws, need, events)
    return O, M_out, cache


def fwd_noalloc(Q, K, V, chunk, decay=None, cu_seqlens=None, M_in=None, *, out, M_out=None,
                state_cache=None):
    """Allocation-free forward (lasp_fwd_noalloc): the caller passes every
    output buffer (O; optionally M_out and a state cache of the call's
    state-cache size) and the library takes its scratch from a static device
    array, so the call itself allocates nothing.  Returns (O, M_out, state_cache)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V), ("out", out)],
              [("M_in", M_in), ("M_out", M_out)], FORM_CAUSAL, 0, decay=decay)
    c.check_cache(state_cache)
    rc = lib().lasp_fwd_noalloc(ctypes.byref(c.S), c.dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(decay),
                                _ptr(cu_seqlens), _ptr(M_in), _ptr(out), _ptr(M_out),
                                _ptr(state_cache), _stream(c.dev))
    if rc != 0:
        raise LaspError(rc, "lasp_fwd_noalloc")
    return out, M_out, state_cache


def bwd(Q, K, V, dO, chunk, decay=None, cu_seqlens=None, M_in=None, dM_out=None,
        state_cache=None, *, want_dm_in=True, out=None, workspace=None, events=None,
        segment_chunks=0):
    """Backward pass for l = <dO, O> + <dM_out, M_out>.  state_cache: the buffer
    fwd returned for the same inputs (and segment_chunks), or None (states are
    recomputed).  out: optional preallocated (dQ, dK, dV), each with Q's dtype,
    shape and device, contiguous.  Returns (dQ, dK, dV, dM_in)."""
    import torch
    outs = (None, None, None) if out is None else tuple(out)
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V), ("dO", dO),
                                     ("dQ", outs[0]), ("dK", outs[1]), ("dV", outs[2])],
              [("M_in", M_in), ("dM_out", dM_out)], FORM_CAUSAL, segment_chunks, decay=decay)
    c.check_cache(state_cache)
    dQ, dK, dV = (torch.empty_like(Q) if t is None else t for t in outs)
    dM_in = c.empty_state(want_dm_in)
    need = c.sizes.bwd_workspace[state_cache is not None]
    ws = c.workspace(need, workspace)
    _run("lasp_bwd", c, [_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(decay), _ptr(cu_seqlens),
                         _ptr(M_in), _ptr(dM_out), _ptr(state_cache), _ptr(dQ), _ptr(dK),
                         _ptr(dV), _ptr(dM_in)], ws, need, events)
    return dQ, dK, dV, dM_in


def fwd_norm(Q, K, V, chunk, decay=None, cu_seqlens=None, M_in=None, *, want_m_out=True,
             want_state_cache=True, workspace=None):
    """Forward with the output normalised row by row (lasp_fwd_norm: Norm of LASP
    Eq. 2 read as an RMS normalisation over d, eps 1e-6, no gain).
    Returns (Y, rstd, M_out, state_cache); rstd is float32 [B, H, N]."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V)], [("M_in", M_in)],
              FORM_NORM, 0, decay=decay)
    Y = torch.empty_like(Q)
    rstd = torch.empty(Q.shape[:3], dtype=torch.float32, device=c.dev)
    M_out = c.empty_state(want_m_out)
    cache = c.new_cache(want_state_cache)
    need = c.sizes.fwd_workspace[cache is not None]
    ws = c.workspace(need, workspace)
    rc = lib().lasp_fwd_norm(ctypes.byref(c.S), c.dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(decay),
                             _ptr(cu_seqlens), _ptr(M_in), _ptr(Y), _ptr(rstd), _ptr(M_out),
                             _ptr(cache), _ptr(ws), need, _stream(c.dev))
    if rc != 0:
        raise LaspError(rc, "lasp_fwd_norm")
    return Y, rstd, M_out, cache


def bwd_norm(Q, K, V, Y, rstd, dY, chunk, decay=None, cu_seqlens=None, M_in=None, dM_out=None,
             state_cache=None, *, want_dm_in=True, workspace=None):
    """Backward of the normalised form for l = <dY, Y> + <dM_out, M_out>
    (lasp_bwd_norm), given the forward's Y and rstd.  Returns (dQ, dK, dV, dM_in)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V), ("Y", Y), ("dY", dY)],
              [("M_in", M_in), ("dM_out", dM_out)], FORM_NORM, 0, decay=decay)
    _check_dev("rstd", rstd, c.dev, torch.float32, Q.shape[:3])
    c.check_cache(state_cache)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dM_in = c.empty_state(want_dm_in)
    need = c.sizes.bwd_workspace[state_cache is not None]
    ws = c.workspace(need, workspace)
    rc = lib().lasp_bwd_norm(ctypes.byref(c.S), c.dt, _ptr(Q), _ptr(K), _ptr(V), _ptr(Y),
                             _ptr(rstd), _ptr(dY), _ptr(decay), _ptr(cu_seqlens), _ptr(M_in),
                             _ptr(dM_out), _ptr(state_cache), _ptr(dQ), _ptr(dK), _ptr(dV),
                             _ptr(dM_in), _ptr(ws), need, _stream(c.dev))
    if rc != 0:
        raise LaspError(rc, "lasp_bwd_norm")
    return dQ, dK, dV, dM_in


def fwd_bidir(Q, K, V, chunk=256, cu_seqlens=None, M_in=None, *, want_m_out=True,
              want_state_cache=True, workspace=None, events=None, segment_chunks=0):
    """Unmasked (bidirectional) forward: O = Q (M_in + sum_i k_i^T v_i) per
    sequence and head (lasp_fwd_bidir).  chunk only sets the work split.
    Returns (O, M_out, state_cache)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V)], [("M_in", M_in)],
              FORM_CAUSAL, segment_chunks)
    O = torch.empty_like(Q)
    M_out = c.empty_state(want_m_out)
    cache = c.new_cache(want_state_cache)
    need = c.sizes.fwd_workspace[cache is not None]
    ws = c.workspace(need, workspace)
    _run("lasp_fwd_bidir", c, [_ptr(Q), _ptr(K), _ptr(V), _ptr(cu_seqlens), _ptr(M_in), _ptr(O),
                               _ptr(M_out), _ptr(cache)], ws, need, events)
    return O, M_out, cache


def bwd_bidir(Q, K, V, dO, chunk=256, cu_seqlens=None, M_in=None, dM_out=None,
              state_cache=None, *, want_dm_in=True, workspace=None, events=None,
              segment_chunks=0):
    """Unmasked (bidirectional) backward for l = <dO, O> + <dM_out, M_out>
    (lasp_bwd_bidir).  Returns (dQ, dK, dV, dM_in)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V), ("dO", dO)],
              [("M_in", M_in), ("dM_out", dM_out)], FORM_CAUSAL, segment_chunks)
    c.check_cache(state_cache)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dM_in = c.empty_state(want_dm_in)
    need = c.sizes.bwd_workspace[state_cache is not None]
    ws = c.workspace(need, workspace)
    _run("lasp_bwd_bidir", c, [_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(cu_seqlens), _ptr(M_in),
                               _ptr(dM_out), _ptr(state_cache), _ptr(dQ), _ptr(dK), _ptr(dV),
                               _ptr(dM_in)], ws, need, events)
    return dQ, dK, dV, dM_in


def fwd_gated(Q, K, V, log_g, chunk=64, cu_seqlens=None, M_in=None, *, want_m_out=True,
              want_state_cache=True, workspace=None, events=None, segment_chunks=0):
    """Gated forward (lasp_fwd_gated): kv_p = Diag(g_p) kv_{p-1} + k_p^T v_p,
    o_p = q_p kv_p, with log_g = log g as a float32 [B, H, N, d] tensor.
    Returns (O, M_out, state_cache)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V)], [("M_in", M_in)],
              FORM_GATED, segment_chunks, log_g=log_g)
    O = torch.empty_like(Q)
    M_out = c.empty_state(want_m_out)
    cache = c.new_cache(want_state_cache)
    need = c.sizes.fwd_workspace[cache is not None]
    ws = c.workspace(need, workspace)
    _run("lasp_fwd_gated", c, [_ptr(Q), _ptr(K), _ptr(V), _ptr(log_g), _ptr(cu_seqlens),
                               _ptr(M_in), _ptr(O), _ptr(M_out), _ptr(cache)], ws, need, events)
    return O, M_out, cache


def bwd_gated(Q, K, V, log_g, dO, chunk=64, cu_seqlens=None, M_in=None, dM_out=None,
              state_cache=None, *, want_dm_in=True, workspace=None, events=None,
              segment_chunks=0):
    """Gated backward for l = <dO, O> + <dM_out, M_out> (lasp_bwd_gated).
    Returns (dQ, dK, dV, dlog_g, dM_in)."""
    import torch
    c = _Call(Q, chunk, cu_seqlens, [("Q", Q), ("K", K), ("V", V), ("dO", dO)],
              [("M_in", M_in), ("dM_out", dM_out)], FORM_GATED, segment_chunks, log_g=log_g)
    c.check_cache(state_cache)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    dLG = torch.empty_like(log_g)
    dM_in = c.empty_state(want_dm_in)
    need = c.sizes.bwd_workspace[state_cache is not None]
    ws = c.workspace(need, workspace)
    _run("lasp_bwd_gated", c, [_ptr(Q), _ptr(K), _ptr(V), _ptr(log_g), _ptr(dO),
                               _ptr(cu_seqlens), _ptr(M_in), _ptr(dM_out), _ptr(state_cache),
                               _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dLG), _ptr(dM_in)],
         ws, need, events)
    return dQ, dK, dV, dLG, dM_in
