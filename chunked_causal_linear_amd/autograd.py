"""torch.autograd.Function wrappers over the forward / backward entry points.

The forward keeps the state cache of "Linear Attention Sequence Parallelism"
(Sec. 3.4, KV State Caching) in the autograd context, so the backward reads
the forward's chunk states instead of recomputing them (Algorithm 3 takes the
cached KV of Algorithm 2).  Both outputs, O and the final state M_out, may
carry gradients; a missing gradient is passed to the library as zero (dO) or
as no array (dM_out).  The decay rates and log-gates' roles follow the entry
points: decay is a constant (no gradient), log_g gets its gradient.

Every call goes to the HIP library; tensors must be on a GPU.
"""
from __future__ import annotations

import torch

from . import bwd, bwd_bidir, bwd_gated, bwd_norm, fwd, fwd_bidir, fwd_gated, fwd_norm

__all__ = ["lasp_attention", "lasp_gated_attention", "lasp_bidir_attention"]


def _grad_tokens(g, like):
    """The token gradient as the library takes it: Q's dtype, contiguous;
    zeros when the output had no gradient."""
    if g is None:
        return torch.zeros_like(like)
    return g.to(like.dtype).contiguous()


def _grad_state(g):
    return None if g is None else g.to(torch.float32).contiguous()


class _Causal(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, M_in, decay, cu_seqlens, chunk, norm):
        if norm:
            O, rstd, M_out, cache = fwd_norm(Q, K, V, chunk, decay, cu_seqlens, M_in)
            ctx.save_for_backward(Q, K, V, M_in, decay, cu_seqlens, cache, O, rstd)
        else:
            O, M_out, cache = fwd(Q, K, V, chunk, decay, cu_seqlens, M_in)
            ctx.save_for_backward(Q, K, V, M_in, decay, cu_seqlens, cache)
        ctx.chunk, ctx.norm = chunk, norm
        return O, M_out

    @staticmethod
    def backward(ctx, dO, dM_out):
        Q, K, V, M_in, decay, cu_seqlens, cache, *yr = ctx.saved_tensors
        want_dm_in = M_in is not None and ctx.needs_input_grad[3]
        dO = _grad_tokens(dO, Q)
        if ctx.norm:
            Y, rstd = yr
            dQ, dK, dV, dM_in = bwd_norm(Q, K, V, Y, rstd, dO, ctx.chunk, decay, cu_seqlens, M_in,
                                         _grad_state(dM_out), cache, want_dm_in=want_dm_in)
        else:
            dQ, dK, dV, dM_in = bwd(Q, K, V, dO, ctx.chunk, decay, cu_seqlens, M_in,
                                    _grad_state(dM_out), cache, want_dm_in=want_dm_in)
        return dQ, dK, dV, dM_in, None, None, None, None


class _Gated(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, log_g, M_in, cu_seqlens, chunk):
        O, M_out, cache = fwd_gated(Q, K, V, log_g, chunk, cu_seqlens, M_in)
        ctx.save_for_backward(Q, K, V, log_g, M_in, cu_seqlens, cache)
        ctx.chunk = chunk
        return O, M_out

    @staticmethod
    def backward(ctx, dO, dM_out):
        Q, K, V, log_g, M_in, cu_seqlens, cache = ctx.saved_tensors
        want_dm_in = M_in is not None and ctx.needs_input_grad[4]
        dQ, dK, dV, dLG, dM_in = bwd_gated(Q, K, V, log_g, _grad_tokens(dO, Q), ctx.chunk,
                                           cu_seqlens, M_in, _grad_state(dM_out), cache,
                                           want_dm_in=want_dm_in)
        return dQ, dK, dV, dLG, dM_in, None, None


class _Bidir(torch.autograd.Function):
    @staticmethod
    def forward(ctx, Q, K, V, M_in, cu_seqlens, chunk):
        O, M_out, cache = fwd_bidir(Q, K, V, chunk, cu_seqlens, M_in)
        ctx.save_for_backward(Q, K, V, M_in, cu_seqlens, cache)
        ctx.chunk = chunk
        return O, M_out

    @staticmethod
    def backward(ctx, dO, dM_out):
        Q, K, V, M_in, cu_seqlens, cache = ctx.saved_tensors
        want_dm_in = M_in is not None and ctx.needs_input_grad[3]
        dQ, dK, dV, dM_in = bwd_bidir(Q, K, V, _grad_tokens(dO, Q), ctx.chunk, cu_seqlens, M_in,
                                      _grad_state(dM_out), cache, want_dm_in=want_dm_in)
        return dQ, dK, dV, dM_in, None, None


def _contig(*ts):
    return [None if t is None else t.contiguous() for t in ts]


def lasp_attention(Q, K, V, chunk, decay=None, cu_seqlens=None, M_in=None, *, norm=False):
    """Chunked causal linear attention with autograd ("Linear Attention Sequence
    Parallelism", Sec. 3.2, Eqs. 7-11 forward, Eqs. 14-23 backward):
    O = [(Q K^T) . D] V + Lambda Q M_in per sequence and head.  norm=True
    normalises each output row (Eq. 2's Norm read as an RMS normalisation over
    d, eps 1e-6, no gain).  Q, K, V: [B, H, N, d] bf16 or float32 on a GPU;
    decay: float32 [H] or None (no gradient); cu_seqlens: int32 [nseq + 1] or
    None; M_in: float32 [S, H, d, d] or None.  Returns (O, M_out)."""
    Q, K, V, M_in = _contig(Q, K, V, M_in)
    O, M_out = _Causal.apply(Q, K, V, M_in, decay, cu_seqlens, chunk, bool(norm))
    return O, M_out


def lasp_gated_attention(Q, K, V, log_g, chunk=64, cu_seqlens=None, M_in=None):
    """Gated form with autograd (LASP Appendix A.4, Eq. 24, per-key-channel
    gates): kv_p = Diag(g_p) kv_{p-1} + k_p^T v_p, o_p = q_p kv_p, with
    log_g = log g float32 [B, H, N, d].  Returns (O, M_out)."""
    Q, K, V, log_g, M_in = _contig(Q, K, V, log_g, M_in)
    return _Gated.apply(Q, K, V, log_g, M_in, cu_seqlens, chunk)


def lasp_bidir_attention(Q, K, V, chunk=256, cu_seqlens=None, M_in=None):
    """Unmasked form with autograd (LASP Sec. 3.1, Eq. 3, without Norm):
    O = Q (M_in + K^T V) per sequence and head.  Returns (O, M_out)."""
    Q, K, V, M_in = _contig(Q, K, V, M_in)
    return _Bidir.apply(Q, K, V, M_in, cu_seqlens, chunk)
