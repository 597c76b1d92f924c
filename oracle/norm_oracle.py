"""Float64 CPU oracle of the output normalisation Norm(.) of [LASP] Eq. 2.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[LASP] Sec. 3.1, Eq. 2 writes causal linear attention as
O = Norm((Q K^T . M) V), Norm being "a normalization operation" taken from
the TransNormer line of work; the pages define it no further, and every
derivation of [LASP] Sec. 3.2 leaves it out.  READING taken here: Norm acts on
each output row (one token of one head) over its d features as a root-mean-
square normalisation without a learned gain,

    Norm(o) = o * r,   r = 1 / sqrt(mean_j o_j^2 + eps),   eps = 1e-6,

applied to the causal output of lasp_oracle (decay, M_in, packed batches
included); the carried state M_out is not normalised.  The backward of
l = <dY, Y> + <dM_out, M_out> passes through Norm row by row:

    dO = r * (dY - Y * mean_j(dY_j Y_j))

and then through the causal map as in lasp_oracle (dO in place of the output
gradient).
"""
from __future__ import annotations

import numpy as np

from . import lasp_oracle as lo

__all__ = ["NORM_EPS", "norm_fwd", "norm_bwd", "batched_norm_fwd", "batched_norm_bwd"]

NORM_EPS = 1e-6


def norm_fwd(o, eps=NORM_EPS):
    """Y = o * r per row (last axis), r = 1/sqrt(mean(o^2) + eps).  Returns (Y, r)."""
    o = np.asarray(o, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1) + eps)
    return o * r[..., None], r


def norm_bwd(y, r, dy):
    """dO for the row map Y = Norm(O), from its output Y, its r and dY:
    dO_j = r (dY_j - Y_j mean_k(dY_k Y_k))."""
    y, r, dy = (np.asarray(x, dtype=np.float64) for x in (y, r, dy))
    m = np.mean(dy * y, axis=-1, keepdims=True)
    return r[..., None] * (dy - y * m)


def batched_norm_fwd(Q, K, V, decay=None, m_in=None, cu_seqlens=None, eps=NORM_EPS):
    """Y = Norm(O), rstd = r per row ([B, H, N]) and M_out for the causal map
    of lasp_oracle.batched_fwd."""
    O, M_out = lo.batched_fwd(Q, K, V, decay, m_in, cu_seqlens)
    Y, r = norm_fwd(O, eps)
    return Y, r, M_out


def batched_norm_bwd(Q, K, V, dY, decay=None, m_in=None, dm_out=None, cu_seqlens=None,
                     eps=NORM_EPS):
    """dQ, dK, dV, dM_in of l = <dY, Norm(O)> + <dM_out, M_out>."""
    O, _ = lo.batched_fwd(Q, K, V, decay, m_in, cu_seqlens)
    Y, r = norm_fwd(O, eps)
    dO = norm_bwd(Y, r, dY)
    return lo.batched_bwd(Q, K, V, dO, decay, m_in, dm_out, cu_seqlens)
