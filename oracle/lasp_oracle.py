"""Float64 CPU oracle: what chunked causal linear attention computes.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain, slow, obviously
correct numpy.  No blocking, fusion or reordering beyond what the cited
definitions state.

Conventions (one sequence of one head):
  q, k, v, do : float64 [L, d], row p is token p (0-based)
  lam         : the decay lambda of [LASP] Sec. 3.2 (lambda = 1: no decay)
  m_in        : float64 [d, d] incoming state (row = key feature, col = value
                feature), or None for zero.  It is the state before token 0, so
                token p sees lam**(p+1) * m_in (reading of [LASP] Alg. 2, where
                the state KV_{t-1} received from the previous rank plays this role).
  m_out       : the state after the last token ([LASP] Eq. 6 at s = L).
  loss for gradients: l = <dO, O> + <dM_out, M_out>, so dM_out seeds the
                reverse recursion and dM_in is the gradient of l w.r.t. M_in.

Normalisation Norm(.) of [LASP] Eq. 2 is omitted, as in every derivation of
[LASP] Sec. 3.2; no feature map and no 1/sqrt(d) scale are applied.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "quadratic_fwd", "quadratic_bwd",
    "recurrent_fwd", "recurrent_bwd",
    "chunked_fwd", "chunked_bwd",
    "sampled_o", "sampled_dq", "sampled_dk", "sampled_dv",
    "closed_m_out", "closed_dm_in",
    "batched_fwd", "batched_bwd",
    "bidir_fwd", "bidir_bwd", "batched_bidir_fwd", "batched_bidir_bwd", "bidir_sampled",
]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _zeros_state(d, m):
    return np.zeros((d, d)) if m is None else _f64(m)


def _decay_mask(L, lam):
    """D[p, i] = lam**(p - i) for i <= p, else 0: the mask M of [LASP] Alg. 2
    (initialisation of M), diagonal included (Eq. 4 sums over i <= s)."""
    p = np.arange(L)[:, None]
    i = np.arange(L)[None, :]
    diff = (p - i).astype(np.float64)
    return np.where(p >= i, np.power(float(lam), np.maximum(diff, 0.0)), 0.0)


# ---------------------------------------------------------------------------
# 1. The quadratic masked definition ([LASP] Eq. 4; Eq. 2 without Norm)
# ---------------------------------------------------------------------------
def quadratic_fwd(q, k, v, lam=1.0, m_in=None):
    """o_p = sum_{i<=p} lam^(p-i) (q_p . k_i) v_i + lam^(p+1) q_p M_in   [LASP Eq. 4]
    M_out = lam^L M_in + sum_i lam^(L-1-i) k_i^T v_i                     [LASP Eq. 6]
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, d = q.shape
    m = _zeros_state(d, m_in)
    D = _decay_mask(L, lam)
    lam_row = np.power(float(lam), np.arange(1, L + 1, dtype=np.float64))   # lam^(p+1)
    o = ((q @ k.T) * D) @ v + lam_row[:, None] * (q @ m)
    g = np.power(float(lam), np.arange(L - 1, -1, -1, dtype=np.float64))    # lam^(L-1-i)
    m_out = float(lam) ** L * m + k.T @ (g[:, None] * v)
    return o, m_out


def quadratic_bwd(q, k, v, do, lam=1.0, m_in=None, dm_out=None):
    """Gradients of l = <dO, O> + <dM_out, M_out> through quadratic_fwd.

    Written out from the definition (the token-level forms of [LASP] Eq. 12,
    with the state carried in and out):
      dq_p  = sum_{j<=p} lam^(p-j) (do_p . v_j) k_j + lam^(p+1) do_p M_in^T
      dk_j  = sum_{p>=j} lam^(p-j) (do_p . v_j) q_p + lam^(L-1-j) v_j dM_out^T
      dv_j  = sum_{p>=j} lam^(p-j) (q_p . k_j) do_p + lam^(L-1-j) k_j dM_out
      dM_in = sum_p lam^(p+1) q_p^T do_p + lam^L dM_out
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    L, d = q.shape
    m = _zeros_state(d, m_in)
    dm = _zeros_state(d, dm_out)
    D = _decay_mask(L, lam)
    lam_row = np.power(float(lam), np.arange(1, L + 1, dtype=np.float64))
    g = np.power(float(lam), np.arange(L - 1, -1, -1, dtype=np.float64))
    A = (q @ k.T) * D          # A[p, j]
    E = (do @ v.T) * D         # E[p, j]
    dq = E @ k + lam_row[:, None] * (do @ m.T)
    dk = E.T @ q + g[:, None] * (v @ dm.T)
    dv = A.T @ do + g[:, None] * (k @ dm)
    dm_in = (lam_row[:, None] * q).T @ do + float(lam) ** L * dm
    return dq, dk, dv, dm_in


# ---------------------------------------------------------------------------
# 2. The token recurrence ([LASP] Eq. 5 forward, Eqs. 12-13 backward)
# ---------------------------------------------------------------------------
def recurrent_fwd(q, k, v, lam=1.0, m_in=None):
    """kv_p = lam kv_{p-1} + k_p^T v_p, kv_{-1} = M_in;  o_p = q_p kv_p   [LASP Eq. 5]"""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, d = q.shape
    kv = _zeros_state(d, m_in).copy()
    o = np.zeros((L, v.shape[1]))
    for p in range(L):
        kv = lam * kv + np.outer(k[p], v[p])
        o[p] = q[p] @ kv
    return o, kv


def recurrent_bwd(q, k, v, do, lam=1.0, m_in=None, dm_out=None):
    """[LASP] Eq. 12: dq_p = do_p kv_p^T, dk_p = v_p dkv_p^T, dv_p = k_p dkv_p, with
    dkv_p = sum_{i>=p} lam^(i-p) q_i^T do_i (plus the carried dM_out term), built
    by the reverse recursion of Eq. 13.  dM_in is lam * dkv_0."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    L, d = q.shape
    kv = _zeros_state(d, m_in).copy()
    dq = np.zeros_like(q)
    for p in range(L):                       # forward sweep recomputes kv_p
        kv = lam * kv + np.outer(k[p], v[p])
        dq[p] = do[p] @ kv.T
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    g = _zeros_state(d, dm_out).copy()       # reverse sweep, Eq. 13
    for p in range(L - 1, -1, -1):
        g = g + np.outer(q[p], do[p])        # g = dkv_p
        dk[p] = v[p] @ g.T
        dv[p] = k[p] @ g
        g = lam * g
    return dq, dk, dv, g


# ---------------------------------------------------------------------------
# 3. The chunked intra/inter form ([LASP] Eqs. 7-11 and 14-23)
#    Used only to show that the chunk decomposition equals the definition.
# ---------------------------------------------------------------------------
def _chunk_bounds(L, C):
    return [(s, min(s + C, L)) for s in range(0, L, C)]


def chunked_fwd(q, k, v, C, lam=1.0, m_in=None, return_states=False):
    """Per chunk t (length C_t, the last one may be shorter):
        O_t,intra = [(Q_t K_t^T) . M] V_t                 [LASP Eq. 7]
        O_t,inter = Lambda Q_t KV_{t-1}                   [LASP Eq. 9]
        O_t = O_t,intra + O_t,inter                       [LASP Eq. 11]
        KV_t = lam^C KV_{t-1} + (lam^C Lambda^-1 K_t)^T V_t   [LASP Eq. 10]
    with Lambda = diag(lam, ..., lam^C_t) and lam^C Lambda^-1 written as
    diag(lam^(C_t-1), ..., 1) (the middle line of Eq. 10)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    L, d = q.shape
    kv = _zeros_state(d, m_in).copy()
    o = np.zeros((L, v.shape[1]))
    states = []
    for s, e in _chunk_bounds(L, C):
        Ct = e - s
        M = _decay_mask(Ct, lam)
        Lam = np.power(float(lam), np.arange(1, Ct + 1, dtype=np.float64))
        Gam = np.power(float(lam), np.arange(Ct - 1, -1, -1, dtype=np.float64))
        Qt, Kt, Vt = q[s:e], k[s:e], v[s:e]
        states.append(kv.copy())                     # the cached KV_{t-1}
        o[s:e] = ((Qt @ Kt.T) * M) @ Vt + Lam[:, None] * (Qt @ kv)
        kv = float(lam) ** Ct * kv + (Gam[:, None] * Kt).T @ Vt
    if return_states:
        return o, kv, states
    return o, kv


def chunked_bwd(q, k, v, do, C, lam=1.0, m_in=None, dm_out=None):
    """Per chunk, in reverse chunk order, with dKV the state received from the
    following chunk ([LASP] Eqs. 14-23; the dKV update of Eq. 20 is applied in
    the form of its last line):
        dQ_t = [(dO_t V_t^T) . M] K_t + Lambda dO_t KV_{t-1}^T       [Eqs. 14, 16]
        dK_t = [(dO_t V_t^T) . M]^T Q_t + lam^C Lambda^-1 V_t dKV^T  [Eqs. 17, 19]
        dV_t = [(Q_t K_t^T) . M]^T dO_t + lam^C Lambda^-1 K_t dKV    [Eqs. 21, 22]
        dKV <- lam^C dKV + (Lambda Q_t)^T dO_t                       [Eq. 20]
    The dKV entering the last chunk is dM_out; the one leaving chunk 0 is dM_in."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    L, d = q.shape
    _, _, states = chunked_fwd(q, k, v, C, lam, m_in, return_states=True)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dkv = _zeros_state(d, dm_out).copy()
    bounds = _chunk_bounds(L, C)
    for t in range(len(bounds) - 1, -1, -1):
        s, e = bounds[t]
        Ct = e - s
        M = _decay_mask(Ct, lam)
        Lam = np.power(float(lam), np.arange(1, Ct + 1, dtype=np.float64))
        Gam = np.power(float(lam), np.arange(Ct - 1, -1, -1, dtype=np.float64))
        Qt, Kt, Vt, dOt = q[s:e], k[s:e], v[s:e], do[s:e]
        E = (dOt @ Vt.T) * M
        A = (Qt @ Kt.T) * M
        dq[s:e] = E @ Kt + Lam[:, None] * (dOt @ states[t].T)
        dk[s:e] = E.T @ Qt + Gam[:, None] * (Vt @ dkv.T)
        dv[s:e] = A.T @ dOt + Gam[:, None] * (Kt @ dkv)
        dkv = float(lam) ** Ct * dkv + (Lam[:, None] * Qt).T @ dOt
    return dq, dk, dv, dkv


# ---------------------------------------------------------------------------
# 4. Row-sampled direct sums of the definition (any length)
# ---------------------------------------------------------------------------
def _pow(lam, e):
    return np.power(float(lam), np.asarray(e, dtype=np.float64))


def _row_weights(a, b, rows, lam, forward=True):
    """W[n, i] = lam^(p_n - i) (a_{p_n} . b_i) for i <= p_n (forward), or
    W[n, i] = lam^(i - p_n) (a_i . b_{p_n}) for i >= p_n (backward), zero elsewhere:
    the rows p_n of the masked score matrix of [LASP] Eq. 7 with C = L."""
    rows = np.asarray(rows)
    L = a.shape[0]
    i = np.arange(L)[None, :]
    p = rows[:, None]
    if forward:
        e = (p - i).astype(np.float64)
        S = a[rows] @ b.T
        keep = i <= p
    else:
        e = (i - p).astype(np.float64)
        S = (a @ b[rows].T).T
        keep = i >= p
    return np.where(keep, S * np.power(float(lam), np.where(keep, e, 0.0)), 0.0)


def sampled_o(q, k, v, rows, lam=1.0, m_in=None):
    """o_p for p in rows: sum_{i<=p} lam^(p-i) (q_p . k_i) v_i + lam^(p+1) q_p M_in."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.asarray(rows)
    m = _zeros_state(q.shape[1], m_in)
    return _row_weights(q, k, rows, lam) @ v + _pow(lam, rows + 1)[:, None] * (q[rows] @ m)


def sampled_dq(q, k, v, do, rows, lam=1.0, m_in=None):
    """dq_p = sum_{j<=p} lam^(p-j) (do_p . v_j) k_j + lam^(p+1) do_p M_in^T."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows)
    m = _zeros_state(q.shape[1], m_in)
    return _row_weights(do, v, rows, lam) @ k + _pow(lam, rows + 1)[:, None] * (do[rows] @ m.T)


def sampled_dk(q, k, v, do, rows, lam=1.0, dm_out=None):
    """dk_j = sum_{p>=j} lam^(p-j) (do_p . v_j) q_p + lam^(L-1-j) v_j dM_out^T."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows)
    L, d = q.shape
    dm = _zeros_state(d, dm_out)
    return (_row_weights(do, v, rows, lam, forward=False) @ q
            + _pow(lam, L - 1 - rows)[:, None] * (v[rows] @ dm.T))


def sampled_dv(q, k, v, do, rows, lam=1.0, dm_out=None):
    """dv_j = sum_{p>=j} lam^(p-j) (q_p . k_j) do_p + lam^(L-1-j) k_j dM_out."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows)
    L, d = q.shape
    dm = _zeros_state(d, dm_out)
    return (_row_weights(q, k, rows, lam, forward=False) @ do
            + _pow(lam, L - 1 - rows)[:, None] * (k[rows] @ dm))


def closed_m_out(k, v, lam=1.0, m_in=None):
    """M_out = lam^L M_in + K^T diag(lam^(L-1-i)) V  ([LASP] Eq. 6 at s = L;
    with lam = 1 and no M_in this is the K^T V of Eq. 3, the LASP-2 state)."""
    k, v = _f64(k), _f64(v)
    L, d = k.shape
    m = _zeros_state(d, m_in)
    g = _pow(lam, np.arange(L - 1, -1, -1))
    return float(lam) ** L * m + k.T @ (g[:, None] * v)


def closed_dm_in(q, do, lam=1.0, dm_out=None):
    """dM_in = sum_p lam^(p+1) q_p^T do_p + lam^L dM_out."""
    q, do = _f64(q), _f64(do)
    L, d = q.shape
    dm = _zeros_state(d, dm_out)
    lr = _pow(lam, np.arange(1, L + 1))
    return (lr[:, None] * q).T @ do + float(lam) ** L * dm


# ---------------------------------------------------------------------------
# 5. Batched drivers over the [B, H, N, d] layout and packed varlen batches
# ---------------------------------------------------------------------------
def _segments(B, N, cu_seqlens):
    """(batch index, start, end) of every sequence: B sequences of length N, or,
    with cu_seqlens, the packed sequences [cu[i], cu[i+1]) of batch row 0."""
    if cu_seqlens is None:
        return [(b, 0, N) for b in range(B)]
    cu = [int(x) for x in cu_seqlens]
    return [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def batched_fwd(Q, K, V, decay=None, m_in=None, cu_seqlens=None, form="quadratic", chunk=None):
    """Q, K, V: [B, H, N, d].  decay: [H] or None.  m_in: [S, H, d, d] or None,
    S = B (or the number of packed sequences).  Returns (O [B,H,N,d], M_out [S,H,d,d])."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    segs = _segments(B, N, cu_seqlens)
    O = np.zeros(Q.shape[:3] + (V.shape[3],))
    Mout = np.zeros((len(segs), H, d, V.shape[3]))
    for si, (b, s, e) in enumerate(segs):
        for h in range(H):
            lam = 1.0 if decay is None else float(decay[h])
            mi = None if m_in is None else m_in[si, h]
            args = (Q[b, h, s:e], K[b, h, s:e], V[b, h, s:e])
            if form == "quadratic":
                o, mo = quadratic_fwd(*args, lam=lam, m_in=mi)
            elif form == "recurrent":
                o, mo = recurrent_fwd(*args, lam=lam, m_in=mi)
            elif form == "chunked":
                o, mo = chunked_fwd(*args, chunk, lam=lam, m_in=mi)
            else:
                raise ValueError(form)
            O[b, h, s:e] = o
            Mout[si, h] = mo
    return O, Mout


def batched_bwd(Q, K, V, dO, decay=None, m_in=None, dm_out=None, cu_seqlens=None,
                form="quadratic", chunk=None):
    """Returns (dQ, dK, dV [B,H,N,d], dM_in [S,H,d,d])."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, N, d = Q.shape
    segs = _segments(B, N, cu_seqlens)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dMin = np.zeros((len(segs), H, d, V.shape[3]))
    for si, (b, s, e) in enumerate(segs):
        for h in range(H):
            lam = 1.0 if decay is None else float(decay[h])
            mi = None if m_in is None else m_in[si, h]
            dmo = None if dm_out is None else dm_out[si, h]
            args = (Q[b, h, s:e], K[b, h, s:e], V[b, h, s:e], dO[b, h, s:e])
            if form == "quadratic":
                r = quadratic_bwd(*args, lam=lam, m_in=mi, dm_out=dmo)
            elif form == "recurrent":
                r = recurrent_bwd(*args, lam=lam, m_in=mi, dm_out=dmo)
            elif form == "chunked":
                r = chunked_bwd(*args, chunk, lam=lam, m_in=mi, dm_out=dmo)
            else:
                raise ValueError(form)
            dQ[b, h, s:e], dK[b, h, s:e], dV[b, h, s:e], dMin[si, h] = r
    return dQ, dK, dV, dMin


# ---------------------------------------------------------------------------
# 6. The unmasked (bidirectional) form: [LASP] Eq. 3 without Norm, i.e. every
#    token attends to every token of its sequence; with sequence parallelism
#    each rank sums all chunk states (LASP-2's M_(1:T), one AllGather and a
#    sum).  M_in stands for the states of the other ranks' chunks; there is
#    no decay in this form.
# ---------------------------------------------------------------------------
def bidir_fwd(q, k, v, m_in=None):
    """o_p = sum_i (q_p . k_i) v_i + q_p M_in   over all tokens i    [LASP Eq. 3, left product]
    M_out = M_in + sum_i k_i^T v_i                                    (the summed state)
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    m = _zeros_state(q.shape[1], m_in)
    o = (q @ k.T) @ v + q @ m
    return o, m + k.T @ v


def bidir_bwd(q, k, v, do, m_in=None, dm_out=None):
    """Gradients of l = <dO, O> + <dM_out, M_out> through bidir_fwd, written
    out from the definition:
      dq_p  = sum_j (do_p . v_j) k_j + do_p M_in^T
      dk_j  = sum_p (do_p . v_j) q_p + v_j dM_out^T
      dv_j  = sum_p (q_p . k_j) do_p + k_j dM_out
      dM_in = sum_p q_p^T do_p + dM_out
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    d = q.shape[1]
    m = _zeros_state(d, m_in)
    dm = _zeros_state(d, dm_out)
    A = q @ k.T                # A[p, j] = q_p . k_j
    E = do @ v.T               # E[p, j] = do_p . v_j
    dq = E @ k + do @ m.T
    dk = E.T @ q + v @ dm.T
    dv = A.T @ do + k @ dm
    dm_in = q.T @ do + dm
    return dq, dk, dv, dm_in


def batched_bidir_fwd(Q, K, V, m_in=None, cu_seqlens=None):
    """[B, H, N, d] (or packed) driver of bidir_fwd.  Returns (O, M_out [S,H,d,d])."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    B, H, N, d = Q.shape
    segs = _segments(B, N, cu_seqlens)
    O = np.zeros(Q.shape[:3] + (V.shape[3],))
    Mout = np.zeros((len(segs), H, d, V.shape[3]))
    for si, (b, s, e) in enumerate(segs):
        for h in range(H):
            mi = None if m_in is None else m_in[si, h]
            O[b, h, s:e], Mout[si, h] = bidir_fwd(Q[b, h, s:e], K[b, h, s:e], V[b, h, s:e], mi)
    return O, Mout


def batched_bidir_bwd(Q, K, V, dO, m_in=None, dm_out=None, cu_seqlens=None):
    """Returns (dQ, dK, dV [B,H,N,d], dM_in [S,H,d,d])."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    B, H, N, d = Q.shape
    segs = _segments(B, N, cu_seqlens)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    dMin = np.zeros((len(segs), H, d, V.shape[3]))
    for si, (b, s, e) in enumerate(segs):
        for h in range(H):
            mi = None if m_in is None else m_in[si, h]
            dmo = None if dm_out is None else dm_out[si, h]
            dQ[b, h, s:e], dK[b, h, s:e], dV[b, h, s:e], dMin[si, h] = bidir_bwd(
                Q[b, h, s:e], K[b, h, s:e], V[b, h, s:e], dO[b, h, s:e], mi, dmo)
    return dQ, dK, dV, dMin


def bidir_sampled(q, k, v, do, rows, m_in=None, dm_out=None):
    """Rows `rows` of O, dQ, dK, dV of the unmasked form, each a direct sum over
    all tokens (left products restricted to the sampled rows), and the full
    M_out and dM_in.  For sequences too long for the L x L products."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    d = q.shape[1]
    m = _zeros_state(d, m_in)
    dm = _zeros_state(d, dm_out)
    r = np.asarray(rows)
    return {
        "O": (q[r] @ k.T) @ v + q[r] @ m,
        "dQ": (do[r] @ v.T) @ k + do[r] @ m.T,
        "dK": (v[r] @ do.T) @ q + v[r] @ dm.T,
        "dV": (k[r] @ q.T) @ do + k[r] @ dm,
        "M_out": m + k.T @ v,
        "dM_in": q.T @ do + dm,
    }
