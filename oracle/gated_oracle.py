"""Float64 CPU oracle of the gated (data-dependent, per-channel decay) form.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy; no blocking,
chunking or reordering.

Source: [LASP] Appendix A.4 ("Generalization of LASP"), the general memory
recurrence m_t = o_t m_{t-1} + e_t i_t^T (Eq. 24) and its GLA / GateLoop row
of Table 5: the oscillation state is g_t 1^T, i.e.

    kv_t = Diag(g_t) kv_{t-1} + k_t^T v_t,        y_t = q_t kv_t

with a gate g_t in R^{d_k} per token that scales the key rows of the d_k x d_v
state.  With g_t = lambda for every channel and token this is the decayed
recurrence of [LASP] Eq. 5 (Eq. 25 of the appendix).

Conventions (one sequence of one head), as in lasp_oracle:
  q, k, v, do : float64 [L, d];  log_g : float64 [L, d], log of the gate
                (g = exp(log_g); the gates are passed as logs, which keeps the
                products of many gates representable)
  m_in        : state before token 0 ([d, d], row = key feature) or None
  loss        : l = <dO, O> + <dM_out, M_out>; gradients are returned for
                q, k, v, log_g and m_in.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "gated_recurrent_fwd", "gated_recurrent_bwd", "gated_unrolled_fwd",
    "batched_gated_fwd", "batched_gated_bwd", "gated_sampled", "gated_closed_states",
    "gated_sampled_sweep",
]


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _state(d, m):
    return np.zeros((d, d)) if m is None else _f64(m).copy()


# ---------------------------------------------------------------------------
# 1. The recurrence itself ([LASP] Eq. 24 with the GLA row of Table 5)
# ---------------------------------------------------------------------------
def gated_recurrent_fwd(q, k, v, log_g, m_in=None):
    """kv_p = Diag(g_p) kv_{p-1} + k_p^T v_p (kv_{-1} = M_in);  o_p = q_p kv_p.
    Returns (O [L, d], M_out = kv_{L-1})."""
    q, k, v, lg = _f64(q), _f64(k), _f64(v), _f64(log_g)
    L, d = q.shape
    kv = _state(d, m_in)
    o = np.zeros((L, v.shape[1]))
    for p in range(L):
        kv = np.exp(lg[p])[:, None] * kv + np.outer(k[p], v[p])
        o[p] = q[p] @ kv
    return o, kv


def gated_recurrent_bwd(q, k, v, log_g, do, m_in=None, dm_out=None):
    """Reverse-mode derivative of gated_recurrent_fwd, written out from the
    recurrence.  With G_p the gradient of l w.r.t. kv_p:
        G_{L-1} = q_{L-1}^T do_{L-1} + dM_out
        G_p     = q_p^T do_p + Diag(g_{p+1}) G_{p+1}
        dq_p = do_p kv_p^T,   dk_p = v_p G_p^T,   dv_p = k_p G_p
        dlog_g_p[c] = g_p[c] * sum_e G_p[c, e] kv_{p-1}[c, e]
        dM_in = Diag(g_0) G_0
    Returns (dq, dk, dv, dlog_g, dM_in)."""
    q, k, v, lg, do = _f64(q), _f64(k), _f64(v), _f64(log_g), _f64(do)
    L, d = q.shape
    kv = _state(d, m_in)
    states = [kv.copy()]                 # states[p] = kv_{p-1}
    dq = np.zeros_like(q)
    for p in range(L):
        kv = np.exp(lg[p])[:, None] * kv + np.outer(k[p], v[p])
        states.append(kv.copy())
        dq[p] = do[p] @ kv.T
    dk, dv, dlg = np.zeros_like(k), np.zeros_like(v), np.zeros_like(lg)
    carry = _state(d, dm_out)           # Diag(g_{p+1}) G_{p+1}, or dM_out
    for p in range(L - 1, -1, -1):
        G = np.outer(q[p], do[p]) + carry
        dk[p] = v[p] @ G.T
        dv[p] = k[p] @ G
        gp = np.exp(lg[p])
        dlg[p] = gp * np.sum(G * states[p], axis=1)
        carry = gp[:, None] * G
    return dq, dk, dv, dlg, carry


# ---------------------------------------------------------------------------
# 2. The recurrence unrolled: its closed-form solution, with the cumulative
#    log-gate B_p = sum_{j<=p} log g_j
#        o_p = sum_{i<=p} (q_p . (k_i * exp(B_p - B_i))) v_i + (q_p * exp(B_p)) M_in
#        M_out = sum_i (k_i * exp(B_{L-1} - B_i))^T v_i + Diag(exp(B_{L-1})) M_in
#    A second, independent statement of the same map (used to pin section 1).
# ---------------------------------------------------------------------------
def gated_unrolled_fwd(q, k, v, log_g, m_in=None):
    q, k, v, lg = _f64(q), _f64(k), _f64(v), _f64(log_g)
    L, d = q.shape
    m = _state(d, m_in)
    B = np.cumsum(lg, axis=0)
    o = np.zeros((L, v.shape[1]))
    for p in range(L):
        w = np.exp(B[p][None, :] - B[: p + 1])            # [i, c] for i <= p
        scores = (k[: p + 1] * w) @ q[p]                   # q_p . (k_i * w_i)
        o[p] = scores @ v[: p + 1] + (q[p] * np.exp(B[p])) @ m
    wl = np.exp(B[L - 1][None, :] - B)
    m_out = (k * wl).T @ v + np.exp(B[L - 1])[:, None] * m
    return o, m_out


# ---------------------------------------------------------------------------
# 3. Batched drivers over [B, H, N, d] and packed batches
# ---------------------------------------------------------------------------
def _segments(B, N, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, N) for b in range(B)]
    cu = [int(x) for x in cu_seqlens]
    return [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]


def batched_gated_fwd(Q, K, V, LG, m_in=None, cu_seqlens=None):
    """Q, K, V, LG: [B, H, N, d].  m_in: [S, H, d, d] or None.
    Returns (O [B,H,N,d], M_out [S,H,d,d])."""
    Q, K, V, LG = _f64(Q), _f64(K), _f64(V), _f64(LG)
    B, H, N, d = Q.shape
    segs = _segments(B, N, cu_seqlens)
    O = np.zeros(Q.shape)
    Mout = np.zeros((len(segs), H, d, d))
    for si, (b, s, e) in enumerate(segs):
        for h in range(H):
            mi = None if m_in is None else m_in[si, h]
            O[b, h, s:e], Mout[si, h] = gated_recurrent_fwd(
                Q[b, h, s:e], K[b, h, s:e], V[b, h, s:e], LG[b, h, s:e], mi)
    return O, Mout


def batched_gated_bwd(Q, K, V, LG, dO, m_in=None, dm_out=None, cu_seqlens=None):
    """Returns (dQ, dK, dV, dLG [B,H,N,d], dM_in [S,H,d,d])."""
    Q, K, V, LG, dO = _f64(Q), _f64(K), _f64(V), _f64(LG), _f64(dO)
    B, H, N, d = Q.shape
    segs = _segments(B, N, cu_seqlens)
    dQ, dK, dV, dLG = (np.zeros(Q.shape) for _ in range(4))
    dMin = np.zeros((len(segs), H, d, d))
    for si, (b, s, e) in enumerate(segs):
        for h in range(H):
            mi = None if m_in is None else m_in[si, h]
            dmo = None if dm_out is None else dm_out[si, h]
            r = gated_recurrent_bwd(Q[b, h, s:e], K[b, h, s:e], V[b, h, s:e], LG[b, h, s:e],
                                    dO[b, h, s:e], mi, dmo)
            dQ[b, h, s:e], dK[b, h, s:e], dV[b, h, s:e], dLG[b, h, s:e], dMin[si, h] = r
    return dQ, dK, dV, dLG, dMin


# ---------------------------------------------------------------------------
# 4. Single rows of a long sequence, from the prefix state kv_p and the
#    suffix gradient state G_p of section 1 written as sums:
#        kv_p = sum_{i<=p} Diag(exp(B_p - B_i)) k_i^T v_i + Diag(exp(B_p)) M_in
#        G_p  = sum_{u>=p} Diag(exp(B_u - B_p)) q_u^T do_u
#               + Diag(exp(B_{L-1} - B_p)) dM_out
#    then o_p = q_p kv_p, dq_p = do_p kv_p^T, dk_p = v_p G_p^T, dv_p = k_p G_p and
#    dlog_g_p = g_p * rowsum(G_p . kv_{p-1}), kv_{p-1} = the first sum without
#    token p, scaled back by the gate of token p.
# ---------------------------------------------------------------------------
def gated_sampled(q, k, v, log_g, do, rows, m_in=None, dm_out=None):
    """Rows `rows` of O, dQ, dK, dV and dlog_g.  O(L d^2) work per row."""
    q, k, v, lg, do = _f64(q), _f64(k), _f64(v), _f64(log_g), _f64(do)
    L, d = q.shape
    m = _state(d, m_in)
    dm = _state(d, dm_out)
    B = np.cumsum(lg, axis=0)
    out = {n: np.zeros((len(rows), d)) for n in ("O", "dQ", "dK", "dV", "dLG")}
    for n, p in enumerate(int(r) for r in rows):
        # kv_{p-1}: tokens i < p, seen from just before token p
        Bprev = B[p - 1] if p > 0 else np.zeros(d)
        kv_prev = (k[:p] * np.exp(Bprev[None, :] - B[:p])).T @ v[:p] + np.exp(Bprev)[:, None] * m
        kv_p = np.exp(lg[p])[:, None] * kv_prev + np.outer(k[p], v[p])
        G = ((q[p:] * np.exp(B[p:] - B[p][None, :])).T @ do[p:]
             + np.exp(B[L - 1] - B[p])[:, None] * dm)
        out["O"][n] = q[p] @ kv_p
        out["dQ"][n] = do[p] @ kv_p.T
        out["dK"][n] = v[p] @ G.T
        out["dV"][n] = k[p] @ G
        out["dLG"][n] = np.exp(lg[p]) * np.sum(G * kv_prev, axis=1)
    return out


def gated_closed_states(q, k, v, log_g, do, m_in=None, dm_out=None):
    """M_out and dM_in of a long sequence in closed form (section 4 at the ends):
        M_out = sum_i Diag(exp(B_{L-1} - B_i)) k_i^T v_i + Diag(exp(B_{L-1})) M_in
        dM_in = sum_u Diag(exp(B_u)) q_u^T do_u + Diag(exp(B_{L-1})) dM_out"""
    q, k, v, lg, do = _f64(q), _f64(k), _f64(v), _f64(log_g), _f64(do)
    L, d = q.shape
    m = _state(d, m_in)
    dm = _state(d, dm_out)
    if L == 0:
        return m, dm
    B = np.cumsum(lg, axis=0)
    m_out = (k * np.exp(B[L - 1][None, :] - B)).T @ v + np.exp(B[L - 1])[:, None] * m
    dm_in = (q * np.exp(B)).T @ do + np.exp(B[L - 1])[:, None] * dm
    return m_out, dm_in


def gated_sampled_sweep(q, k, v, log_g, do, rows, m_in=None, dm_out=None):
    """The rows of gated_sampled and the states of gated_closed_states at once,
    the same sums regrouped over the sorted rows: one pass forwards carries
    kv_{p-1} from one row to the next, one pass backwards carries G_p (the
    gradient of l w.r.t. kv_p), O(L d^2) in all instead of per row:

        kv_{p-1} = Diag(exp(B_{p-1} - B_{a-1})) kv_{a-1}
                   + sum_{a <= i < p} Diag(exp(B_{p-1} - B_i)) k_i^T v_i      (a < p)
        G_p      = Diag(exp(B_b - B_p)) G_b
                   + sum_{p <= u < b} Diag(exp(B_u - B_p)) q_u^T do_u          (p < b)

    with B the running sum of the log-gates, B_{-1} = 0, and G_L = dM_out,
    B_L = B_{L-1}; kv_{L-1} is M_out and G_{-1} is dM_in.  Every exponent is
    <= 0 for log-gates <= 0.  Returns (rows dict as gated_sampled, M_out, dM_in)."""
    q, k, v, lg, do = _f64(q), _f64(k), _f64(v), _f64(log_g), _f64(do)
    L, d = q.shape
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    B = np.cumsum(lg, axis=0)
    zero = np.zeros(d)

    def b_before(p):          # B_{p-1}
        return B[p - 1] if p > 0 else zero

    kv_prev = {}
    cur, a = _state(d, m_in), 0            # cur = kv_{a-1}
    for p in [int(r) for r in rows] + [L]:
        if p > a:
            e = b_before(p)
            cur = (np.exp(e - b_before(a))[:, None] * cur
                   + (k[a:p] * np.exp(e[None, :] - B[a:p])).T @ v[a:p])
            a = p
        kv_prev[p] = cur
    m_out = kv_prev[L]

    def b_at(p):              # B_p, with B_L = B_{L-1} and B_{-1} = 0
        return zero if p < 0 else B[min(p, L - 1)]

    G = {}
    cur, b = _state(d, dm_out), L          # cur = G_b
    for p in [int(r) for r in rows[::-1]] + [-1]:
        e = b_at(p)
        lo = max(p, 0)
        cur = (np.exp(b_at(b) - e)[:, None] * cur
               + (q[lo:b] * np.exp(B[lo:b] - e[None, :])).T @ do[lo:b])
        b = lo if p >= 0 else 0
        G[p] = cur
    dm_in = G[-1]

    out = {n: np.zeros((len(rows), d)) for n in ("O", "dQ", "dK", "dV", "dLG")}
    for n, p in enumerate(int(r) for r in rows):
        kv_p = np.exp(lg[p])[:, None] * kv_prev[p] + np.outer(k[p], v[p])
        out["O"][n] = q[p] @ kv_p
        out["dQ"][n] = do[p] @ kv_p.T
        out["dK"][n] = v[p] @ G[p].T
        out["dV"][n] = k[p] @ G[p]
        out["dLG"][n] = np.exp(lg[p]) * np.sum(G[p] * kv_prev[p], axis=1)
    return out, m_out, dm_in
