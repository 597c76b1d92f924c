"""Pins for the gated-form oracle (no GPU).

The gated recurrence of "Linear Attention Sequence Parallelism", Appendix A.4
(Eq. 24, GLA / GateLoop row of Table 5), is tied to: a hand-worked example, its
unrolled closed form, the decayed form of Sec. 3.2 (constant gates; the pinned
scalar-decay oracle), per-channel decomposition into scalar-decay problems,
finite differences, machine differentiation of an independent torch recurrence,
exact invariances, and planted mistakes that these checks must catch.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import gated_oracle as go
from oracle import lasp_oracle as lo

GOLD = os.path.join(os.path.dirname(__file__), "golden", "gated_hand.json")


def case(L, d, seed, strong=False, with_m=True):
    r = np.random.default_rng(seed)
    q, k, v, do = (r.standard_normal((L, d)) for _ in range(4))
    lg = -np.abs(r.standard_normal((L, d))) * (2.0 if strong else 0.3)
    m = r.standard_normal((d, d)) if with_m else None
    dm = r.standard_normal((d, d)) if with_m else None
    return q, k, v, lg, do, m, dm


def loss(o, mo, do, dm):
    return float(np.sum(o * do) + (0.0 if dm is None else np.sum(mo * dm)))


# --- hand-worked example ----------------------------------------------------
def test_hand_example():
    for ex in json.load(open(GOLD))["examples"]:
        a = {n: np.array(x, dtype=np.float64) for n, x in ex.items()
             if n not in ("name", "derivation")}
        lg = np.log(a["g"])
        for fwd in (go.gated_recurrent_fwd, go.gated_unrolled_fwd):
            o, mo = fwd(a["q"], a["k"], a["v"], lg, a["m_in"])
            np.testing.assert_allclose(o, a["o"], atol=1e-12)
            np.testing.assert_allclose(mo, a["m_out"], atol=1e-12)
        dq, dk, dv, dlg, dmi = go.gated_recurrent_bwd(a["q"], a["k"], a["v"], lg, a["do"],
                                                      a["m_in"], a["dm_out"])
        for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (dlg, "dlog_g"), (dmi, "dm_in")):
            np.testing.assert_allclose(got, a[key], atol=1e-12, err_msg=key)


# --- the recurrence equals its unrolled closed form -------------------------
@pytest.mark.parametrize("L,d,strong,with_m", [(1, 3, False, True), (9, 4, False, True),
                                                (23, 3, True, True), (16, 5, False, False)])
def test_unrolled_equals_recurrent(L, d, strong, with_m):
    q, k, v, lg, do, m, dm = case(L, d, L + d, strong, with_m)
    o1, m1 = go.gated_recurrent_fwd(q, k, v, lg, m)
    o2, m2 = go.gated_unrolled_fwd(q, k, v, lg, m)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(m1, m2, rtol=1e-10, atol=1e-12)


def test_empty_sequence_passes_the_state_through():
    d = 3
    m = np.arange(9.0).reshape(3, 3)
    o, mo = go.gated_recurrent_fwd(np.zeros((0, d)), np.zeros((0, d)), np.zeros((0, d)),
                                   np.zeros((0, d)), m)
    assert o.shape == (0, d)
    np.testing.assert_array_equal(mo, m)
    r = go.gated_recurrent_bwd(*(np.zeros((0, d)),) * 5, m, 2 * m)
    np.testing.assert_array_equal(r[4], 2 * m)


# --- constant gates: the decayed form of Sec. 3.2 (Eq. 25 of the appendix) ---
@pytest.mark.parametrize("lam", [1.0, 0.9, 0.5])
def test_constant_gate_is_the_decayed_form(lam):
    L, d = 13, 4
    q, k, v, _, do, m, dm = case(L, d, 7)
    lg = np.full((L, d), np.log(lam))
    o1, m1 = go.gated_recurrent_fwd(q, k, v, lg, m)
    o2, m2 = lo.quadratic_fwd(q, k, v, lam, m)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(m1, m2, rtol=1e-11, atol=1e-12)
    g1 = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    g2 = lo.quadratic_bwd(q, k, v, do, lam, m, dm)
    for a, b in zip((g1[0], g1[1], g1[2], g1[4]), g2):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)
    # every log-gate shifted together is log(lambda) shifted: the summed
    # log-gate gradient is lambda * dl/dlambda of the decayed form
    h = 1e-6
    lp = loss(*lo.quadratic_fwd(q, k, v, lam + h, m), do, dm)
    lm = loss(*lo.quadratic_fwd(q, k, v, lam - h, m), do, dm)
    np.testing.assert_allclose(g1[3].sum(), lam * (lp - lm) / (2 * h), rtol=1e-6)


def test_channel_constant_gates_split_into_scalar_problems():
    """Gates constant in time but different per key channel: the map is the sum
    over key channels c of scalar-decay problems with d_k = 1 and lambda_c."""
    L, d = 11, 4
    q, k, v, _, do, m, dm = case(L, d, 8)
    lams = np.array([1.0, 0.8, 0.5, 0.95])
    lg = np.tile(np.log(lams), (L, 1))
    o, mo = go.gated_recurrent_fwd(q, k, v, lg, m)
    osum = np.zeros_like(o)
    for c in range(d):
        oc, mc = lo.quadratic_fwd(q[:, c:c + 1], k[:, c:c + 1], v, lams[c], m[c:c + 1, :])
        osum += oc
        np.testing.assert_allclose(mo[c], mc[0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(o, osum, rtol=1e-11, atol=1e-12)
    dq, dk, dv, dlg, dmi = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    dvsum = np.zeros_like(dv)
    for c in range(d):
        r = lo.quadratic_bwd(q[:, c:c + 1], k[:, c:c + 1], v, do, lams[c], m[c:c + 1, :],
                             dm[c:c + 1, :])
        np.testing.assert_allclose(dq[:, c], r[0][:, 0], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dk[:, c], r[1][:, 0], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dmi[c], r[3][0], rtol=1e-10, atol=1e-11)
        dvsum += r[2]
    np.testing.assert_allclose(dv, dvsum, rtol=1e-10, atol=1e-11)


# --- finite differences ------------------------------------------------------
def test_finite_differences():
    L, d = 6, 3
    q, k, v, lg, do, m, dm = case(L, d, 11)
    dq, dk, dv, dlg, dmi = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    args = dict(q=q, k=k, v=v, lg=lg, m=m)
    grads = dict(q=dq, k=dk, v=dv, lg=dlg, m=dmi)
    h = 1e-6
    rng = np.random.default_rng(0)
    for name in args:
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in args[name].shape)
            vals = []
            for sgn in (1, -1):
                a = {n: x.copy() for n, x in args.items()}
                a[name][idx] += sgn * h
                o, mo = go.gated_recurrent_fwd(a["q"], a["k"], a["v"], a["lg"], a["m"])
                vals.append(loss(o, mo, do, dm))
            np.testing.assert_allclose(grads[name][idx], (vals[0] - vals[1]) / (2 * h),
                                       rtol=1e-6, atol=1e-8, err_msg=name)


def test_torch_autograd_of_an_independent_recurrence():
    """Machine differentiation of the recurrence written again in torch."""
    L, d = 9, 4
    q, k, v, lg, do, m, dm = case(L, d, 12, strong=True)
    t = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for n, x in dict(q=q, k=k, v=v, lg=lg, m=m).items()}
    kv = t["m"]
    outs = []
    for p in range(L):
        kv = torch.exp(t["lg"][p]).unsqueeze(1) * kv + torch.outer(t["k"][p], t["v"][p])
        outs.append(t["q"][p] @ kv)
    lt = (torch.stack(outs) * torch.tensor(do)).sum() + (kv * torch.tensor(dm)).sum()
    lt.backward()
    got = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    for g, n in zip(got, ("q", "k", "v", "lg", "m")):
        np.testing.assert_allclose(g, t[n].grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=n)


# --- exact invariances --------------------------------------------------------
def test_zero_gate_resets_the_state():
    """A gate of exactly 0 (log-gate -800: exp underflows to 0) at token p makes
    o_p.. and M_out independent of everything before p; with dO zero before p,
    the gradients of everything before p (and of M_in) are zero."""
    L, d, p = 12, 3, 5
    q, k, v, lg, do, m, dm = case(L, d, 13)
    lg[p] = -800.0
    o1, m1 = go.gated_recurrent_fwd(q, k, v, lg, m)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:p] += 1.0
    k2[:p] -= 2.0
    v2[:p] *= 3.0
    o2, m2 = go.gated_recurrent_fwd(q2, k2, v2, lg, 5 * m)
    np.testing.assert_array_equal(o1[p:], o2[p:])
    np.testing.assert_array_equal(m1, m2)
    do[:p] = 0.0
    dq, dk, dv, dlg, dmi = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    assert np.all(dk[:p] == 0) and np.all(dv[:p] == 0) and np.all(dmi == 0)


def test_split_into_two_calls_equals_one():
    L, d, s = 17, 4, 7
    q, k, v, lg, do, m, dm = case(L, d, 14)
    o, mo = go.gated_recurrent_fwd(q, k, v, lg, m)
    oa, ma = go.gated_recurrent_fwd(q[:s], k[:s], v[:s], lg[:s], m)
    ob, mb = go.gated_recurrent_fwd(q[s:], k[s:], v[s:], lg[s:], ma)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(mb, mo, rtol=1e-11, atol=1e-12)
    full = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    b = go.gated_recurrent_bwd(q[s:], k[s:], v[s:], lg[s:], do[s:], ma, dm)
    a = go.gated_recurrent_bwd(q[:s], k[:s], v[:s], lg[:s], do[:s], m, b[4])
    for i in range(4):
        np.testing.assert_allclose(np.concatenate([a[i], b[i]]), full[i], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(a[4], full[4], rtol=1e-10, atol=1e-11)


def test_key_channel_permutation():
    L, d = 10, 5
    q, k, v, lg, do, m, dm = case(L, d, 15)
    pi = np.array([3, 0, 4, 1, 2])
    o, mo = go.gated_recurrent_fwd(q, k, v, lg, m)
    op, mop = go.gated_recurrent_fwd(q[:, pi], k[:, pi], v, lg[:, pi], m[pi])
    np.testing.assert_allclose(op, o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(mop, mo[pi], rtol=1e-11, atol=1e-12)
    g = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    gp = go.gated_recurrent_bwd(q[:, pi], k[:, pi], v, lg[:, pi], do, m[pi], dm[pi])
    for i in (0, 1, 3):
        np.testing.assert_allclose(gp[i], g[i][:, pi], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gp[2], g[2], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(gp[4], g[4][pi], rtol=1e-10, atol=1e-11)


# --- drivers and sampled rows -------------------------------------------------
def test_batched_packed_equals_separate():
    r = np.random.default_rng(16)
    H, d, lens = 2, 3, [5, 0, 9, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    N = int(cu[-1])
    Q, K, V, dO = (r.standard_normal((1, H, N, d)) for _ in range(4))
    LG = -np.abs(r.standard_normal((1, H, N, d)))
    Mi, dMo = (r.standard_normal((len(lens), H, d, d)) for _ in range(2))
    O, Mo = go.batched_gated_fwd(Q, K, V, LG, Mi, cu)
    G = go.batched_gated_bwd(Q, K, V, LG, dO, Mi, dMo, cu)
    for i in range(len(lens)):
        s, e = cu[i], cu[i + 1]
        for h in range(H):
            o, mo = go.gated_recurrent_fwd(Q[0, h, s:e], K[0, h, s:e], V[0, h, s:e],
                                           LG[0, h, s:e], Mi[i, h])
            np.testing.assert_array_equal(O[0, h, s:e], o)
            np.testing.assert_array_equal(Mo[i, h], mo)
            g = go.gated_recurrent_bwd(Q[0, h, s:e], K[0, h, s:e], V[0, h, s:e],
                                       LG[0, h, s:e], dO[0, h, s:e], Mi[i, h], dMo[i, h])
            for j in range(4):
                np.testing.assert_array_equal(G[j][0, h, s:e], g[j])
            np.testing.assert_array_equal(G[4][i, h], g[4])


def test_sampled_rows_match_full():
    L, d = 40, 4
    q, k, v, lg, do, m, dm = case(L, d, 17, strong=True)
    o, mo = go.gated_recurrent_fwd(q, k, v, lg, m)
    dq, dk, dv, dlg, dmi = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    cm, cdm = go.gated_closed_states(q, k, v, lg, do, m, dm)
    np.testing.assert_allclose(cm, mo, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(cdm, dmi, rtol=1e-10, atol=1e-12)
    rows = [0, 1, 17, 38, 39]
    s = go.gated_sampled(q, k, v, lg, do, rows, m, dm)
    for name, full in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv), ("dLG", dlg)):
        np.testing.assert_allclose(s[name], full[rows], rtol=1e-9, atol=1e-11, err_msg=name)


# --- planted mistakes fail the pins --------------------------------------------
def _mistaken_fwd(kind):
    def fwd(q, k, v, lg, m_in=None):
        L, d = q.shape
        kv = np.zeros((d, d)) if m_in is None else np.array(m_in, dtype=np.float64)
        o = np.zeros((L, d))
        for p in range(L):
            g = np.exp(lg[p])
            if kind == "value_axis":
                kv = kv * g[None, :] + np.outer(k[p], v[p])
            elif kind == "gate_after_add":
                kv = g[:, None] * (kv + np.outer(k[p], v[p]))
            elif kind == "output_before_update":
                o[p] = q[p] @ kv
                kv = g[:, None] * kv + np.outer(k[p], v[p])
                continue
            o[p] = q[p] @ kv
        return o, kv
    return fwd


@pytest.mark.parametrize("kind", ["value_axis", "gate_after_add", "output_before_update"])
def test_planted_forward_mistakes_fail(kind):
    bad = _mistaken_fwd(kind)
    ex = json.load(open(GOLD))["examples"][0]
    a = {n: np.array(x, dtype=np.float64) for n, x in ex.items() if n not in ("name", "derivation")}
    o, mo = bad(a["q"], a["k"], a["v"], np.log(a["g"]), a["m_in"])
    hand_ok = np.allclose(o, a["o"]) and np.allclose(mo, a["m_out"])
    L, d = 11, 4
    q, k, v, _, do, m, dm = case(L, d, 8)
    lams = np.array([1.0, 0.8, 0.5, 0.95])
    ob, _ = bad(q, k, v, np.tile(np.log(lams), (L, 1)), m)
    osum = sum(lo.quadratic_fwd(q[:, c:c + 1], k[:, c:c + 1], v, lams[c], m[c:c + 1, :])[0]
               for c in range(d))
    split_ok = np.allclose(ob, osum)
    assert not (hand_ok and split_ok)


def test_planted_backward_mistake_fails():
    """dlog_g without the gate factor, and dM_in without the first gate."""
    ex = json.load(open(GOLD))["examples"][0]
    a = {n: np.array(x, dtype=np.float64) for n, x in ex.items() if n not in ("name", "derivation")}
    g0 = a["g"][0]
    dq, dk, dv, dlg, dmi = go.gated_recurrent_bwd(a["q"], a["k"], a["v"], np.log(a["g"]),
                                                  a["do"], a["m_in"], a["dm_out"])
    assert not np.allclose(dlg / np.exp(np.log(a["g"])), a["dlog_g"])
    assert not np.allclose(dmi / g0[:, None], a["dm_in"])


def test_log_gate_gradient_as_a_suffix_sum():
    """The identity the HIP backward uses for the log-gate gradient: with the
    cumulative log-gate B_p, the map depends on B through exp(B_p - B_i) and
    exp(B_p), so dl/dB_u = q_u * dq_u - k_u * dk_u (per channel), plus
    rowsum(dM_out . M_out) at the last token; the log-gate of token p enters
    every B_u with u >= p, so dlog_g_p is the suffix sum of these."""
    L, d = 21, 4
    q, k, v, lg, do, m, dm = case(L, d, 18, strong=True)
    _, mo = go.gated_recurrent_fwd(q, k, v, lg, m)
    dq, dk, dv, dlg, _ = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    dB = q * dq - k * dk
    dB[-1] += np.sum(dm * mo, axis=1)
    np.testing.assert_allclose(np.cumsum(dB[::-1], axis=0)[::-1], dlg, rtol=1e-9, atol=1e-10)
    # the part of the suffix past a split point s is rowsum(R . P): P the state
    # after token s-1 and R the gradient reaching it from the tokens from s on
    s = 8
    _, ma = go.gated_recurrent_fwd(q[:s], k[:s], v[:s], lg[:s], m)
    R = go.gated_recurrent_bwd(q[s:], k[s:], v[s:], lg[s:], do[s:], ma, dm)[4]
    np.testing.assert_allclose(np.sum(R * ma, axis=1), dB[s:].sum(axis=0), rtol=1e-9, atol=1e-10)


@pytest.mark.parametrize("a,b", [(0, 21), (5, 13), (20, 21), (0, 1), (7, 8)])
def test_span_total_from_the_inter_span_terms(a, b):
    """The identity the HIP backward carries its log-gate gradient sum with:
    over a span of tokens [a, b), the total of q_u dq_u - k_u dk_u equals that
    of the terms through the states at the span's ends only,
        sum_u q_u exp(C_u) (dO_u P^T) - k_u exp(C_last - C_u) (V_u R^T),
    C_u the running log-gate from the span start to u, P the state entering
    the span, R the gradient reaching the state after it (the terms between
    two tokens of the span cancel: a common shift of the span's running
    log-gates leaves them unchanged)."""
    L, d = 21, 4
    q, k, v, lg, do, m, dm = case(L, d, 19, strong=True)
    dq, dk, _, _, _ = go.gated_recurrent_bwd(q, k, v, lg, do, m, dm)
    P = go.gated_recurrent_fwd(q[:a], k[:a], v[:a], lg[:a], m)[1] if a else m
    _, mb = go.gated_recurrent_fwd(q[:b], k[:b], v[:b], lg[:b], m)
    R = go.gated_recurrent_bwd(q[b:], k[b:], v[b:], lg[b:], do[b:], mb, dm)[4] if b < L else dm
    C = np.cumsum(lg[a:b], axis=0)
    rhs = (q[a:b] * np.exp(C) * (do[a:b] @ P.T) - k[a:b] * np.exp(C[-1] - C) * (v[a:b] @ R.T)).sum(axis=0)
    lhs = (q[a:b] * dq[a:b] - k[a:b] * dk[a:b]).sum(axis=0)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-10)
    # and not with the in-span terms: they do not vanish token by token
    if b - a > 1:
        assert not np.allclose(q[a:b] * dq[a:b] - k[a:b] * dk[a:b],
                               q[a:b] * np.exp(C) * (do[a:b] @ P.T) - k[a:b] * np.exp(C[-1] - C) * (v[a:b] @ R.T))


@pytest.mark.parametrize("L,d,seed", [(1, 4, 0), (7, 3, 1), (200, 8, 2), (600, 16, 3)])
def test_sampled_sweep_matches_rows_and_closed_states(L, d, seed):
    """gated_sampled_sweep regroups the sums of gated_sampled (rows) and
    gated_closed_states (M_out, dM_in), both pinned above, into one pass each
    way: it must give the same values, rows 0 and L-1 and repeated rows
    included."""
    r = np.random.default_rng(seed)
    q, k, v, do = (r.standard_normal((L, d)) for _ in range(4))
    lg = np.log(1 / (1 + np.exp(-r.standard_normal((L, d))))) * 0.7
    mi, dmo = r.standard_normal((d, d)), r.standard_normal((d, d))
    rows = np.concatenate([[0, L - 1, L - 1], r.integers(0, L, 6)])
    a = go.gated_sampled(q, k, v, lg, do, np.unique(rows), mi, dmo)
    mo, dmi = go.gated_closed_states(q, k, v, lg, do, mi, dmo)
    b, mo2, dmi2 = go.gated_sampled_sweep(q, k, v, lg, do, rows, mi, dmo)
    for n in a:
        assert np.abs(a[n] - b[n]).max() <= 1e-12 * max(1.0, np.abs(a[n]).max()), n
    assert np.abs(mo - mo2).max() <= 1e-12 * max(1.0, np.abs(mo).max())
    assert np.abs(dmi - dmi2).max() <= 1e-12 * max(1.0, np.abs(dmi).max())
