"""Pins for the CPU oracle (no GPU).

Each check ties the oracle to something other than itself: hand-worked values,
an independent formulation, finite differences, closed forms, exact identities,
or special cases.  A planted-mistake test shows the checks catch the typical
slips (a transposed state, a dropped term, an off-by-one decay power).
"""
import json
import os

import numpy as np
import pytest

from oracle import lasp_oracle as lo
from oracle import crecurrent

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_case(L, d, seed, lam=1.0, with_m=True, dv=None):
    r = np.random.default_rng(seed)
    dv = d if dv is None else dv
    q, k = r.standard_normal((L, d)), r.standard_normal((L, d))
    v, do = r.standard_normal((L, dv)), r.standard_normal((L, dv))
    m = r.standard_normal((d, dv)) if with_m else None
    dm = r.standard_normal((d, dv)) if with_m else None
    return q, k, v, do, m, dm


# --- hand-worked values (tests/golden/hand_examples.json) -------------------
@pytest.mark.parametrize("form", ["quadratic", "recurrent", "chunked1", "chunked2"])
def test_hand_examples(form):
    for ex in json.load(open(GOLD))["examples"]:
        a = {k: np.array(v, dtype=np.float64) for k, v in ex.items()
             if k not in ("name", "derivation", "lam")}
        lam = ex["lam"]
        if form == "quadratic":
            o, mo = lo.quadratic_fwd(a["q"], a["k"], a["v"], lam, a["m_in"])
            g = lo.quadratic_bwd(a["q"], a["k"], a["v"], a["do"], lam, a["m_in"], a["dm_out"])
        elif form == "recurrent":
            o, mo = lo.recurrent_fwd(a["q"], a["k"], a["v"], lam, a["m_in"])
            g = lo.recurrent_bwd(a["q"], a["k"], a["v"], a["do"], lam, a["m_in"], a["dm_out"])
        else:
            C = int(form[-1])
            o, mo = lo.chunked_fwd(a["q"], a["k"], a["v"], C, lam, a["m_in"])
            g = lo.chunked_bwd(a["q"], a["k"], a["v"], a["do"], C, lam, a["m_in"], a["dm_out"])
        np.testing.assert_allclose(o, a["o"], atol=1e-12)
        np.testing.assert_allclose(mo, a["m_out"], atol=1e-12)
        for got, key in zip(g, ["dq", "dk", "dv", "dm_in"]):
            np.testing.assert_allclose(got, a[key], atol=1e-12, err_msg=ex["name"] + key)


# --- two independent formulations agree (Eq. 4 vs Eq. 5; Eq. 12-13) --------
@pytest.mark.parametrize("L,d,lam,with_m", [(0, 3, 0.9, True), (1, 4, 1.0, True),
                                             (17, 5, 0.9, True), (24, 3, 1.0, False),
                                             (33, 4, 1.1, True), (20, 2, 0.0, True)])
def test_quadratic_equals_recurrent(L, d, lam, with_m):
    q, k, v, do, m, dm = rand_case(L, d, 1 + L, lam, with_m)
    o1, m1 = lo.quadratic_fwd(q, k, v, lam, m)
    o2, m2 = lo.recurrent_fwd(q, k, v, lam, m)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(m1, m2, atol=1e-12)
    g1 = lo.quadratic_bwd(q, k, v, do, lam, m, dm)
    g2 = lo.recurrent_bwd(q, k, v, do, lam, m, dm)
    for a, b in zip(g1, g2):
        np.testing.assert_allclose(a, b, atol=1e-11)


def test_rectangular_value_dim():
    q, k, v, do, m, dm = rand_case(13, 3, 7, with_m=True, dv=5)
    o1, m1 = lo.quadratic_fwd(q, k, v, 0.8, m)
    o2, m2 = lo.recurrent_fwd(q, k, v, 0.8, m)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(m1, m2, atol=1e-12)


# --- chunk invariance: the intra/inter decomposition equals the definition --
@pytest.mark.parametrize("lam", [1.0, 0.9, 0.97])
def test_chunk_invariance(lam):
    L, d = 24, 5
    q, k, v, do, m, dm = rand_case(L, d, 3, lam)
    o_ref, m_ref = lo.quadratic_fwd(q, k, v, lam, m)
    g_ref = lo.quadratic_bwd(q, k, v, do, lam, m, dm)
    for C in [1, 2, 3, 4, 5, 6, 7, 8, 12, 24, 31]:
        o, mo = lo.chunked_fwd(q, k, v, C, lam, m)
        np.testing.assert_allclose(o, o_ref, atol=1e-12, err_msg=f"C={C}")
        np.testing.assert_allclose(mo, m_ref, atol=1e-12)
        g = lo.chunked_bwd(q, k, v, do, C, lam, m, dm)
        for a, b in zip(g, g_ref):
            np.testing.assert_allclose(a, b, atol=1e-11, err_msg=f"C={C}")


# --- finite differences of l = <dO,O> + <dM_out,M_out> ----------------------
def _loss(q, k, v, do, lam, m, dm):
    o, mo = lo.quadratic_fwd(q, k, v, lam, m)
    return float(np.sum(do * o) + np.sum(dm * mo))


def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("lam", [1.0, 0.85])
@pytest.mark.parametrize("bwd", ["quadratic", "recurrent"])
def test_finite_differences(lam, bwd):
    L, d = 9, 3
    q, k, v, do, m, dm = rand_case(L, d, 11, lam)
    f = lambda: _loss(q, k, v, do, lam, m, dm)
    fn = lo.quadratic_bwd if bwd == "quadratic" else lo.recurrent_bwd
    dq, dk, dv, dmi = fn(q, k, v, do, lam, m, dm)
    for x, g in [(q, dq), (k, dk), (v, dv), (m, dmi)]:
        np.testing.assert_allclose(g, _fd(f, x), atol=2e-7)


# --- closed forms and special cases -----------------------------------------
def test_m_out_closed_form_and_kTv():
    q, k, v, do, m, dm = rand_case(40, 4, 5)
    _, mo = lo.recurrent_fwd(q, k, v, 0.93, m)
    np.testing.assert_allclose(mo, lo.closed_m_out(k, v, 0.93, m), atol=1e-12)
    # lambda = 1, no incoming state: the plain K^T V state (Eq. 3; LASP-2's M_t)
    _, mo = lo.recurrent_fwd(q, k, v, 1.0, None)
    np.testing.assert_allclose(mo, k.T @ v, atol=1e-12)
    dmi = lo.recurrent_bwd(q, k, v, do, 0.93, m, dm)[3]
    np.testing.assert_allclose(dmi, lo.closed_dm_in(q, do, 0.93, dm), atol=1e-12)


def test_last_row_reads_m_out():
    # o_{L-1} = q_{L-1} kv_{L-1} and kv_{L-1} = M_out (Eq. 5 at the last token)
    q, k, v, do, m, dm = rand_case(19, 4, 6)
    o, mo = lo.quadratic_fwd(q, k, v, 0.9, m)
    np.testing.assert_allclose(o[-1], q[-1] @ mo, atol=1e-12)


def test_zero_decay_is_diagonal_only():
    # lambda = 0: only the current token contributes (0^0 = 1 on the diagonal)
    q, k, v, do, m, dm = rand_case(11, 3, 8)
    o, mo = lo.quadratic_fwd(q, k, v, 0.0, m)
    np.testing.assert_allclose(o, np.sum(q * k, 1)[:, None] * v, atol=1e-12)
    np.testing.assert_allclose(mo, np.outer(k[-1], v[-1]), atol=1e-12)


def test_causality():
    # changing a future token never changes an earlier output
    q, k, v, do, m, dm = rand_case(15, 3, 9)
    o1, _ = lo.quadratic_fwd(q, k, v, 0.9, m)
    k2, v2 = k.copy(), v.copy()
    k2[10:] += 1.0
    v2[10:] -= 2.0
    o2, _ = lo.quadratic_fwd(q, k2, v2, 0.9, m)
    np.testing.assert_allclose(o1[:10], o2[:10], atol=1e-13)
    assert np.abs(o1[10:] - o2[10:]).max() > 1e-3


# --- exact identities that hold at any size ---------------------------------
def test_homogeneity_identities():
    L, d, lam = 50, 4, 0.95
    q, k, v, do, m, dm = rand_case(L, d, 12, lam)
    o, mo = lo.quadratic_fwd(q, k, v, lam, m)
    dq, dk, dv, dmi = lo.quadratic_bwd(q, k, v, do, lam, m, dm)
    o_m = lo.quadratic_fwd(np.asarray(q), np.zeros_like(k), np.zeros_like(v), lam, m)[0]
    ip = lambda a, b: float(np.sum(a * b))
    np.testing.assert_allclose(ip(dq, q), ip(do, o) + 0.0, rtol=1e-11)
    rhs = ip(do, o - o_m) + ip(dm, mo - lam ** L * m)
    np.testing.assert_allclose(ip(dk, k), rhs, rtol=1e-11)
    np.testing.assert_allclose(ip(dv, v), rhs, rtol=1e-11)
    np.testing.assert_allclose(ip(dmi, m), ip(do, o_m) + ip(dm, lam ** L * m), rtol=1e-11)


def test_split_invariance():
    # whole sequence == first part, then its M_out fed as M_in of the second part;
    # backward: dM_in of the second part seeds dM_out of the first part
    L, d, lam, cut = 37, 4, 0.9, 16
    q, k, v, do, m, dm = rand_case(L, d, 13, lam)
    o, mo = lo.quadratic_fwd(q, k, v, lam, m)
    o1, mo1 = lo.quadratic_fwd(q[:cut], k[:cut], v[:cut], lam, m)
    o2, mo2 = lo.quadratic_fwd(q[cut:], k[cut:], v[cut:], lam, mo1)
    np.testing.assert_allclose(np.concatenate([o1, o2]), o, atol=1e-12)
    np.testing.assert_allclose(mo2, mo, atol=1e-12)
    g = lo.quadratic_bwd(q, k, v, do, lam, m, dm)
    g2 = lo.quadratic_bwd(q[cut:], k[cut:], v[cut:], do[cut:], lam, mo1, dm)
    g1 = lo.quadratic_bwd(q[:cut], k[:cut], v[:cut], do[:cut], lam, m, g2[3])
    for i in range(3):
        np.testing.assert_allclose(np.concatenate([g1[i], g2[i]]), g[i], atol=1e-11)
    np.testing.assert_allclose(g1[3], g[3], atol=1e-11)


def test_linearity():
    q, k, v, do, m, dm = rand_case(21, 3, 14)
    v2 = np.random.default_rng(1).standard_normal(v.shape)
    a = lo.quadratic_fwd(q, k, v + v2, 0.9, None)[0]
    b = lo.quadratic_fwd(q, k, v, 0.9, None)[0] + lo.quadratic_fwd(q, k, v2, 0.9, None)[0]
    np.testing.assert_allclose(a, b, atol=1e-12)


# --- batched drivers: packed batches and per-head decay ---------------------
def test_batched_varlen_equals_separate_and_per_head_decay():
    r = np.random.default_rng(15)
    lens = [5, 1, 0, 9, 4]
    N, H, d = sum(lens), 3, 4
    Q, K, V, dO = (r.standard_normal((1, H, N, d)) for _ in range(4))
    decay = np.array([1.0, 0.9, 0.5])
    cu = np.concatenate([[0], np.cumsum(lens)])
    m_in = r.standard_normal((len(lens), H, d, d))
    dm = r.standard_normal((len(lens), H, d, d))
    O, Mo = lo.batched_fwd(Q, K, V, decay, m_in, cu)
    G = lo.batched_bwd(Q, K, V, dO, decay, m_in, dm, cu)
    for i, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        for h in range(H):
            o, mo = lo.quadratic_fwd(Q[0, h, s:e], K[0, h, s:e], V[0, h, s:e], decay[h],
                                     m_in[i, h])
            np.testing.assert_allclose(O[0, h, s:e], o, atol=1e-12)
            np.testing.assert_allclose(Mo[i, h], mo, atol=1e-12)
            g = lo.recurrent_bwd(Q[0, h, s:e], K[0, h, s:e], V[0, h, s:e], dO[0, h, s:e],
                                 decay[h], m_in[i, h], dm[i, h])
            np.testing.assert_allclose(G[0][0, h, s:e], g[0], atol=1e-11)
            np.testing.assert_allclose(G[3][i, h], g[3], atol=1e-11)
    # empty sequence: M_out = M_in, dM_in = dM_out
    np.testing.assert_allclose(Mo[2], m_in[2], atol=0)
    np.testing.assert_allclose(G[3][2], dm[2], atol=0)
    # decay=None equals an all-ones decay array
    O1, _ = lo.batched_fwd(Q, K, V, None, None, cu)
    O2, _ = lo.batched_fwd(Q, K, V, np.ones(H), None, cu)
    np.testing.assert_allclose(O1, O2, atol=0)


def test_sampled_rows_match_full():
    L, d, lam = 70, 4, 0.97
    q, k, v, do, m, dm = rand_case(L, d, 16, lam)
    o, _ = lo.quadratic_fwd(q, k, v, lam, m)
    dq, dk, dv, _ = lo.quadratic_bwd(q, k, v, do, lam, m, dm)
    rows = [0, 1, 33, 69]
    np.testing.assert_allclose(lo.sampled_o(q, k, v, rows, lam, m), o[rows], atol=1e-12)
    np.testing.assert_allclose(lo.sampled_dq(q, k, v, do, rows, lam, m), dq[rows], atol=1e-12)
    np.testing.assert_allclose(lo.sampled_dk(q, k, v, do, rows, lam, dm), dk[rows], atol=1e-12)
    np.testing.assert_allclose(lo.sampled_dv(q, k, v, do, rows, lam, dm), dv[rows], atol=1e-12)


# --- the C recurrence equals the numpy definition ---------------------------
def test_c_recurrence_matches_quadratic():
    r = np.random.default_rng(17)
    B, H, N, d = 2, 3, 45, 8
    Q, K, V, dO = (r.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(4))
    decay = np.array([1.0, 0.9, 0.7], dtype=np.float32)
    m_in = r.standard_normal((B, H, d, d))
    dm = r.standard_normal((B, H, d, d))
    ref_o, ref_m = lo.batched_fwd(Q, K, V, decay, m_in)
    ref = lo.batched_bwd(Q, K, V, dO, decay, m_in, dm)
    out = crecurrent.run(Q, K, V, dO, decay, m_in, dm)
    np.testing.assert_allclose(out["O"], ref_o, atol=1e-10)
    np.testing.assert_allclose(out["M_out"], ref_m, atol=1e-10)
    for key, a in zip(["dQ", "dK", "dV", "dM_in"], ref):
        np.testing.assert_allclose(out[key], a, atol=1e-9, err_msg=key)
    # varlen through the C driver
    lens = [10, 0, 35]
    cu = np.concatenate([[0], np.cumsum(lens)])
    Q1, K1, V1, dO1 = Q[:1], K[:1], V[:1], dO[:1]
    ref_o, ref_m = lo.batched_fwd(Q1, K1, V1, None, None, cu)
    out = crecurrent.run(Q1, K1, V1, dO1, None, None, None, cu)
    np.testing.assert_allclose(out["O"], ref_o, atol=1e-10)
    np.testing.assert_allclose(out["M_out"], ref_m, atol=1e-10)


# --- planted mistakes are caught --------------------------------------------
def test_planted_mistakes_fail_the_pins():
    """Mutated copies of the backward must fail the finite-difference pin; a
    mutated forward must fail the hand example.  Guards the strength of the pins."""
    L, d, lam = 7, 3, 0.8
    q, k, v, do, m, dm = rand_case(L, d, 21, lam)
    f = lambda: _loss(q, k, v, do, lam, m, dm)
    fd = [_fd(f, x) for x in (q, k, v, m)]

    def good():
        return lo.quadratic_bwd(q, k, v, do, lam, m, dm)

    def transposed_state():       # uses M_in instead of M_in^T in dq
        dq, dk, dv, dmi = good()
        lr = lam ** np.arange(1, L + 1)
        return dq - lr[:, None] * (do @ m.T) + lr[:, None] * (do @ m), dk, dv, dmi

    def dropped_dm_out_term():    # forgets the carried dM_out in dk
        dq, dk, dv, dmi = good()
        g = lam ** np.arange(L - 1, -1, -1)
        return dq, dk - g[:, None] * (v @ dm.T), dv, dmi

    def off_by_one_decay():       # lam^p instead of lam^(p+1) for the M_in term
        dq, dk, dv, dmi = good()
        return dq, dk, dv, dmi / lam

    def ok(gr):
        return all(np.allclose(a, b, atol=2e-7) for a, b in zip(gr, fd))

    assert ok(good())
    for bad in (transposed_state, dropped_dm_out_term, off_by_one_decay):
        assert not ok(bad()), bad.__name__


# --- the unmasked (bidirectional) form ---------------------------------------
def _bidir_loss(q, k, v, do, m, dm):
    o, mo = lo.bidir_fwd(q, k, v, m)
    return float(np.sum(do * o) + np.sum(dm * mo))


def test_bidir_is_causal_plus_reversed_causal():
    """Without a mask every token sees the tokens up to it (the causal oracle,
    lambda = 1) and the tokens from it on (the causal oracle on the reversed
    sequence), the diagonal counted once; M_in enters once, M_out is the causal
    M_out."""
    q, k, v, do, m, dm = rand_case(23, 5, 31)
    o, mo = lo.bidir_fwd(q, k, v, m)
    oc, moc = lo.quadratic_fwd(q, k, v, 1.0, m)
    orr, _ = lo.quadratic_fwd(q[::-1], k[::-1], v[::-1], 1.0, None)
    diag = np.sum(q * k, axis=1)[:, None] * v
    np.testing.assert_allclose(o, oc + orr[::-1] - diag, atol=1e-11)
    np.testing.assert_allclose(mo, moc, atol=1e-11)


def test_bidir_loops_tiny():
    """Pure-Python double loop over token pairs and features (no matrix products)."""
    q, k, v, do, m, dm = rand_case(4, 3, 37)
    L, d = q.shape
    ref = [[sum(sum(q[p][a] * k[i][a] for a in range(d)) * v[i][n] for i in range(L)) +
            sum(q[p][a] * m[a][n] for a in range(d)) for n in range(d)] for p in range(L)]
    o, _ = lo.bidir_fwd(q, k, v, m)
    np.testing.assert_allclose(o, np.array(ref), atol=1e-12)


def test_bidir_finite_differences():
    q, k, v, do, m, dm = rand_case(8, 3, 41)
    f = lambda: _bidir_loss(q, k, v, do, m, dm)
    dq, dk, dv, dmi = lo.bidir_bwd(q, k, v, do, m, dm)
    for x, g in [(q, dq), (k, dk), (v, dv), (m, dmi)]:
        np.testing.assert_allclose(g, _fd(f, x), atol=2e-7)
    # planted mistakes fail the same pin: M_in untransposed in dq, dM_out^T in dv
    assert not np.allclose(dq - do @ m.T + do @ m, _fd(f, q), atol=2e-7)
    assert not np.allclose(dv - k @ dm + k @ dm.T, _fd(f, v), atol=2e-7)


def test_bidir_permutation_invariance():
    """Reordering the tokens permutes O's rows and leaves M_out unchanged."""
    q, k, v, do, m, dm = rand_case(17, 4, 43)
    perm = np.random.default_rng(5).permutation(17)
    o, mo = lo.bidir_fwd(q, k, v, m)
    op, mop = lo.bidir_fwd(q[perm], k[perm], v[perm], m)
    np.testing.assert_allclose(op, o[perm], atol=1e-11)
    np.testing.assert_allclose(mop, mo, atol=1e-11)


def test_bidir_batched_varlen():
    rng = np.random.default_rng(7)
    H, d, lens = 2, 4, [5, 0, 9, 1]
    cu = np.cumsum([0] + lens)
    N = int(cu[-1])
    Q, K, V, dO = (rng.standard_normal((1, H, N, d)) for _ in range(4))
    Mi, dMo = (rng.standard_normal((len(lens), H, d, d)) for _ in range(2))
    O, Mo = lo.batched_bidir_fwd(Q, K, V, Mi, cu)
    dQ, dK, dV, dMi = lo.batched_bidir_bwd(Q, K, V, dO, Mi, dMo, cu)
    for i, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        for h in range(H):
            o, mo = lo.bidir_fwd(Q[0, h, s:e], K[0, h, s:e], V[0, h, s:e], Mi[i, h])
            np.testing.assert_allclose(O[0, h, s:e], o)
            np.testing.assert_allclose(Mo[i, h], mo)
            g = lo.bidir_bwd(Q[0, h, s:e], K[0, h, s:e], V[0, h, s:e], dO[0, h, s:e], Mi[i, h], dMo[i, h])
            for a, b in zip((dQ[0, h, s:e], dK[0, h, s:e], dV[0, h, s:e], dMi[i, h]), g):
                np.testing.assert_allclose(a, b)


def test_bidir_sampled_rows_match_full():
    q, k, v, do, m, dm = rand_case(31, 4, 47)
    rows = [0, 5, 30]
    got = lo.bidir_sampled(q, k, v, do, rows, m, dm)
    o, mo = lo.bidir_fwd(q, k, v, m)
    dq, dk, dv, dmi = lo.bidir_bwd(q, k, v, do, m, dm)
    for name, full in (("O", o[rows]), ("dQ", dq[rows]), ("dK", dk[rows]), ("dV", dv[rows]),
                       ("M_out", mo), ("dM_in", dmi)):
        np.testing.assert_allclose(got[name], full, atol=1e-10)
