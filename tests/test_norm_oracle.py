"""Pins of the Norm(.) oracle (oracle/norm_oracle.py, the reading of [LASP]
Sec. 3.1, Eq. 2 stated there), each chosen so that a plausible mistake fails:
  * hand-worked values (tests/golden/norm_hand.json), rows and end to end;
  * finite differences of l = <dY, Norm(O(Q, K, V, M_in))> + <dM_out, M_out>
    with respect to Q, K, V and M_in (decay on), through the pinned causal oracle;
  * exact identities: every output row has mean square ms/(ms + eps); the
    gradient of a row satisfies <dO, O> = r <dY, O> eps/(ms + eps), i.e. it is
    orthogonal to O when eps = 0; Norm(c O) = Norm(O) for c > 0 when eps = 0;
  * planted mistakes (the mean term dropped, Y in place of O, the mean over
    the wrong axis) are caught by the finite-difference pin.
"""
import json
import os

import numpy as np
import pytest

from oracle import lasp_oracle as lo
from oracle import norm_oracle as no

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "norm_hand.json")))


def test_hand_rows():
    for ex in GOLD["row_examples"]:
        y, r = no.norm_fwd(np.array(ex["o"], float), eps=ex["eps"])
        assert np.allclose(y, ex["y"], atol=1e-14, rtol=0) and abs(r - ex["r"]) < 1e-14
        do = no.norm_bwd(y, r, np.array(ex["dy"], float))
        assert np.allclose(do, ex["do"], atol=1e-14, rtol=0)


def test_hand_causal():
    ex = GOLD["causal_example"]
    f = lambda a: np.array(a, float)[None, None]
    Y, r, _ = no.batched_norm_fwd(f(ex["q"]), f(ex["k"]), f(ex["v"]), eps=0.0)
    assert np.allclose(Y[0, 0], ex["y"], atol=1e-14, rtol=0)
    assert np.allclose(r[0, 0], ex["rstd"], atol=1e-14, rtol=0)


def _problem(seed, L=7, d=4, H=1):
    r = np.random.default_rng(seed)
    q, k, v = (r.standard_normal((1, H, L, d)) for _ in range(3))
    dy = r.standard_normal((1, H, L, d))
    m_in = r.standard_normal((1, H, d, d)) * 0.3
    dm_out = r.standard_normal((1, H, d, d)) * 0.3
    return q, k, v, dy, m_in, dm_out


def _loss(q, k, v, dy, decay, m_in, dm_out, eps):
    Y, _, M = no.batched_norm_fwd(q, k, v, decay, m_in, eps=eps)
    return float(np.sum(dy * Y) + np.sum(dm_out * M))


def _fd_check(grad_fn, eps=no.NORM_EPS, seed=3):
    q, k, v, dy, m_in, dm_out = _problem(seed)
    decay = np.array([0.8])
    got = dict(zip(("Q", "K", "V", "M_in"), grad_fn(q, k, v, dy, decay, m_in, dm_out, eps)))
    h, worst = 1e-6, 0.0
    args = {"Q": q, "K": k, "V": v, "M_in": m_in}
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            a = dict(args, **{name: xp})
            b = dict(args, **{name: xm})
            fd[idx] = (_loss(a["Q"], a["K"], a["V"], dy, decay, a["M_in"], dm_out, eps)
                       - _loss(b["Q"], b["K"], b["V"], dy, decay, b["M_in"], dm_out, eps)) / (2 * h)
        worst = max(worst, float(np.abs(fd - got[name]).max()))
    return worst


def _grads(q, k, v, dy, decay, m_in, dm_out, eps):
    dq, dk, dv, dmi = no.batched_norm_bwd(q, k, v, dy, decay, m_in, dm_out, eps=eps)
    return dq, dk, dv, dmi


@pytest.mark.parametrize("eps", [no.NORM_EPS, 0.5])
def test_finite_differences(eps):
    assert _fd_check(_grads, eps) < 1e-7


def test_row_identities():
    r = np.random.default_rng(9)
    o = r.standard_normal((50, 16)) * r.uniform(0.01, 3, (50, 1))
    dy = r.standard_normal((50, 16))
    for eps in (0.0, 1e-6, 0.3):
        y, rs = no.norm_fwd(o, eps)
        ms = np.mean(o * o, axis=-1)
        assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13, atol=0)
        do = no.norm_bwd(y, rs, dy)
        lhs = np.sum(do * o, axis=-1)
        rhs = rs * np.sum(dy * o, axis=-1) * eps / (ms + eps)
        assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-12)
    y1, _ = no.norm_fwd(o, 0.0)
    y2, _ = no.norm_fwd(3.7 * o, 0.0)
    assert np.allclose(y1, y2, rtol=1e-14, atol=1e-14)


def _mistake_no_mean(q, k, v, dy, decay, m_in, dm_out, eps):
    O, _ = lo.batched_fwd(q, k, v, decay, m_in)
    Y, r = no.norm_fwd(O, eps)
    return lo.batched_bwd(q, k, v, r[..., None] * dy, decay, m_in, dm_out)


def _mistake_o_for_y(q, k, v, dy, decay, m_in, dm_out, eps):
    O, _ = lo.batched_fwd(q, k, v, decay, m_in)
    Y, r = no.norm_fwd(O, eps)
    return lo.batched_bwd(q, k, v, no.norm_bwd(O, r, dy), decay, m_in, dm_out)


def _mistake_axis(q, k, v, dy, decay, m_in, dm_out, eps):
    O, _ = lo.batched_fwd(q, k, v, decay, m_in)
    Y, r = no.norm_fwd(O, eps)
    m = np.mean(dy * Y, axis=-2, keepdims=True)
    return lo.batched_bwd(q, k, v, r[..., None] * (dy - Y * m), decay, m_in, dm_out)


@pytest.mark.parametrize("bad", [_mistake_no_mean, _mistake_o_for_y, _mistake_axis])
def test_planted_mistakes_are_caught(bad):
    assert _fd_check(bad) > 1e-3
