"""The torch.autograd wrappers (chunked_causal_linear_amd.autograd) on the GPU.

Gradients through autograd must be the bits of the direct backward calls on
the same inputs (the wrappers only marshal arguments and keep the forward's
state cache), and match the CPU oracle at the parity bar.
"""
import numpy as np
import pytest
import torch

import chunked_causal_linear_amd as cca
from chunked_causal_linear_amd.autograd import (lasp_attention, lasp_bidir_attention,
                                                lasp_gated_attention)
from chunked_causal_linear_amd.workloads import make_inputs, small
from oracle import lasp_oracle as lo

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cca.lib()
    yield


def case(dtype="bf16", decay=True, m_in=True, d=64, chunk=64, N=300, seed=7, gates="none"):
    w = small("autograd", dtype=dtype, B=2, H=2, N=N, d=d, chunk=chunk, seed=seed,
              decay="lightning" if decay else "none", m_in_scale=0.05 if m_in else None,
              dm_out_scale=0.05, gates=gates)
    inp = make_inputs(w)
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}


def leaf(t):
    return None if t is None else t.detach().clone().requires_grad_(True)


def rel(a, ref):
    a = a.detach().double().cpu().numpy()
    den = np.abs(ref).max()
    return float(np.abs(a - ref).max() / (den if den > 0 else 1.0))


def test_causal_matches_direct_and_oracle():
    inp = case()
    sh = inp["shape"]
    Q, K, V, M_in = leaf(inp["Q"]), leaf(inp["K"]), leaf(inp["V"]), leaf(inp["M_in"])
    O, M_out = lasp_attention(Q, K, V, sh["chunk"], inp["decay"], None, M_in)
    loss = (O.float() * inp["dO"].float()).sum() + (M_out * inp["dM_out"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    # direct calls on the same inputs
    O2, Mo2, cache = cca.fwd(inp["Q"], inp["K"], inp["V"], sh["chunk"], inp["decay"], None, inp["M_in"])
    g = cca.bwd(inp["Q"], inp["K"], inp["V"], inp["dO"], sh["chunk"], inp["decay"], None, inp["M_in"],
                inp["dM_out"], cache)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(M_out, Mo2)
    for got, want in zip((Q.grad, K.grad, V.grad, M_in.grad), g):
        assert torch.equal(got, want)
    # oracle
    a = {k: inp[k].double().cpu().numpy() for k in ("Q", "K", "V", "dO", "M_in", "dM_out", "decay")}
    dQ, dK, dV, dMi = lo.batched_bwd(a["Q"], a["K"], a["V"], a["dO"], a["decay"], a["M_in"], a["dM_out"], None)
    for got, ref in zip((Q.grad, K.grad, V.grad, M_in.grad), (dQ, dK, dV, dMi)):
        assert rel(got, ref) <= 2e-2


def test_causal_output_gradient_only_and_no_m_in_gradient():
    """Only M_out in the loss: the library gets dO = 0; M_in without
    requires_grad gets no dM_in."""
    inp = case(dtype="fp32")
    sh = inp["shape"]
    Q, K, V = leaf(inp["Q"]), leaf(inp["K"]), leaf(inp["V"])
    O, M_out = lasp_attention(Q, K, V, sh["chunk"], inp["decay"], None, inp["M_in"])
    (M_out * inp["dM_out"]).sum().backward()
    torch.cuda.synchronize()
    zero = torch.zeros_like(inp["Q"])
    _, _, cache = cca.fwd(inp["Q"], inp["K"], inp["V"], sh["chunk"], inp["decay"], None, inp["M_in"])
    g = cca.bwd(inp["Q"], inp["K"], inp["V"], zero, sh["chunk"], inp["decay"], None, inp["M_in"],
                inp["dM_out"], cache)
    torch.cuda.synchronize()
    for got, want in zip((Q.grad, K.grad, V.grad), g[:3]):
        assert torch.equal(got, want)


def test_norm_matches_direct():
    inp = case(decay=False)
    sh = inp["shape"]
    Q, K, V = leaf(inp["Q"]), leaf(inp["K"]), leaf(inp["V"])
    Y, M_out = lasp_attention(Q, K, V, sh["chunk"], None, None, inp["M_in"], norm=True)
    (Y.float() * inp["dO"].float()).sum().backward()
    torch.cuda.synchronize()
    Y2, rstd, _, cache = cca.fwd_norm(inp["Q"], inp["K"], inp["V"], sh["chunk"], None, None, inp["M_in"])
    g = cca.bwd_norm(inp["Q"], inp["K"], inp["V"], Y2, rstd, inp["dO"], sh["chunk"], None, None,
                     inp["M_in"], None, cache)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
    for got, want in zip((Q.grad, K.grad, V.grad), g[:3]):
        assert torch.equal(got, want)


def test_gated_matches_direct():
    inp = case(decay=False, chunk=64, gates="gla")
    log_g = inp["log_g"]
    Q, K, V, LG, M_in = leaf(inp["Q"]), leaf(inp["K"]), leaf(inp["V"]), leaf(log_g), leaf(inp["M_in"])
    O, M_out = lasp_gated_attention(Q, K, V, LG, 64, None, M_in)
    loss = (O.float() * inp["dO"].float()).sum() + (M_out * inp["dM_out"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    _, _, cache = cca.fwd_gated(inp["Q"], inp["K"], inp["V"], log_g, 64, None, inp["M_in"])
    g = cca.bwd_gated(inp["Q"], inp["K"], inp["V"], log_g, inp["dO"], 64, None, inp["M_in"],
                      inp["dM_out"], cache)
    torch.cuda.synchronize()
    for got, want in zip((Q.grad, K.grad, V.grad, LG.grad, M_in.grad), g):
        assert torch.equal(got, want)


def test_bidir_matches_direct():
    inp = case(decay=False, chunk=64)
    Q, K, V, M_in = leaf(inp["Q"]), leaf(inp["K"]), leaf(inp["V"]), leaf(inp["M_in"])
    O, M_out = lasp_bidir_attention(Q, K, V, 64, None, M_in)
    loss = (O.float() * inp["dO"].float()).sum() + (M_out * inp["dM_out"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    _, _, cache = cca.fwd_bidir(inp["Q"], inp["K"], inp["V"], 64, None, inp["M_in"])
    g = cca.bwd_bidir(inp["Q"], inp["K"], inp["V"], inp["dO"], 64, None, inp["M_in"], inp["dM_out"], cache)
    torch.cuda.synchronize()
    for got, want in zip((Q.grad, K.grad, V.grad, M_in.grad), g):
        assert torch.equal(got, want)
