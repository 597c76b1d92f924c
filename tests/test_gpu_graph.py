"""The library's calls under HIP graph capture.

A forward + backward step (and a gated one) issues only kernel launches on the
caller's stream: no memsets, copies or host synchronisation outside the debug
path, so it can be captured into a HIP graph and replayed.  The test captures
one step through the Python binding, then, several times, writes new inputs
into the captured buffers, runs unrelated eager work and synchronises, replays
the graph and compares every output with an eager call on the same inputs
(bit for bit: the same kernels with the same launch shapes run in both)."""
import pytest
import torch

import chunked_causal_linear_amd as cca
from chunked_causal_linear_amd.workloads import make_inputs, small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cca.lib()
    yield


def fresh(w, seed):
    import dataclasses
    inp = make_inputs(dataclasses.replace(w, seed=seed))
    return {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in inp.items()}


def check_replays(w, step, names, replays=3):
    static = fresh(w, 500)
    # warm up on a side stream (first-call work stays out of the capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step(static)
    for r in range(replays):
        new = fresh(w, 501 + r)
        for k in names:
            static[k].copy_(new[k])
        junk = torch.randn(1 << 20, device="cuda").cumsum(0)   # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = step(new)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            if a is not None:
                assert torch.equal(a, b), "replay %d differs from the eager call" % r
        del junk


def test_causal_step_replays_in_a_graph():
    w = small("graph bf16 d128 C256 decay", "bf16", B=2, H=4, N=2000, d=128, chunk=256, seed=500,
              decay="lightning", m_in_scale=0.05, dm_out_scale=0.05)

    def step(x):
        C = x["shape"]["chunk"]
        O, M_out, cache = cca.fwd(x["Q"], x["K"], x["V"], C, x["decay"], None, x["M_in"])
        g = cca.bwd(x["Q"], x["K"], x["V"], x["dO"], C, x["decay"], None, x["M_in"], x["dM_out"], cache)
        return (O, M_out) + tuple(g)

    check_replays(w, step, ["Q", "K", "V", "dO", "M_in", "dM_out"])


def test_packed_no_decay_step_replays_in_a_graph():
    w = small("graph bf16 packed d64 C128", "bf16", H=2, d=64, chunk=128, seed=500,
              lengths=[300, 1, 0, 777, 128], m_in_scale=0.05, dm_out_scale=0.05)

    def step(x):
        C = x["shape"]["chunk"]
        O, M_out, cache = cca.fwd(x["Q"], x["K"], x["V"], C, None, x["cu_seqlens"], x["M_in"])
        g = cca.bwd(x["Q"], x["K"], x["V"], x["dO"], C, None, x["cu_seqlens"], x["M_in"], x["dM_out"],
                    cache)
        return (O, M_out) + tuple(g)

    check_replays(w, step, ["Q", "K", "V", "dO", "M_in", "dM_out"])


def test_gated_step_replays_in_a_graph():
    w = small("graph gated bf16 d64", "bf16", B=1, H=2, N=700, d=64, chunk=64, seed=500,
              gates="gla", m_in_scale=0.05, dm_out_scale=0.05)

    def step(x):
        O, M_out, cache = cca.fwd_gated(x["Q"], x["K"], x["V"], x["log_g"], 64, None, x["M_in"])
        g = cca.bwd_gated(x["Q"], x["K"], x["V"], x["log_g"], x["dO"], 64, None, x["M_in"],
                          x["dM_out"], cache)
        return (O, M_out) + tuple(g)

    check_replays(w, step, ["Q", "K", "V", "dO", "log_g", "M_in", "dM_out"])
