"""GPU parity of the gated form: lasp_fwd_gated / lasp_bwd_gated through the C
ABI against the oracle's gated recurrence ("Linear Attention Sequence
Parallelism", Appendix A.4, Eq. 24 with the GLA / GateLoop row of Table 5).
Metric: max|gpu - ref| / max|ref| per tensor, <= 1e-4 for float32 inputs and
<= 2e-2 for bf16 inputs (the same bar as the causal parity tests).  Gate
recipes: "gla" (every diagonal tile takes the factorised MFMA products),
"strong" (every diagonal tile is summed pair by pair), "mixed" (both)."""
import dataclasses

import numpy as np
import pytest
import torch

import chunked_causal_linear_amd as cca
from chunked_causal_linear_amd.workloads import GATED, make_inputs, small
from oracle import gated_oracle as go
from test_gpu_parity import TOL, check, dev, np64, rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cca.lib()       # raises if the HIP library is missing: no fallback
    yield


def run_gated(inp, use_cache=True, seg=0):
    sh = inp["shape"]
    Q, K, V, LG = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(inp["log_g"])
    cu, M_in = dev(inp["cu_seqlens"]), dev(inp["M_in"])
    O, M_out, cache = cca.fwd_gated(Q, K, V, LG, sh["chunk"], cu, M_in, want_state_cache=use_cache,
                                    segment_chunks=seg)
    dQ, dK, dV, dLG, dM_in = cca.bwd_gated(Q, K, V, LG, dev(inp["dO"]), sh["chunk"], cu, M_in,
                                           dev(inp["dM_out"]), cache, segment_chunks=seg)
    torch.cuda.synchronize()
    return dict(O=O, M_out=M_out, dQ=dQ, dK=dK, dV=dV, dLG=dLG, dM_in=dM_in)


def oracle_gated(inp):
    a = {k: np64(inp[k]) for k in ("Q", "K", "V", "dO", "log_g", "M_in", "dM_out")}
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    O, Mo = go.batched_gated_fwd(a["Q"], a["K"], a["V"], a["log_g"], a["M_in"], cu)
    dQ, dK, dV, dLG, dMi = go.batched_gated_bwd(a["Q"], a["K"], a["V"], a["log_g"], a["dO"],
                                                a["M_in"], a["dM_out"], cu)
    return dict(O=O, M_out=Mo, dQ=dQ, dK=dK, dV=dV, dLG=dLG, dM_in=dMi)


SMALL = [
    small("gated fp32 d32 B2 H2 gla Min dMout ragged", "fp32", B=2, H=2, N=300, d=32, seed=60,
          gates="gla", m_in_scale=0.1, dm_out_scale=0.1),
    small("gated fp32 d64 strong Min dMout", "fp32", B=1, H=2, N=200, d=64, seed=61,
          gates="strong", m_in_scale=0.1, dm_out_scale=0.1),
    small("gated fp32 d64 mixed", "fp32", B=1, H=1, N=333, d=64, seed=62, gates="mixed"),
    small("gated bf16 d64 B2 H2 gla", "bf16", B=2, H=2, N=300, d=64, seed=63, gates="gla"),
    small("gated bf16 d128 mixed Min dMout", "bf16", B=1, H=2, N=700, d=128, seed=64,
          gates="mixed", m_in_scale=0.1, dm_out_scale=0.1),
    small("gated bf16 d128 strong", "bf16", B=1, H=1, N=257, d=128, seed=65, gates="strong"),
    small("gated bf16 d32 B3 gla Min dMout", "bf16", B=3, H=1, N=150, d=32, seed=66, gates="gla",
          m_in_scale=0.1, dm_out_scale=0.1),
    small("gated bf16 packed d64 edge lengths", "bf16", H=2, d=64, seed=67, gates="mixed",
          lengths=[1, 63, 64, 65, 0, 200, 33, 128], m_in_scale=0.1, dm_out_scale=0.1),
    small("gated fp32 packed d32 edge lengths", "fp32", H=2, d=32, seed=68, gates="gla",
          lengths=[0, 1, 64, 127, 31, 2], m_in_scale=0.1, dm_out_scale=0.1),
    small("gated bf16 one token", "bf16", B=1, H=1, N=1, d=64, seed=69, gates="gla",
          m_in_scale=0.1, dm_out_scale=0.1),
    small("gated fp32 d128 mixed Min dMout", "fp32", B=1, H=2, N=333, d=128, seed=73,
          gates="mixed", m_in_scale=0.1, dm_out_scale=0.1),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_gated_small(w):
    say("case:", w.name)
    inp = make_inputs(w)
    check(w.name, run_gated(inp), oracle_gated(inp), TOL[w.dtype])


@pytest.mark.parametrize("G", [1, 3])
def test_gated_segment_sizes(G):
    w = small("gated fp32 d32 many chunks", "fp32", B=2, H=2, N=64 * 11 + 17, d=32, seed=70,
              gates="mixed", m_in_scale=0.1, dm_out_scale=0.1)
    say("case: gated segment chunks", G)
    inp = make_inputs(w)
    check("gated G=%d" % G, run_gated(inp, seg=G), oracle_gated(inp), TOL["fp32"])


def test_gated_medium_multi_segment():
    """bf16 B2 H4 N4096 d128 (64 chunks per sequence) in segments of 8 chunks,
    every element against the oracle's recurrence."""
    w = small("gated bf16 d128 B2 H4 N4096 G8", "bf16", B=2, H=4, N=4096, d=128, seed=76,
              gates="mixed", m_in_scale=0.05, dm_out_scale=0.05)
    say("case:", w.name)
    inp = make_inputs(w)
    check(w.name, run_gated(inp, seg=8), oracle_gated(inp), TOL["bf16"])


CKPT = [
    (16, small("gated fp32 d64 41 chunks Min dMout", "fp32", B=1, H=2, N=64 * 40 + 13, d=64, seed=80,
               gates="mixed", m_in_scale=0.1, dm_out_scale=0.1)),
    (17, small("gated bf16 d128 41 chunks Min dMout", "bf16", B=1, H=2, N=64 * 40 + 13, d=128, seed=81,
               gates="gla", m_in_scale=0.1, dm_out_scale=0.1)),
    (9, small("gated bf16 packed d64", "bf16", H=2, d=64, seed=82, gates="mixed",
              lengths=[700, 1100, 64 * 8, 1], m_in_scale=0.1, dm_out_scale=0.1)),
]


@pytest.mark.parametrize("G,w", CKPT, ids=["G%d %s" % (g, w.name) for g, w in CKPT])
def test_gated_checkpointed_segments(G, w):
    """Segments long enough to hold forward-state checkpoints (every 8 chunks
    inside a segment), where the reverse walk resets its log-gate gradient
    carry: G = 16 puts the second one on the segment end (none kept there),
    G = 17 keeps two per full segment and none in the short last one, G = 9
    one per full segment of a packed batch.  Every element against the
    oracle."""
    say("case:", w.name, "G", G)
    inp = make_inputs(w)
    check("%s G=%d" % (w.name, G), run_gated(inp, seg=G), oracle_gated(inp), TOL[w.dtype])


def test_gated_recompute_equals_cache():
    w = small("gated bf16 d128", "bf16", B=1, H=2, N=900, d=128, seed=71, gates="gla",
              m_in_scale=0.1, dm_out_scale=0.1)
    inp = make_inputs(w)
    say("case: gated recompute vs cache")
    a = run_gated(inp, use_cache=True)
    b = run_gated(inp, use_cache=False)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_constant_gates_match_the_decayed_path():
    """log g = log(lambda_h) everywhere: the gated kernels and the decayed ones
    (lasp_fwd / lasp_bwd with decay) compute the same map."""
    w = small("gated fp32 d64 constant", "fp32", B=1, H=2, N=500, d=64, seed=72,
              m_in_scale=0.1, dm_out_scale=0.1)
    inp = make_inputs(w)
    lam = torch.tensor([0.97, 0.8])
    inp["log_g"] = torch.log(lam)[None, :, None, None].expand(1, 2, 500, 64).contiguous()
    say("case: constant gates vs decay")
    g = run_gated(inp)
    Q, K, V, dO = (dev(inp[x]) for x in ("Q", "K", "V", "dO"))
    O, M_out, cache = cca.fwd(Q, K, V, 64, dev(lam), None, dev(inp["M_in"]))
    dQ, dK, dV, dM_in = cca.bwd(Q, K, V, dO, 64, dev(lam), None, dev(inp["M_in"]),
                                dev(inp["dM_out"]), cache)
    ref = dict(O=O, M_out=M_out, dQ=dQ, dK=dK, dV=dV, dM_in=dM_in)
    errs = {k: rel(np64(g[k]), np64(ref[k])) for k in ref}
    say(" ".join("%s=%.2e" % kv for kv in errs.items()))
    assert all(e <= TOL["fp32"] for e in errs.values()), errs


def test_gated_rejects_bad_configurations():
    inp = make_inputs(small("bf16 C96", "bf16", B=1, H=1, N=64, d=64, seed=74, gates="gla"))
    with pytest.raises(cca.LaspError) as e:
        cca.fwd_gated(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(inp["log_g"]), 96)
    assert e.value.status == 2


@pytest.mark.parametrize("chunk", [128, 256])
def test_gated_other_chunk_lengths_equal_64(chunk):
    """The gated kernels work on 64-token chunks whatever supported length the
    call names: chunk 128 and 256 give the bits of chunk 64 (and so the oracle's
    values at the parity bar)."""
    import dataclasses
    w = small("gated bf16 d64 ragged Min dMout", "bf16", B=2, H=2, N=300, d=64, chunk=64, seed=75,
              gates="mixed", m_in_scale=0.1, dm_out_scale=0.1)
    inp = make_inputs(w)
    say("case: gated chunk", chunk)
    a = run_gated(inp)
    inp_c = dict(inp, shape=dict(inp["shape"], chunk=chunk))
    b = run_gated(inp_c)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    check("gated chunk %d" % chunk, b, oracle_gated(inp), TOL["bf16"])


def test_gated_full_size_sampled():
    """bf16 B1 H32 N131072 d128 C64 with GLA gates, M_in and dM_out (the
    benchmark's gated workload): on every one of the 32 heads, sampled rows of
    O, dQ, dK, dV and dlog_g and the full M_out and dM_in, against the
    oracle's prefix / suffix sums (gated_sampled_sweep)."""
    w = dataclasses.replace(GATED, dm_out_scale=0.01, seed=75)
    say("case:", w.name)
    inp = make_inputs(w)
    out = run_gated(inp)
    r = np.random.default_rng(175)
    L = w.N
    names = ("O", "dQ", "dK", "dV", "dLG")
    acc = {k: ([], []) for k in names + ("M_out", "dM_in")}
    for h in range(w.H):
        rows = np.unique(np.concatenate([[0, 1, 63, 64, L - 65, L - 1], r.integers(0, L, 10)]))
        idx = torch.as_tensor(rows)
        q, k, v, lg, do = (np64(inp[x][0, h]) for x in ("Q", "K", "V", "log_g", "dO"))
        mi, dmo = np64(inp["M_in"][0, h]), np64(inp["dM_out"][0, h])
        ref, mo, dmi = go.gated_sampled_sweep(q, k, v, lg, do, rows, mi, dmo)
        for name in names:
            acc[name][0].append(np64(out[name][0, h].index_select(0, idx.to(out[name].device))))
            acc[name][1].append(ref[name])
        acc["M_out"][0].append(np64(out["M_out"][0, h]))
        acc["M_out"][1].append(mo)
        acc["dM_in"][0].append(np64(out["dM_in"][0, h]))
        acc["dM_in"][1].append(dmi)
        if h % 8 == 7:
            say("  heads checked:", h + 1)
    errs = {k: rel(np.concatenate(g), np.concatenate(rv)) for k, (g, rv) in acc.items()}
    say(w.name, " ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {k: e for k, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad
