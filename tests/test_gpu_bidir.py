"""GPU parity of the unmasked (bidirectional) form: lasp_fwd_bidir /
lasp_bwd_bidir through the C ABI against the oracle's bidir_* functions
("Linear Attention Sequence Parallelism", Eq. 3 without Norm; LASP-2's sum of
all chunk states).  Same metric and bar as the causal parity tests:
max|gpu - ref| / max|ref| per tensor <= 2e-2 for bf16 inputs, 1e-4 for
float32 inputs."""
import numpy as np
import pytest
import torch

import chunked_causal_linear_amd as cca
from chunked_causal_linear_amd.workloads import CONFIGS, make_inputs, small
from oracle import lasp_oracle as lo
from test_gpu_parity import TOL, check, dev, np64, rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    cca.lib()       # raises if the HIP library is missing: no fallback
    yield


def run_bidir(inp, use_cache=True, seg=0):
    sh = inp["shape"]
    Q, K, V = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"])
    cu, M_in = dev(inp["cu_seqlens"]), dev(inp["M_in"])
    O, M_out, cache = cca.fwd_bidir(Q, K, V, sh["chunk"], cu, M_in, want_state_cache=use_cache,
                                    segment_chunks=seg)
    dQ, dK, dV, dM_in = cca.bwd_bidir(Q, K, V, dev(inp["dO"]), sh["chunk"], cu, M_in,
                                      dev(inp["dM_out"]), cache, segment_chunks=seg)
    torch.cuda.synchronize()
    return dict(O=O, M_out=M_out, dQ=dQ, dK=dK, dV=dV, dM_in=dM_in)


def oracle_bidir(inp):
    a = {k: np64(inp[k]) for k in ("Q", "K", "V", "dO", "M_in", "dM_out")}
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy()
    O, Mo = lo.batched_bidir_fwd(a["Q"], a["K"], a["V"], a["M_in"], cu)
    dQ, dK, dV, dMi = lo.batched_bidir_bwd(a["Q"], a["K"], a["V"], a["dO"], a["M_in"], a["dM_out"], cu)
    return dict(O=O, M_out=Mo, dQ=dQ, dK=dK, dV=dV, dM_in=dMi)


SMALL = [
    small("bidir bf16 d64 C64 B2 H2 Min dMout", "bf16", B=2, H=2, N=300, d=64, chunk=64, seed=50,
          m_in_scale=0.1, dm_out_scale=0.1),
    small("bidir bf16 d128 C256 ragged", "bf16", B=1, H=2, N=700, d=128, chunk=256, seed=51),
    small("bidir bf16 d32 C64 B3 H1 Min dMout", "bf16", B=3, H=1, N=200, d=32, chunk=64, seed=52,
          m_in_scale=0.1, dm_out_scale=0.1),
    small("bidir bf16 packed d128 C128 edge lengths", "bf16", H=2, d=128, chunk=128, seed=53,
          lengths=[1, 127, 128, 129, 0, 300, 64, 1000], m_in_scale=0.1, dm_out_scale=0.1),
    small("bidir bf16 one token", "bf16", B=1, H=1, N=1, d=64, chunk=64, seed=54, m_in_scale=0.1,
          dm_out_scale=0.1),
    # float32: the same products in float32 MFMAs, bar 1e-4
    small("bidir fp32 d32 C64 B2 H2 Min dMout", "fp32", B=2, H=2, N=300, d=32, chunk=64, seed=57,
          m_in_scale=0.1, dm_out_scale=0.1),
    small("bidir fp32 d64 C128 ragged", "fp32", B=1, H=3, N=700, d=64, chunk=128, seed=58),
    small("bidir fp32 d128 C256 ragged Min dMout", "fp32", B=1, H=2, N=600, d=128, chunk=256, seed=59,
          m_in_scale=0.1, dm_out_scale=0.1),
    small("bidir fp32 packed d128 C64 edge lengths", "fp32", H=2, d=128, chunk=64, seed=60,
          lengths=[1, 63, 64, 65, 0, 300, 1000], m_in_scale=0.1, dm_out_scale=0.1),
    small("bidir fp32 one token", "fp32", B=1, H=1, N=1, d=128, chunk=128, seed=61, m_in_scale=0.1,
          dm_out_scale=0.1),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_bidir_small(w):
    say("case:", w.name)
    inp = make_inputs(w)
    check(w.name, run_bidir(inp), oracle_bidir(inp), TOL[w.dtype])


# Every (dtype, d, chunk) the unmasked entry points accept (no decay): the
# kernels are compiled per d; the chunk sets the segments the totals and the
# row-block products work on.  Four chunks and a ragged tail in segments of two
# chunks; M_in and dM_out on.
MATRIX = [(dt, d, C) for dt in ("bf16", "fp32") for d in (32, 64, 128) for C in (64, 128, 256)]


@pytest.mark.parametrize("dt,d,C", MATRIX, ids=["%s-d%d-C%d" % m for m in MATRIX])
def test_bidir_every_accepted_configuration(dt, d, C):
    w = small("bidir %s d%d C%d" % (dt, d, C), dt, B=1, H=2, N=3 * C + C // 2 + 7, d=d, chunk=C,
              seed=3000 + d + C + (dt == "fp32") * 7, m_in_scale=0.1, dm_out_scale=0.1)
    say("case:", w.name)
    inp = make_inputs(w)
    check(w.name, run_bidir(inp, seg=2), oracle_bidir(inp), TOL[dt])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("G", [1, 3])
def test_bidir_segment_sizes(G, dtype):
    w = small("bidir %s d64 C64 many chunks" % dtype, dtype, B=2, H=2, N=64 * 11 + 17, d=64, chunk=64,
              seed=55, m_in_scale=0.1, dm_out_scale=0.1)
    say("case: bidir segment chunks", G, dtype)
    inp = make_inputs(w)
    check("bidir %s G=%d" % (dtype, G), run_bidir(inp, seg=G), oracle_bidir(inp), TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bidir_recompute_equals_cache(dtype):
    w = small("bidir %s d128 C128" % dtype, dtype, B=1, H=2, N=900, d=128, chunk=128, seed=56,
              m_in_scale=0.1, dm_out_scale=0.1)
    inp = make_inputs(w)
    say("case: bidir recompute vs cache", dtype)
    a = run_bidir(inp, use_cache=True)
    b = run_bidir(inp, use_cache=False)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_bidir_full_size_sampled():
    """bf16 B1 H32 N131072 d128 (the benchmark's shape, with M_in and dM_out):
    sampled rows of O, dQ, dK, dV as direct sums over all tokens, full M_out and
    dM_in, one head at a time."""
    import dataclasses
    w = dataclasses.replace(CONFIGS[3], name="bidir " + CONFIGS[3].name, dm_out_scale=0.01, seed=58)
    say("case:", w.name)
    inp = make_inputs(w)
    out = run_bidir(inp)
    r = np.random.default_rng(158)
    L = w.N
    rows = np.unique(np.concatenate([[0, L - 1], r.integers(0, L, 32)]))
    idx = torch.as_tensor(rows)
    acc = {k: ([], []) for k in ("O", "dQ", "dK", "dV", "M_out", "dM_in")}
    for h in range(w.H):
        q, k, v, do = (np64(inp[x][0, h]) for x in ("Q", "K", "V", "dO"))
        ref = lo.bidir_sampled(q, k, v, do, rows, np64(inp["M_in"][0, h]), np64(inp["dM_out"][0, h]))
        for name in ("O", "dQ", "dK", "dV"):
            acc[name][0].append(np64(out[name][0, h].index_select(0, idx.to(out[name].device))))
            acc[name][1].append(ref[name])
        acc["M_out"][0].append(np64(out["M_out"][0, h]))
        acc["M_out"][1].append(ref["M_out"])
        acc["dM_in"][0].append(np64(out["dM_in"][0, h]))
        acc["dM_in"][1].append(ref["dM_in"])
    errs = {k: rel(np.concatenate(g), np.concatenate(rv)) for k, (g, rv) in acc.items()}
    say(w.name, " ".join("%s=%.2e" % kv for kv in errs.items()))
    bad = {k: e for k, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad
