"""The allocation-free forward (lasp_fwd_noalloc) against lasp_fwd, through the
C ABI: same inputs, same kernels, so the outputs (O, M_out and the state cache)
must be identical, on two calls in a row (the second smaller, so stale scratch
from the first would show), with and without a state cache; and a call that
needs more scratch than the static array holds is refused before anything runs."""
import ctypes
import sys

import pytest
import torch

import chunked_causal_linear_amd as cca
from chunked_causal_linear_amd.workloads import make_inputs, small

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_both(w, with_cache):
    inp = make_inputs(w, device="cuda")
    Q, K, V = inp["Q"], inp["K"], inp["V"]
    decay, cu, M_in = inp["decay"], inp["cu_seqlens"], inp["M_in"]
    C = w.chunk
    ref_O, ref_M, ref_cache = cca.fwd(Q, K, V, C, decay, cu, M_in, want_state_cache=with_cache)
    O = torch.empty_like(Q)
    M_out = torch.empty_like(ref_M)
    cache = torch.empty_like(ref_cache) if with_cache else None
    torch.cuda.synchronize()
    cca.fwd_noalloc(Q, K, V, C, decay, cu, M_in, out=O, M_out=M_out, state_cache=cache)
    torch.cuda.synchronize()
    assert torch.equal(O, ref_O)
    assert torch.equal(M_out, ref_M)
    if with_cache:
        # the cache it wrote serves lasp_bwd exactly like lasp_fwd's (its raw
        # bytes are not compared: a packed batch's cache is sized for the most
        # segments any split could need, and the unused tail is never written)
        dO = inp["dO"]
        a = cca.bwd(Q, K, V, dO, C, decay, cu, M_in, inp["dM_out"], cache)
        b = cca.bwd(Q, K, V, dO, C, decay, cu, M_in, inp["dM_out"], ref_cache)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("with_cache", [True, False])
def test_noalloc_matches_fwd_twice(with_cache):
    big = small("bf16 B1 H32 N65536 d128 C256 M_in", "bf16", B=1, H=32, N=65536, d=128,
                chunk=256, seed=90, m_in_scale=0.01, dm_out_scale=0.01)
    little = small("bf16 packed d64 C128 decay", "bf16", H=4, d=64, chunk=128, seed=91,
                   lengths=[1, 300, 0, 1000, 129], decay="lightning", m_in_scale=0.1,
                   dm_out_scale=0.1)
    for w in (big, little):
        say("case: noalloc", w.name, "cache" if with_cache else "no cache")
        run_both(w, with_cache)


def test_noalloc_rejects_oversized_calls():
    """A shape whose scratch exceeds the static array: LASP_ESCRATCH, returned
    before the device is touched (the buffers below are never read or written)."""
    L = cca.lib()
    cap = L.lasp_noalloc_scratch_bytes()
    assert cap == 64 << 20
    x = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    p = ctypes.c_void_p(x.data_ptr())
    big = cca.Shape(1, 256, 1 << 22, 128, 256, 0)
    sz = cca.query_sizes(big, cca.LASP_BF16)
    assert sz.fwd_workspace[1] > cap
    rc = L.lasp_fwd_noalloc(ctypes.byref(big), cca.LASP_BF16, p, p, p, None, None, None, p,
                            None, p, None)
    assert rc == 5, rc
    assert b"static" in L.lasp_status_string(5)
