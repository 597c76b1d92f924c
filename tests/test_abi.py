"""C ABI contract, checked without a GPU: the library loads, exports every symbol
include/lasp.h declares, and rejects bad arguments before any HIP call (so fake,
never-dereferenced pointers are safe here)."""
import ctypes
import os
import re

import pytest

import chunked_causal_linear_amd as cca
from chunked_causal_linear_amd import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lasp.h")

OK, EINVAL, EUNSUP, EWS, EHIP = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(cca.LIB_PATH):
        from chunked_causal_linear_amd import build
        build.build()
    return cca.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lasp_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"lasp_fwd", "lasp_bwd", "lasp_state_cache_bytes", "lasp_status_string"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    for s in (OK, EINVAL, EUNSUP, EWS, EHIP, 99):
        assert isinstance(L.lasp_status_string(s), bytes)
    assert L.lasp_version() >= 100


A = 1 << 20        # fake, 16-byte aligned, never dereferenced device addresses
GAP = 1 << 36


def fake(i):
    return ctypes.c_void_p(A + i * GAP)


def fwd_call(L, shape, dtype=1, Q=0, K=1, V=2, decay=None, cu=None, M_in=None, O=3, M_out=None,
             cache=None, ws=5, ws_bytes=None, overrides=None):
    args = dict(Q=fake(Q) if Q is not None else None, K=fake(K) if K is not None else None,
                V=fake(V), decay=None if decay is None else fake(decay),
                cu=None if cu is None else fake(cu), M_in=None if M_in is None else fake(M_in),
                O=None if O is None else fake(O), M_out=None if M_out is None else fake(M_out),
                cache=None if cache is None else fake(cache), ws=None if ws is None else fake(ws))
    if overrides:
        args.update(overrides)
    if ws_bytes is None:
        ws_bytes = L.lasp_fwd_workspace_bytes(ctypes.byref(shape), dtype, int(cache is not None))
    return L.lasp_fwd(ctypes.byref(shape), dtype, args["Q"], args["K"], args["V"], args["decay"],
                      args["cu"], args["M_in"], args["O"], args["M_out"], args["cache"],
                      args["ws"], ws_bytes, None)


def test_fwd_rejects_bad_arguments(L):
    good = Shape(2, 4, 1000, 64, 128, 0)
    # dims
    for bad in [Shape(0, 4, 1000, 64, 128, 0), Shape(2, 0, 1000, 64, 128, 0),
                Shape(2, 4, 0, 64, 128, 0), Shape(2, 4, 1000, 64, 128, -1)]:
        assert fwd_call(L, bad) == EINVAL
    # unsupported d / chunk / dtype
    assert fwd_call(L, Shape(2, 4, 1000, 48, 128, 0)) == EUNSUP
    assert fwd_call(L, Shape(2, 4, 1000, 64, 100, 0)) == EUNSUP
    assert fwd_call(L, Shape(2, 4, 1000, 64, 32, 0)) == EUNSUP
    assert fwd_call(L, good, dtype=7) == EUNSUP
    # required pointers
    assert fwd_call(L, good, Q=None) == EINVAL
    assert fwd_call(L, good, O=None) == EINVAL
    # packed batch needs B == 1 and cu_seqlens; cu_seqlens needs nseq > 0
    assert fwd_call(L, Shape(2, 4, 1000, 64, 128, 3), cu=6) == EINVAL
    assert fwd_call(L, Shape(1, 4, 1000, 64, 128, 3)) == EINVAL
    assert fwd_call(L, good, cu=6) == EINVAL
    # alignment
    assert fwd_call(L, good, overrides=dict(Q=ctypes.c_void_p(A + 8))) == EINVAL
    assert fwd_call(L, good, overrides=dict(decay=ctypes.c_void_p(A + 7 * GAP + 2))) == EINVAL
    # workspace
    need = L.lasp_fwd_workspace_bytes(ctypes.byref(good), 1, 0)
    assert need > 0
    assert fwd_call(L, good, ws_bytes=need - 1) == EWS
    assert fwd_call(L, good, ws=None) == EWS
    # outputs overlapping inputs
    assert fwd_call(L, good, O=0) == EINVAL
    assert fwd_call(L, good, overrides=dict(O=ctypes.c_void_p(A + 2 * GAP + 4096))) == EINVAL
    assert fwd_call(L, good, M_out=3) == EINVAL            # M_out inside O
    assert fwd_call(L, good, ws=2) == EINVAL               # workspace inside V


def test_bwd_rejects_bad_arguments(L):
    s = Shape(1, 2, 300, 32, 64, 0)
    need = L.lasp_bwd_workspace_bytes(ctypes.byref(s), 0, 0)
    p = [fake(i) for i in range(12)]

    def call(shape=s, dt=0, ws_bytes=need, **kw):
        a = dict(Q=p[0], K=p[1], V=p[2], dO=p[3], decay=None, cu=None, M_in=None, dM_out=None,
                 cache=None, dQ=p[4], dK=p[5], dV=p[6], dM_in=None, ws=p[7])
        a.update(kw)
        return L.lasp_bwd(ctypes.byref(shape), dt, a["Q"], a["K"], a["V"], a["dO"], a["decay"],
                          a["cu"], a["M_in"], a["dM_out"], a["cache"], a["dQ"], a["dK"], a["dV"],
                          a["dM_in"], a["ws"], ws_bytes, None)

    assert call(dO=None) == EINVAL
    assert call(dK=None) == EINVAL
    assert call(shape=Shape(1, 2, 300, 256, 64, 0)) == EUNSUP
    assert call(ws_bytes=need - 256) == EWS
    assert call(dQ=p[3]) == EINVAL                 # dQ aliases dO
    assert call(dV=p[5]) == EINVAL                 # two outputs alias
    assert call(dM_in=ctypes.c_void_p(A + 4)) == EINVAL   # misaligned
    # with a state cache the workspace may be smaller
    assert L.lasp_bwd_workspace_bytes(ctypes.byref(s), 0, 1) < need


def test_sizes_follow_the_shape(L):
    # bf16: the state cache holds one float32 state per (segment, head); the
    # per-chunk states are recomputed inside the segment sweep
    c3 = Shape(1, 32, 131072, 128, 256, 0)
    n = L.lasp_state_cache_bytes(ctypes.byref(c3), 1)
    chunks = 131072 // 256
    assert 32 * 128 * 128 * 4 <= n <= chunks * 32 * 128 * 128 * 4 // 2
    # float32: per-chunk local states (float32) + per-segment states
    n32 = L.lasp_state_cache_bytes(ctypes.byref(c3), 0)
    assert chunks * 32 * 128 * 128 * 4 <= n32 <= chunks * 32 * 128 * 128 * 4 * 1.5
    # packed batch bounds cover any split of N into nseq sequences
    pk = Shape(1, 8, 5000, 64, 128, 7)
    assert L.lasp_state_cache_bytes(ctypes.byref(pk), 0) >= (5000 // 128 + 7) * 8 * 64 * 64 * 4
    # invalid shapes report 0
    assert L.lasp_state_cache_bytes(ctypes.byref(Shape(1, 1, 1, 33, 64, 0)), 1) == 0
    assert L.lasp_fwd_workspace_bytes(None, 1, 0) == 0


def test_bidir_rejects_bad_arguments(L):
    """The unmasked entry points share the checks of lasp_fwd / lasp_bwd (every
    case here fails before anything is enqueued)."""
    s = Shape(1, 2, 300, 64, 128, 0)
    p = [fake(i) for i in range(12)]
    nf = L.lasp_fwd_workspace_bytes(ctypes.byref(s), 1, 0)
    nb = L.lasp_bwd_workspace_bytes(ctypes.byref(s), 1, 0)

    def fwd(shape=s, dt=1, ws_bytes=nf, **kw):
        a = dict(Q=p[0], K=p[1], V=p[2], cu=None, M_in=None, O=p[3], M_out=None, cache=None, ws=p[5])
        a.update(kw)
        return L.lasp_fwd_bidir(ctypes.byref(shape), dt, a["Q"], a["K"], a["V"], a["cu"], a["M_in"],
                                a["O"], a["M_out"], a["cache"], a["ws"], ws_bytes, None)

    def bwd(shape=s, dt=1, ws_bytes=nb, **kw):
        a = dict(Q=p[0], K=p[1], V=p[2], dO=p[3], cu=None, M_in=None, dM_out=None, cache=None,
                 dQ=p[4], dK=p[5], dV=p[6], dM_in=None, ws=p[7])
        a.update(kw)
        return L.lasp_bwd_bidir(ctypes.byref(shape), dt, a["Q"], a["K"], a["V"], a["dO"], a["cu"],
                                a["M_in"], a["dM_out"], a["cache"], a["dQ"], a["dK"], a["dV"],
                                a["dM_in"], a["ws"], ws_bytes, None)

    assert fwd(dt=2) == EUNSUP and bwd(dt=2) == EUNSUP          # no such dtype
    assert fwd(shape=Shape(1, 2, 300, 48, 128, 0)) == EUNSUP
    assert fwd(O=None) == EINVAL and bwd(dV=None) == EINVAL
    assert fwd(O=p[1]) == EINVAL and bwd(dK=p[0]) == EINVAL    # output aliases an input
    assert fwd(ws_bytes=nf - 1) == EWS and bwd(ws_bytes=nb - 1) == EWS
    assert fwd(cu=p[8]) == EINVAL                               # cu_seqlens without nseq


def test_gated_rejects_bad_arguments(L):
    """The gated entry points: chunks of 64 tokens whatever supported length the
    shape names (sizes equal for 64, 128, 256), log_g (and dlog_g) required,
    aligned and disjoint from the outputs."""
    s = Shape(1, 2, 300, 64, 64, 0)
    p = [fake(i) for i in range(14)]
    nf = L.lasp_gated_fwd_workspace_bytes(ctypes.byref(s), 1, 0)
    nb = L.lasp_gated_bwd_workspace_bytes(ctypes.byref(s), 1, 0)
    assert nf > 0 and nb > 0

    def fwd(shape=s, dt=1, ws_bytes=nf, **kw):
        a = dict(Q=p[0], K=p[1], V=p[2], LG=p[9], cu=None, M_in=None, O=p[3], M_out=None,
                 cache=None, ws=p[5])
        a.update(kw)
        return L.lasp_fwd_gated(ctypes.byref(shape), dt, a["Q"], a["K"], a["V"], a["LG"], a["cu"],
                                a["M_in"], a["O"], a["M_out"], a["cache"], a["ws"], ws_bytes, None)

    def bwd(shape=s, dt=1, ws_bytes=nb, **kw):
        a = dict(Q=p[0], K=p[1], V=p[2], LG=p[9], dO=p[3], cu=None, M_in=None, dM_out=None,
                 cache=None, dQ=p[4], dK=p[5], dV=p[6], dLG=p[10], dM_in=None, ws=p[7])
        a.update(kw)
        return L.lasp_bwd_gated(ctypes.byref(shape), dt, a["Q"], a["K"], a["V"], a["LG"], a["dO"],
                                a["cu"], a["M_in"], a["dM_out"], a["cache"], a["dQ"], a["dK"],
                                a["dV"], a["dLG"], a["dM_in"], a["ws"], ws_bytes, None)

    for c in (128, 256):
        sc = Shape(1, 2, 300, 64, c, 0)
        for dt in (0, 1):
            for q in (L.lasp_gated_state_cache_bytes,):
                assert q(ctypes.byref(sc), dt) == q(ctypes.byref(s), dt)
            for q in (L.lasp_gated_fwd_workspace_bytes, L.lasp_gated_bwd_workspace_bytes):
                assert q(ctypes.byref(sc), dt, 0) == q(ctypes.byref(s), dt, 0)
                assert q(ctypes.byref(sc), dt, 1) == q(ctypes.byref(s), dt, 1)
    for c in (32, 96, 512):
        assert fwd(shape=Shape(1, 2, 300, 64, c, 0)) == EUNSUP
        assert bwd(shape=Shape(1, 2, 300, 64, c, 0)) == EUNSUP
    assert fwd(shape=Shape(1, 2, 300, 48, 64, 0)) == EUNSUP
    for dt in (0, 1):
        assert L.lasp_gated_state_cache_bytes(ctypes.byref(Shape(1, 2, 300, 128, 64, 0)), dt) > 0
    assert fwd(LG=None) == EINVAL and bwd(LG=None) == EINVAL and bwd(dLG=None) == EINVAL
    assert fwd(LG=ctypes.c_void_p(A + 9 * GAP + 4)) == EINVAL        # misaligned log_g
    assert fwd(O=p[9]) == EINVAL                                      # O aliases log_g
    assert bwd(dLG=p[9]) == EINVAL and bwd(dLG=p[4]) == EINVAL       # dlog_g aliases
    assert fwd(ws_bytes=nf - 1) == EWS and bwd(ws_bytes=nb - 1) == EWS
    assert fwd(cu=p[8]) == EINVAL
    # the gated state cache: the segments' entering states, each sequence's
    # final state and the segments' gate products (float32), no per-chunk
    # states (B1 H2 N300 d64: 5 chunks of 64, one chunk per segment)
    def al(n):
        return (n + 255) // 256 * 256
    for dt in (0, 1):
        assert (L.lasp_gated_state_cache_bytes(ctypes.byref(s), dt)
                == al(5 * 2 * 64 * 64 * 4) + al(2 * 64 * 64 * 4) + al(5 * 2 * 64 * 4))


SHAPES = [Shape(1, 32, 131072, 128, 256, 0), Shape(4, 16, 8192, 128, 256, 0),
          Shape(2, 16, 32768, 128, 256, 0), Shape(1, 32, 69632, 64, 128, 8),
          Shape(1, 2, 256, 32, 64, 0), Shape(3, 5, 1000, 64, 128, 0), Shape(1, 4, 777, 32, 64, 5)]


def all_sizes(L, s, dt, form):
    if form == 1:
        return (L.lasp_gated_state_cache_bytes(ctypes.byref(s), dt),
                L.lasp_gated_fwd_workspace_bytes(ctypes.byref(s), dt, 0),
                L.lasp_gated_fwd_workspace_bytes(ctypes.byref(s), dt, 1),
                L.lasp_gated_bwd_workspace_bytes(ctypes.byref(s), dt, 0),
                L.lasp_gated_bwd_workspace_bytes(ctypes.byref(s), dt, 1))
    return (L.lasp_state_cache_bytes(ctypes.byref(s), dt),
            L.lasp_fwd_workspace_bytes(ctypes.byref(s), dt, 0),
            L.lasp_fwd_workspace_bytes(ctypes.byref(s), dt, 1),
            L.lasp_bwd_workspace_bytes(ctypes.byref(s), dt, 0),
            L.lasp_bwd_workspace_bytes(ctypes.byref(s), dt, 1))


def test_sizes_do_not_depend_on_the_environment(L, monkeypatch):
    """The state-cache layout (and so every size) is a pure function of the
    call's arguments: environment variables, including the names a segment
    override or a debug switch might use, change nothing."""
    cases = [(s, dt, form) for s in SHAPES for dt in (0, 1) for form in (0, 1)
             if form == 0 or s.chunk == 64]
    before = [all_sizes(L, *c) for c in cases]
    for k, v in (("LASP_SEGMENT_CHUNKS", "3"), ("LASP_DEBUG", "1"), ("LASP_G", "7"),
                 ("HIP_VISIBLE_DEVICES", "0")):
        monkeypatch.setenv(k, v)
    after = [all_sizes(L, *c) for c in cases]
    assert before == after


def test_segment_length_of_the_benchmark_shapes(L):
    """The library's segment lengths at the benchmark-sized shapes: every
    segment sweep of a launch in one round of 256 workgroups where the
    sequences allow it (config 3: 8 segments of 64 chunks per head)."""
    bf16 = 1
    assert cca.query_sizes(Shape(1, 32, 131072, 128, 256, 0), bf16).segment_chunks == 64
    assert cca.query_sizes(Shape(4, 16, 8192, 128, 256, 0), bf16).segment_chunks == 8
    assert cca.query_sizes(Shape(2, 16, 32768, 128, 256, 0), bf16).segment_chunks == 16


def test_query_sizes_agrees_with_the_plain_queries(L):
    """lasp_query_sizes with segment_chunks = 0 reports what the plain size
    queries report (the forward and backward use one plan), and an explicit
    segment length changes the layout consistently for both directions."""
    for s in SHAPES:
        for dt in (0, 1):
            for form in ((0, 1) if s.chunk == 64 else (0,)):
                q = cca.query_sizes(s, dt, form, 0)
                assert (q.state_cache, q.fwd_workspace[0], q.fwd_workspace[1], q.bwd_workspace[0],
                        q.bwd_workspace[1]) == all_sizes(L, s, dt, form)
                assert q.segment_chunks >= 1
                for G in (1, 2, 3, 16):
                    g = cca.query_sizes(s, dt, form, G)
                    assert g.segment_chunks == G
                    # without a cache buffer, each workspace holds the whole cache
                    assert g.fwd_workspace[0] - g.fwd_workspace[1] == g.state_cache
                    assert g.bwd_workspace[0] - g.bwd_workspace[1] >= g.state_cache
    out = cca.Sizes()
    assert L.lasp_query_sizes(ctypes.byref(SHAPES[0]), 1, 0, -1, ctypes.byref(out)) == EINVAL
    assert L.lasp_query_sizes(ctypes.byref(SHAPES[0]), 1, 3, 0, ctypes.byref(out)) == EINVAL
    assert L.lasp_query_sizes(ctypes.byref(SHAPES[0]), 1, 2, 4, ctypes.byref(out)) == EINVAL
    # the normalised form: the causal sizes, plus one token array in the backward
    for s in SHAPES:
        for dt in (0, 1):
            a, b = cca.query_sizes(s, dt, 0), cca.query_sizes(s, dt, 2)
            tens = s.B * s.H * s.N * s.d * (2 if dt else 4)
            assert a.state_cache == b.state_cache and list(a.fwd_workspace) == list(b.fwd_workspace)
            for i in (0, 1):
                assert tens <= b.bwd_workspace[i] - a.bwd_workspace[i] < tens + 256
    assert L.lasp_query_sizes(ctypes.byref(SHAPES[0]), 1, 0, 0, None) == EINVAL
    assert L.lasp_query_sizes(ctypes.byref(Shape(1, 1, 8, 48, 64, 0)), 1, 0, 0,
                              ctypes.byref(out)) == EUNSUP


def test_binding_rejects_bad_out_and_host_tensors():
    """The binding validates a preallocated O / dQ, dK, dV like every other
    tensor (so a wrong buffer never reaches the kernels), and refuses host
    tensors outright."""
    import torch
    q = torch.zeros(1, 2, 64, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cca.fwd(q, q, q, 64)                                  # host tensors
    meta = torch.device("meta")
    qm = torch.empty(1, 2, 64, 32, dtype=torch.bfloat16, device=meta)
    with pytest.raises(ValueError):
        cca.fwd(qm, qm, qm, 64)


def _no_gpu_here():
    if os.path.exists("/dev/kfd"):
        return False
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu_here(), reason="needs a host without a GPU (fake pointers)")
def test_validated_call_without_a_gpu_reports_ehip(L):
    """A call whose arguments pass every check reaches the first launch; on a
    host without a GPU that launch fails and the call returns LASP_EHIP with
    the HIP error text, without raising or crashing."""
    s = Shape(1, 2, 300, 64, 64, 0)
    assert fwd_call(L, s) == EHIP
    msg = L.lasp_status_string(EHIP)
    assert isinstance(msg, bytes) and len(msg) > 0


def declared_arity():
    """Number of parameters of every function include/lasp.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(lasp_\w+)\s*\(([^;{]*?)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def test_binding_signatures_match_the_header(L):
    """Every function the binding gives argtypes to takes as many arguments as
    include/lasp.h declares (a miscounted ctypes signature would pass pointers
    in the wrong slots)."""
    arity = declared_arity()
    checked = 0
    for name, n in arity.items():
        f = getattr(L, name)
        if f.argtypes is not None:
            assert len(f.argtypes) == n, (name, len(f.argtypes), n)
            checked += 1
    assert checked >= 20


def test_autograd_wrappers_reject_host_tensors():
    """The autograd wrappers go through the same argument checks: host tensors
    are refused before the library is touched."""
    import torch
    from chunked_causal_linear_amd.autograd import (lasp_attention, lasp_bidir_attention,
                                                    lasp_gated_attention)
    Q = torch.zeros(1, 1, 64, 32)
    with pytest.raises(ValueError, match="GPU"):
        lasp_attention(Q, Q, Q, 64)
    with pytest.raises(ValueError, match="GPU"):
        lasp_bidir_attention(Q, Q, Q, 64)
    with pytest.raises(ValueError, match="GPU"):
        lasp_gated_attention(Q, Q, Q, Q, 64)
