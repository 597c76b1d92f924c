"""ctypes driver for oracle/crecurrent.c (float64 token recurrence, OpenMP).

TEST INFRASTRUCTURE ONLY.  Built with gcc into oracle/_crecurrent.so.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "crecurrent.c")
_LIB = os.path.join(_HERE, "_crecurrent.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle (gcc -O3 -fopenmp).  Returns the library path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v2", "-fopenmp", "-shared",
                               "-fPIC", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.lasp_ref_run.argtypes = [ctypes.c_int, P, P, P, ctypes.c_int,
                                     P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.lasp_ref_run.restype = ctypes.c_int
        lib.lasp_ref_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    return int(_load().lasp_ref_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def run(Q, K, V, dO=None, decay=None, m_in=None, dm_out=None, cu_seqlens=None,
        heads=None, backward=True):
    """Q, K, V, dO: float32-representable arrays [B, H, N, d] (bf16 inputs are
    passed upcast; the upcast is exact).  Computes in float64.

    heads: optional list of head indices to restrict the work to (a bounded
    sample); outputs for other heads are left zero.
    Returns dict with O, M_out and (if backward) dQ, dK, dV, dM_in, float64.
    """
    lib = _load()
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    B, H, N, d = Q.shape
    if cu_seqlens is None:
        seqs = [(b, 0, N) for b in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        seqs = [(0, cu[i], cu[i + 1]) for i in range(len(cu) - 1)]
    S = len(seqs)
    hs = list(range(H)) if heads is None else list(heads)
    row_off, lens, lams, unit_idx = [], [], [], []
    for si, (b, s, e) in enumerate(seqs):
        for h in hs:
            row_off.append((b * H + h) * N + s)
            lens.append(e - s)
            lams.append(1.0 if decay is None else float(np.float32(decay[h])))
            unit_idx.append((si, h))
    n = len(row_off)
    row_off = np.asarray(row_off, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    lams = np.asarray(lams, dtype=np.float64)

    def gather_state(m):
        if m is None:
            return None
        m = np.asarray(m, dtype=np.float64)
        return np.ascontiguousarray(np.stack([m[si, h] for si, h in unit_idx]) if n else
                                    np.zeros((0, d, d)))

    mi = gather_state(m_in)
    dmo = gather_state(dm_out)
    O = np.zeros((B, H, N, d))
    mo = np.zeros((n, d, d))
    out = {"O": O}
    args_bwd = [None] * 4
    if backward:
        dO = np.ascontiguousarray(dO, dtype=np.float32)
        dQ, dK, dV = np.zeros((B, H, N, d)), np.zeros((B, H, N, d)), np.zeros((B, H, N, d))
        dmi = np.zeros((n, d, d))
        args_bwd = [dQ, dK, dV, dmi]
    rc = lib.lasp_ref_run(n, _ptr(row_off), _ptr(lens), _ptr(lams), d, _ptr(Q), _ptr(K),
                          _ptr(V), _ptr(dO if backward else None), _ptr(mi), _ptr(dmo),
                          _ptr(O), _ptr(mo), *[_ptr(a) for a in args_bwd], int(backward))
    if rc != 0:
        raise MemoryError("crecurrent: scratch allocation failed")

    def scatter_state(m):
        full = np.zeros((S, H, d, d))
        for u, (si, h) in enumerate(unit_idx):
            full[si, h] = m[u]
        return full

    out["M_out"] = scatter_state(mo)
    if backward:
        out.update(dQ=args_bwd[0], dK=args_bwd[1], dV=args_bwd[2],
                   dM_in=scatter_state(args_bwd[3]))
    return out
