"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The C ABI (chunked_causal_linear_amd/csrc/lasp_api.cpp) is compiled with g++
  into tests/sanitize/api_driver.cpp, whose stubbed kernel launchers check that
  every array the plan places in the caller's workspace and state cache lies
  inside that buffer and overlaps no other, over shapes up to 2^21 tokens x 96
  heads, every dtype, form, segment length and cache setting, plus the
  LASP_DEBUG validation of cu_seqlens and decay.
* The C float64 oracle (oracle/crecurrent.c) is compiled with gcc into
  tests/sanitize/crec_driver.c and run on ragged packed sequences (lengths 0,
  1, 5, 64, 65, 200) with decay, M_in and dM_out; its outputs must equal the
  Python quadratic oracle's.
Both builds are host-only (g++ / gcc, no .hip source), with -fno-sanitize-recover
so that any report fails the run.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import lasp_oracle as lo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs g++ and gcc")


def test_api_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_driver")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-o", exe, os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp")],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr


def test_c_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "crec_driver")
    subprocess.run(["gcc", *SAN, "-fopenmp", "-o", exe,
                    os.path.join(ROOT, "tests", "sanitize", "crec_driver.c")],
                   check=True, capture_output=True, text=True)
    r = np.random.default_rng(5)
    d, H, lens = 16, 2, [0, 1, 5, 64, 65, 200]
    N = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    Q, K, V = (r.standard_normal((1, H, N, d)).astype(np.float32) / 4 for _ in range(3))
    dO = r.standard_normal((1, H, N, d)).astype(np.float32)
    lam = np.array([0.9, 1.0])
    S = len(lens)
    m_in = r.standard_normal((S, H, d, d)) * 0.1
    dm_out = r.standard_normal((S, H, d, d)) * 0.1
    units = [(si, h) for si in range(S) for h in range(H)]
    off = np.array([h * N + cu[si] for si, h in units], dtype=np.int64)
    ln = np.array([lens[si] for si, _ in units], dtype=np.int64)
    lm = np.array([lam[h] for _, h in units], dtype=np.float64)
    mi = np.stack([m_in[si, h] for si, h in units])
    dmo = np.stack([dm_out[si, h] for si, h in units])
    rows = H * N
    inp = str(tmp_path / "in.bin")
    with open(inp, "wb") as f:
        np.array([len(units), d, rows, 1], dtype=np.int32).tofile(f)
        off.tofile(f), ln.tofile(f), lm.tofile(f)
        for a in (Q, K, V, dO):
            a.reshape(-1).tofile(f)
        mi.tofile(f), dmo.tofile(f)
    out = str(tmp_path / "out.bin")
    p = subprocess.run([exe, inp, out], capture_output=True, text=True, env=ENV, timeout=300)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "runtime error" not in p.stderr, p.stderr
    res = np.fromfile(out, dtype=np.float64)
    n4 = rows * d
    got = {k: res[i * n4:(i + 1) * n4].reshape(1, H, N, d) for i, k in enumerate(("O", "dQ", "dK", "dV"))}
    nd = len(units) * d * d
    mo = res[4 * n4:4 * n4 + nd].reshape(len(units), d, d)
    dmi = res[4 * n4 + nd:].reshape(len(units), d, d)
    O, Mo = lo.batched_fwd(Q.astype(np.float64), K.astype(np.float64), V.astype(np.float64),
                           lam, m_in, cu)
    dQ, dK, dV, dMi = lo.batched_bwd(Q.astype(np.float64), K.astype(np.float64),
                                     V.astype(np.float64), dO.astype(np.float64), lam, m_in,
                                     dm_out, cu)
    for k, ref in (("O", O), ("dQ", dQ), ("dK", dK), ("dV", dV)):
        assert np.abs(got[k] - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), k
    for u, (si, h) in enumerate(units):
        assert np.abs(mo[u] - Mo[si, h]).max() <= 1e-12
        assert np.abs(dmi[u] - dMi[si, h]).max() <= 1e-12
