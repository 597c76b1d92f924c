"""Build the HIP library (gfx950) in-tree: chunked_causal_linear_amd/liblasp.so.

The sources are compiled to objects in parallel (one hipcc process each) and
linked into one shared library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = [os.path.join(HERE, "csrc", n) for n in ("lasp_kernels.hip", "lasp_gated.hip", "lasp_api.cpp")]
LIB = os.path.join(HERE, "liblasp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from emitting packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
_NOISE = "packed-fp32-ops' is not a recognized feature"


def _filter(text):
    return [l for l in text.splitlines() if _NOISE not in l]


def build(verbose: bool = False) -> str:
    """Compile liblasp.so (always recompiles).  Returns its path."""
    with tempfile.TemporaryDirectory(prefix="lasp_build_") as tmpdir:
        objs, procs = [], []
        for src in SRC:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            procs.append((src, subprocess.Popen([HIPCC, *FLAGS, "-c", "-o", obj, src],
                                                stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
        msgs, failed = [], []
        for src, pr in procs:
            out, _ = pr.communicate()
            msgs += _filter(out)
            if pr.returncode != 0:
                failed.append(os.path.basename(src))
        if failed:
            raise RuntimeError("hipcc failed on %s:\n%s" % (", ".join(failed), "\n".join(msgs)))
        tmp = LIB + ".tmp%d" % os.getpid()
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                           capture_output=True, text=True)
        msgs += _filter(r.stdout + r.stderr)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
