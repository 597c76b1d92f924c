"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte counts behind the roofline, and the rule that committed HBM counters are
reported only for the kernel source and the workload they were taken on."""
import json
import os
import subprocess
import sys

import bench
from chunked_causal_linear_amd.workloads import CONFIGS, GATED

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_work_counts_every_array_once():
    # bf16 B1 H32 N131072 d128 C256 without per-chunk states: U token-heads
    sh = dict(B=1, H=32, N=131072, d=128, chunk=256, dtype="bf16", nseq=0)
    U, d, e = 32 * 131072, 128, 2
    seg_b = 1 << 20
    work = bench.kernel_work(sh, 0, seg_b, 0)
    assert work["fwd_local"][0] == 2 * U * d * e + seg_b          # K, V in; totals out
    assert work["fwd_out"][0] == 4 * U * d * e + seg_b            # Q, K, V in; O out
    assert work["bwd_grads"][0] == 7 * U * d * e + 2 * seg_b      # Q, K, V, dO in; dQ, dK, dV out
    # one output role: causal intra-chunk products + inter-chunk product + state update
    role = U * (2 * d * (256 + 1) + 4 * d * d)
    assert work["fwd_out"][1] == role and work["bwd_grads"][1] == 3 * role


def test_kernel_work_leaves_out_the_skipped_totals():
    """With the end states written by the sweeps, the forward totals read no
    token of a sequence's last segment and the backward totals none of its
    first."""
    assert bench.end_segment_tokens([131072], 256, 64) == (16384, 16384)
    # 300 tokens in chunks of 64: 5 chunks, segments of 2 chunks: 128 | 128 | 44
    assert bench.end_segment_tokens([300, 0, 1], 64, 2) == (44 + 1, 128 + 1)
    sh = dict(B=1, H=32, N=131072, d=128, chunk=256, dtype="bf16", nseq=0)
    U, d, e = 32 * 131072, 128, 2
    seg_b, fin_b, st = 1 << 20, 1 << 16, 32 * 128 * 128 * 4
    work = bench.kernel_work(sh, 0, seg_b, fin_b, G=64)
    assert work["fwd_local"][0] == 2 * (U * 7 // 8) * d * e + seg_b
    assert work["bwd_local"][0] == 2 * (U * 7 // 8) * d * e + seg_b
    assert work["fwd_out"][0] == 4 * U * d * e + seg_b + st + fin_b      # M_out, Pfin out
    assert work["bwd_grads"][0] == 7 * U * d * e + 2 * seg_b + 2 * fin_b + st
    assert work["fwd_scan"][0] == 2 * seg_b + st                          # M_in in


def test_counters_only_for_their_source_and_workload(tmp_path):
    f = tmp_path / "t.json"
    json.dump({"source_sha256": bench.src_sha(), "workload": CONFIGS[3].name,
               "kernels": {"bwd_grads": {"hbm_bytes_per_launch": 123.0}}}, open(f, "w"))
    assert bench.measured_traffic("bwd_grads", CONFIGS[3].name, str(f)) == 123.0
    assert bench.measured_traffic("bwd_grads", CONFIGS[4].name, str(f)) is None
    assert bench.measured_traffic("fwd_out", CONFIGS[3].name, str(f)) is None
    json.dump({"source_sha256": "0" * 64, "workload": CONFIGS[3].name,
               "kernels": {"bwd_grads": {"hbm_bytes_per_launch": 123.0}}}, open(f, "w"))
    assert bench.measured_traffic("bwd_grads", CONFIGS[3].name, str(f)) is None
    assert bench.measured_traffic("bwd_grads", CONFIGS[3].name, str(tmp_path / "missing.json")) is None


def test_committed_counters_name_their_workloads():
    for path, name in ((bench.TRAFFIC_FILE, CONFIGS[3].name), (bench.GATED_TRAFFIC_FILE, GATED.name)):
        t = json.load(open(path))
        assert t["workload"] == name
        assert len(t["source_sha256"]) == 64
