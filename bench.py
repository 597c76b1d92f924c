#!/usr/bin/env python3
"""Benchmark: one step = lasp_fwd + lasp_bwd (the whole hot path: chunk states,
state scan, fused output, reverse scan, dQ/dK/dV) over one batch of synthetic
input on one MI355X, with inputs resident in HBM.

Default workload: bf16, B=1, H=32, N=131072, d=128, chunk=256, with an incoming
state M_in and the outgoing M_out (one device's share of a long sequence).

Prints ONE JSON line.  Besides the contract fields it carries:
  roofline      for the dominant kernel, timed live with HIP events recorded on
                the launch stream around that kernel inside the library;
  cpu_baseline  the float64 C oracle (token recurrence) timed on the host cores
                over a bounded sample of the same workload;
  kernels_ms    average duration of every kernel of the step.
Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 3] [--bidir | --gated]
--bidir times the unmasked (bidirectional) form instead (lasp_fwd_bidir +
lasp_bwd_bidir on the same inputs, no decay) and prints its own line.
--gated times the gated form (lasp_fwd_gated + lasp_bwd_gated) on its own
workload: bf16 B1 H32 N131072 d128 C64 with GLA-style gates, M_in and M_out.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
CSRC = os.path.join(ROOT, "chunked_causal_linear_amd", "csrc")
KERNEL_SRC = [os.path.join(CSRC, "lasp_kernels.hip"), os.path.join(CSRC, "lasp_device.h")]
GATED_SRC = [os.path.join(CSRC, "lasp_gated.hip"), os.path.join(CSRC, "lasp_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
GATED_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters_gated.json")


def hip():
    L = ctypes.CDLL("libamdhip64.so")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


def make_events(L, n):
    arr = (ctypes.c_void_p * n)()
    for i in range(n):
        h = ctypes.c_void_p()
        assert L.hipEventCreate(ctypes.byref(h)) == 0
        arr[i] = h
    return arr


def elapsed(L, a, b):
    ms = ctypes.c_float()
    assert L.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
    return ms.value


def end_segment_tokens(lengths, C, G):
    """Tokens of the sequences' last segments and of their first segments (G
    chunks of C tokens; a sequence's last segment may be short)."""
    last = first = 0
    for n in lengths:
        if n > 0:
            T = -(-n // C)
            S = -(-T // G)
            last += n - (S - 1) * G * C
            first += min(n, G * C)
    return last, first


def kernel_work(sh, local_b, seg_b, fin_b, G=0, lengths=None):
    """Algorithmic HBM bytes and flops per launch of every kernel of a step.

    U = token-heads, e = element bytes; local_b / seg_b / fin_b: bytes of the
    per-chunk (element type, none for bf16), per-segment (float32) and
    per-sequence final (float32, bf16 only) state arrays, from the library's
    size queries.  Bytes count every distinct array once:
      local  : reads 2 token arrays (K,V resp. Q,dO), writes the local states
      scan   : reads and writes the segment states, M_in/M_out (dM_out/dM_in)
      out    : reads Q,K,V and the segment states, writes O
      grads  : reads Q,K,V,dO and both segment-state arrays, writes dQ,dK,dV
    In the bf16 path (fin_b > 0) the sweeps write the end states: the output
    sweep M_out and the final states, the gradient sweep dM_in and the reverse
    final states (and it reads the forward's final states).
    The bf16 path (fin_b > 0) writes the end states from the sweeps and skips
    the totals of each sequence's last segment (forward) and first segment
    (backward): with G (chunks per segment) and the sequence lengths, the
    local kernels' token reads leave those segments out.
    Flops count the useful causal work per token-head and output role: the
    intra-chunk products over c <= r (2d(C+1) on average: QK^T and SV), the
    inter-chunk product A.X (2d^2) and the state update (2d^2)."""
    B, H, N, d, C = sh["B"], sh["H"], sh["N"], sh["d"], sh["chunk"]
    e = 2 if sh["dtype"] == "bf16" else 4
    U = B * H * N
    nS = sh["nseq"] or B
    st_io = nS * H * d * d * 4                    # M_in / M_out, dM_out / dM_in
    role = U * (2 * d * (C + 1) + 4 * d * d)      # one output role (O, dQ, dK or dV)
    Uf = Ub = U
    ends = 0                                      # end-state bytes moved from the scans to the sweeps
    if fin_b:
        ends = st_io
        if G:
            last, first = end_segment_tokens(lengths or [N] * B, C, G)
            Uf, Ub = U - H * last, U - H * first
    return {
        "fwd_local": (2 * Uf * d * e + local_b + seg_b, 2 * Uf * d * d),
        "fwd_scan": (2 * seg_b + 2 * st_io - ends, seg_b // 2),
        "fwd_out": (4 * U * d * e + local_b + seg_b + ends + fin_b, role),
        "bwd_local": (2 * Ub * d * e + local_b + seg_b, 2 * Ub * d * d),
        "bwd_scan": (2 * seg_b + 2 * st_io - ends, seg_b // 2),
        "bwd_grads": (7 * U * d * e + 2 * local_b + 2 * seg_b + 2 * fin_b + ends, 3 * role),
    }


def src_sha(files=None):
    """sha256 over the kernel sources (the kernel file and the shared device header)."""
    h = hashlib.sha256()
    for f in files or KERNEL_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel, workload, traffic_file=None, files=None):
    """HBM bytes per launch from committed rocprofv3 counters, if they were taken
    on the current kernel source and on this workload; else None."""
    try:
        t = json.load(open(traffic_file or TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != src_sha(files) or t.get("workload") != workload:
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def cpu_baseline(inp, H, tokens):
    """The float64 C oracle over a bounded sample: the first `tokens` tokens of
    every head (OpenMP over heads), forward + backward."""
    from oracle import crecurrent
    threads = crecurrent.threads()
    nh = H
    take = lambda x: x[:, :nh, :tokens].float().cpu().numpy()
    Q, K, V, dO = (take(inp[k]) for k in ("Q", "K", "V", "dO"))
    M_in = None if inp["M_in"] is None else inp["M_in"][:, :nh].double().cpu().numpy()
    t0 = time.perf_counter()
    crecurrent.run(Q, K, V, dO, None, M_in, None)
    dt = time.perf_counter() - t0
    th = Q.shape[0] * nh * Q.shape[2]            # token-heads processed
    cpu = "?"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": th / H / dt, "unit": "tokens/s", "cores": min(threads, nh), "kind": "oracle",
            "cpu": cpu,
            "sample": "%d of %d heads x first %d tokens, fwd+bwd float64 token recurrence "
                      "(C, OpenMP over heads), %.2f s; tokens/s counts all %d heads per token"
                      % (nh, H, Q.shape[2], dt, H)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=0,
                    help="override the workload's chunk length (64, 128 or 256)")
    ap.add_argument("--cpu-tokens", type=int, default=131072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bidir", action="store_true",
                    help="time the unmasked (bidirectional) form instead")
    ap.add_argument("--gated", action="store_true",
                    help="time the gated (per-channel decay) form on its own workload")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (3 times), to calibrate "
                         "the HBM byte counters of a profiler against known traffic")
    a = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d, WORLD_SIZE %d requested)" % (a.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    if a.copy_calib:
        n = a.copy_calib << 20
        x = torch.empty(n, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        x.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": n, "copy_calib_bytes_written": n}), flush=True)
        return
    import chunked_causal_linear_amd as cca
    from chunked_causal_linear_amd.workloads import CONFIGS, GATED, make_inputs

    w = GATED if a.gated else CONFIGS[a.config]
    if a.chunk:
        import dataclasses
        w = dataclasses.replace(w, chunk=a.chunk, name=w.name.replace("C%d" % w.chunk, "C%d" % a.chunk))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w, device="cuda")
    sh = dict(inp["shape"], dtype=w.dtype)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    decay, cu, M_in, dM_out = inp["decay"], inp["cu_seqlens"], inp["M_in"], inp["dM_out"]
    C = sh["chunk"]

    if a.bidir:
        return bench_bidir(a, w, sh, inp, torch, cca)
    if a.gated:
        return bench_gated(a, w, sh, inp, torch, cca)
    S = cca.Shape(sh["B"], sh["H"], sh["N"], sh["d"], C, sh["nseq"])
    dt_code = cca.LASP_BF16 if w.dtype == "bf16" else cca.LASP_FP32
    wsf = torch.empty(max(1, cca.fwd_workspace_bytes(S, dt_code, True)), dtype=torch.uint8,
                      device=dev)
    wsb = torch.empty(max(1, cca.bwd_workspace_bytes(S, dt_code, True)), dtype=torch.uint8,
                      device=dev)

    L = hip()
    n = a.warmup + a.steps
    evf = [make_events(L, 4) for _ in range(n)]
    evb = [make_events(L, 4) for _ in range(n)]

    def step(i):
        O, M_out, cache = cca.fwd(Q, K, V, C, decay, cu, M_in, workspace=wsf, events=evf[i])
        g = cca.bwd(Q, K, V, dO, C, decay, cu, M_in, dM_out, cache, workspace=wsb,
                    events=evb[i])
        return O, g

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.warmup, n):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / a.steps

    names = ["fwd_local", "fwd_scan", "fwd_out", "bwd_local", "bwd_scan", "bwd_grads"]
    kms = {k: 0.0 for k in names}
    step_ms = []
    for i in range(a.warmup, n):
        for j in range(3):
            kms[names[j]] += elapsed(L, evf[i][j], evf[i][j + 1]) / a.steps
            kms[names[3 + j]] += elapsed(L, evb[i][j], evb[i][j + 1]) / a.steps
        step_ms.append(elapsed(L, evf[i][0], evb[i][3]))
    step_ms.sort()

    # state array sizes (fwd workspace with a cache = tables + per-segment states;
    # state cache = per-chunk states + per-segment states + final states)
    table_b = 0 if not sh["nseq"] else -(-8 * (sh["nseq"] + 1) // 256) * 256
    seg_b = cca.fwd_workspace_bytes(S, dt_code, True) - table_b
    fin_b = 0 if sh["dtype"] != "bf16" else -(-(sh["nseq"] or sh["B"]) * sh["H"] * sh["d"] ** 2 * 4 // 256) * 256
    local_b = cca.state_cache_bytes(S, dt_code) - seg_b - fin_b
    lengths = None if cu is None else [int(x) for x in (cu[1:] - cu[:-1]).tolist()]
    G = cca.query_sizes(S, dt_code).segment_chunks
    work = kernel_work(sh, local_b, seg_b, fin_b, G, lengths)
    dom = max(names, key=lambda k: kms[k])
    bytes_, flops = work[dom]
    t_dom = kms[dom] * 1e-3
    hbm_time, mfma_time = bytes_ / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if hbm_time >= mfma_time:
        roof = {"bound": "hbm", "achieved": bytes_ / t_dom / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, w.name)
    roof.update(kernel=dom, ms=kms[dom], algorithmic_bytes=bytes_, algorithmic_flops=flops)

    tokens = sh["B"] * sh["N"]
    d = sh["d"]
    U = tokens * sh["H"]
    f_dense = U * (12 * d * d + 14 * C * d)
    f_causal = U * (12 * d * d + 7 * C * d)
    out = {
        "metric": "causal linear-attn fwd+bwd tokens/s and % bf16 MFMA peak, d=128, N=131072",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": sh["B"], "H": sh["H"], "N": sh["N"], "d": d,
                   "chunk": C, "nseq": sh["nseq"], "decay": w.decay,
                   "m_in": M_in is not None, "parallelism": "single GPU"},
        "tflops_dense_chunk": f_dense / (ms * 1e-3) / 1e12,
        "tflops_causal_useful": f_causal / (ms * 1e-3) / 1e12,
        "mfma_peak_frac_dense": f_dense / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "compulsory_io_GBs": (U * d * (8 + 14) * (2 if w.dtype == "bf16" else 4) / 2)
                             / (ms * 1e-3) / 1e9,
        "ms_per_step_events": {"median": step_ms[len(step_ms) // 2], "min": step_ms[0]},
        "kernels_ms": kms,
        "roofline": roof,
        "gpu": torch.cuda.get_device_name(dev),
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, sh["H"], min(a.cpu_tokens, sh["N"]))
    print(json.dumps(out), flush=True)


def bench_bidir(a, w, sh, inp, torch, cca):
    """One step = lasp_fwd_bidir + lasp_bwd_bidir (segment totals, scan, row-block
    products) on the workload's inputs; timed with events on the launch stream
    around each call.  Roofline: the whole step against HBM (every kernel of
    this form streams its rows once)."""
    if w.dtype != "bf16":
        sys.exit("--bidir needs a bf16 workload")
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    cu, M_in, dM_out = inp["cu_seqlens"], inp["M_in"], inp["dM_out"]
    C = sh["chunk"]
    n = a.warmup + a.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]

    def step(i):
        ev[i][0].record()
        O, M_out, cache = cca.fwd_bidir(Q, K, V, C, cu, M_in)
        ev[i][1].record()
        g = cca.bwd_bidir(Q, K, V, dO, C, cu, M_in, dM_out, cache)
        ev[i][2].record()
        return O, g

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.warmup, n):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    fwd_ms = sorted(ev[i][0].elapsed_time(ev[i][1]) for i in range(a.warmup, n))
    bwd_ms = sorted(ev[i][1].elapsed_time(ev[i][2]) for i in range(a.warmup, n))
    tokens = sh["B"] * sh["N"]
    U, d = tokens * sh["H"], sh["d"]
    bytes_ = 12 * U * d * 2          # fwd: K, V, Q in, O out; bwd: Q, dO, dO, K, V in, dQ, dK, dV out
    flops = 12 * U * d * d           # six d x d contractions per token-head
    med = fwd_ms[len(fwd_ms) // 2] + bwd_ms[len(bwd_ms) // 2]
    out = {
        "metric": "unmasked linear-attn fwd+bwd tokens/s, d=128, N=131072",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name + ", unmasked", "B": sh["B"], "H": sh["H"], "N": sh["N"],
                   "d": d, "chunk": C, "nseq": sh["nseq"], "m_in": M_in is not None,
                   "parallelism": "single GPU"},
        "calls_ms": {"fwd_bidir": fwd_ms[len(fwd_ms) // 2], "bwd_bidir": bwd_ms[len(bwd_ms) // 2]},
        "roofline": {"bound": "hbm", "achieved": bytes_ / (med * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": bytes_ / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": None, "kernel": "whole step", "algorithmic_bytes": bytes_,
                     "algorithmic_flops": flops},
        "gpu": torch.cuda.get_device_name(torch.device("cuda:0")),
    }
    print(json.dumps(out), flush=True)


def gated_work(sh, P):
    """Algorithmic HBM bytes and flops per launch of the gated kernels (U token-
    heads, e element bytes, log-gates and their gradient float32).  P: the
    library's array sizes (seg_b per-segment float32 states, gate_s per-segment
    gate products, fin_b final states).  Bytes: the token rows each kernel needs,
    its outputs and the segment states it reads or writes; the backward walks'
    intermediate arrays (q . dq parked in the log-gate gradient, per-chunk sums,
    state checkpoints) are overhead, not counted.  Flops count useful causal
    work: intra-chunk products over c <= r (2d(C+1) per output role) and the
    d x d state products (2d^2 each)."""
    B, H, N, d, C = sh["B"], sh["H"], sh["N"], sh["d"], sh["chunk"]
    e = 2 if sh["dtype"] == "bf16" else 4
    U = B * H * N
    nS = sh["nseq"] or B
    st_io = nS * H * d * d * 4
    T, G = U * d * e, U * d * 4                  # one token array, the log-gate array
    sb, gs, fb = P["seg_b"], P["gate_s"], P["fin_b"]
    intra = 2 * d * (C + 1)
    return {
        "fwd_local": (2 * T + G + sb + gs, 2 * U * d * d),
        "fwd_scan": (2 * sb + gs + fb + 2 * st_io, sb // 2),
        "fwd_out": (4 * T + G + sb, U * (intra + 4 * d * d)),
        "bwd_local": (2 * T + G + sb, 2 * U * d * d),
        "bwd_scan": (2 * sb + gs + 2 * st_io, sb // 2),
        "bwd_grads": (11 * T + 3 * G + 2 * sb, U * (3 * intra + 10 * d * d)),
    }


def bench_gated(a, w, sh, inp, torch, cca):
    """One step = lasp_fwd_gated + lasp_bwd_gated (segment totals, scan, output
    walk; reverse segment totals, reverse scan, the dQ walk and the dV / dK /
    log-gate gradient walk, timed together as bwd_grads),
    with per-kernel HIP events recorded on the launch stream inside the library."""
    Q, K, V, dO, LG = inp["Q"], inp["K"], inp["V"], inp["dO"], inp["log_g"]
    cu, M_in, dM_out = inp["cu_seqlens"], inp["M_in"], inp["dM_out"]
    C = sh["chunk"]
    dev = torch.device("cuda:0")
    S = cca.Shape(sh["B"], sh["H"], sh["N"], sh["d"], C, sh["nseq"])
    dt_code = cca.LASP_BF16 if w.dtype == "bf16" else cca.LASP_FP32
    wsf = torch.empty(max(1, cca.gated_fwd_workspace_bytes(S, dt_code, True)), dtype=torch.uint8,
                      device=dev)
    wsb = torch.empty(max(1, cca.gated_bwd_workspace_bytes(S, dt_code, True)), dtype=torch.uint8,
                      device=dev)
    L = hip()
    n = a.warmup + a.steps
    evf = [make_events(L, 4) for _ in range(n)]
    evb = [make_events(L, 4) for _ in range(n)]

    def step(i):
        O, M_out, cache = cca.fwd_gated(Q, K, V, LG, C, cu, M_in, workspace=wsf, events=evf[i])
        g = cca.bwd_gated(Q, K, V, LG, dO, C, cu, M_in, dM_out, cache, workspace=wsb,
                          events=evb[i])
        return O, g

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.warmup, n):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    names = ["fwd_local", "fwd_scan", "fwd_out", "bwd_local", "bwd_scan", "bwd_grads"]
    kms = {k: 0.0 for k in names}
    for i in range(a.warmup, n):
        for j in range(3):
            kms[names[j]] += elapsed(L, evf[i][j], evf[i][j + 1]) / a.steps
            kms[names[3 + j]] += elapsed(L, evb[i][j], evb[i][j + 1]) / a.steps
    # array sizes from the size queries: fwd workspace with a cache = tables + Z;
    # cache = Pseg + Pfin + Gs
    U, d = sh["B"] * sh["H"] * sh["N"], sh["d"]
    e = 2 if w.dtype == "bf16" else 4
    table_b = 0 if not sh["nseq"] else -(-8 * (sh["nseq"] + 1) // 256) * 256
    seg_b = cca.gated_fwd_workspace_bytes(S, dt_code, True) - table_b
    cache_b = cca.gated_state_cache_bytes(S, dt_code)
    fin_b = -(-(sh["nseq"] or sh["B"]) * sh["H"] * d * d * 4 // 256) * 256
    gate_s = cache_b - seg_b - fin_b
    work = gated_work(sh, dict(seg_b=seg_b, gate_s=gate_s, fin_b=fin_b))
    dom = max(names, key=lambda k: kms[k])
    bytes_, flops = work[dom]
    t_dom = kms[dom] * 1e-3
    if bytes_ / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12):
        roof = {"bound": "hbm", "achieved": bytes_ / t_dom / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dom, w.name, GATED_TRAFFIC_FILE, GATED_SRC)
    roof.update(kernel="gated " + dom, ms=kms[dom], algorithmic_bytes=bytes_,
                algorithmic_flops=flops)
    tokens = sh["B"] * sh["N"]
    step_bytes = sum(b for b, _ in work.values())
    out = {
        "metric": "gated (per-channel decay) linear-attn fwd+bwd tokens/s, d=128, N=131072",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": sh["B"], "H": sh["H"], "N": sh["N"], "d": d,
                   "chunk": C, "nseq": sh["nseq"], "gates": w.gates, "m_in": M_in is not None,
                   "parallelism": "single GPU"},
        "kernels_ms": kms,
        "step_algorithmic_GBs": step_bytes / (ms * 1e-3) / 1e9,
        "roofline": roof,
        "gpu": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
