"""Seeded synthetic inputs for chunked causal linear attention.

This module only draws random inputs; it holds none of the method's arithmetic.
Both the HIP path's callers (tests, benchmark) and the CPU oracle's callers take
their inputs from here, so both sides see identical values.

Recipe (all configurations):
  * torch.Generator('cpu').manual_seed(seed), draws in the fixed order
    lengths (packed batches only), Q, K, V, dO, M_in, dM_out;
  * Q, K, V ~ N(0, 1) / sqrt(d); dO ~ N(0, 1); M_in, dM_out ~ N(0, 1) * scale;
  * values are drawn in float32; bf16 workloads round them to bfloat16 with
    round-to-nearest-even, and both sides consume the rounded values;
  * per-head decay (the lightning-attention style workload):
    lambda_h = 1 - 2^-(5 + 8 h / H), h = 0..H-1, computed in float64 and rounded
    to float32 (the decay is a fixed hyperparameter, never learned).
  * gated workloads draw, after everything above, x ~ N(0, 1) of shape
    [B, H, N, d] and take float32 log-gates from it:
      "gla"    log g = logsigmoid(x) / 16   (GLA-style gates near 1)
      "strong" log g = 4 logsigmoid(x) - 1  (gates from e^-1 down to ~0)
      "mixed"  "gla", except "strong" for tokens n with (n // 32) % 3 == 1
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "fp32" or "bf16"
    B: int
    H: int
    N: int                # tokens per sequence, or total tokens of a packed batch
    d: int
    chunk: int
    seed: int
    lengths: Optional[tuple] = None      # packed batch: drawn lengths are stored here
    len_range: Optional[tuple] = None    # packed batch: (nseq, lo, hi) to draw from
    decay: str = "none"                  # "none" | "lightning"
    gates: str = "none"                  # "none" | "gla" | "strong" | "mixed"
    m_in_scale: Optional[float] = None
    dm_out_scale: Optional[float] = None
    backward: bool = True

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


def _lengths(w: Workload, g: torch.Generator):
    if w.lengths is not None:
        return list(w.lengths)
    if w.len_range is not None:
        n, lo, hi = w.len_range
        return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]
    return None


def lightning_decay(H: int) -> torch.Tensor:
    """lambda_h = 1 - 2^-(5 + 8h/H), h = 0..H-1, float64 then rounded to float32."""
    return torch.tensor([1.0 - 2.0 ** (-(5.0 + 8.0 * h / H)) for h in range(H)],
                        dtype=torch.float64).to(torch.float32)


def make_inputs(w: Workload, backward: Optional[bool] = None, device: str = "cpu") -> dict:
    """Draw the inputs of workload w on `device` (a generator on that device,
    seeded with w.seed; draws on the GPU give other values than on the CPU, with
    the same recipe).  Returns a dict with
    Q, K, V (and dO when backward) in w's dtype [B, H, N, d]; decay float32 [H]
    or None; log_g float32 [B, H, N, d] or None (gated workloads); cu_seqlens int32 [nseq+1] or None; M_in / dM_out float32
    [S, H, d, d] or None; and the resolved shape (B, H, N, d, chunk, nseq)."""
    backward = w.backward if backward is None else backward
    g = torch.Generator("cpu").manual_seed(w.seed)
    lens = _lengths(w, g)
    if str(device) != "cpu":
        g = torch.Generator(device).manual_seed(w.seed)
    B, H, d = w.B, w.H, w.d
    if lens is not None:
        B, N = 1, int(sum(lens))
        cu = torch.tensor([0] + list(torch.cumsum(torch.tensor(lens), 0).tolist()),
                          dtype=torch.int32)
        S = len(lens)
    else:
        N, cu, S = w.N, None, w.B
    scale = 1.0 / math.sqrt(d)

    def draw(shape, s):
        return torch.randn(shape, generator=g, dtype=torch.float32, device=device) * s

    Q = draw((B, H, N, d), scale).to(w.torch_dtype)
    K = draw((B, H, N, d), scale).to(w.torch_dtype)
    V = draw((B, H, N, d), scale).to(w.torch_dtype)
    dO = draw((B, H, N, d), 1.0).to(w.torch_dtype) if backward else None
    M_in = draw((S, H, d, d), w.m_in_scale) if w.m_in_scale is not None else None
    dM_out = (draw((S, H, d, d), w.dm_out_scale)
              if (backward and w.dm_out_scale is not None) else None)
    decay = lightning_decay(H).to(device) if w.decay == "lightning" else None
    log_g = None
    if w.gates != "none":
        x = draw((B, H, N, d), 1.0)
        gla = torch.nn.functional.logsigmoid(x) / 16.0
        strong = 4.0 * torch.nn.functional.logsigmoid(x) - 1.0
        if w.gates == "gla":
            log_g = gla
        elif w.gates == "strong":
            log_g = strong
        elif w.gates == "mixed":
            n = torch.arange(N, device=device)
            log_g = torch.where(((n // 32) % 3 == 1)[:, None], strong, gla)
        else:
            raise ValueError(w.gates)
    if cu is not None:
        cu = cu.to(device)
    return dict(Q=Q, K=K, V=V, dO=dO, M_in=M_in, dM_out=dM_out, decay=decay, log_g=log_g,
                cu_seqlens=cu, lengths=lens,
                shape=dict(B=B, H=H, N=N, d=d, chunk=w.chunk,
                           nseq=(len(lens) if lens is not None else 0)))


# The five workloads: shapes of Linear-Llama3-1B-like attention heads (d = 128)
# and the small float32 case.  Packed-batch lengths are drawn from the seed.
CONFIGS = {
    1: Workload("fp32 B1 H2 N256 d32 C64 (forward only)", "fp32", 1, 2, 256, 32, 64,
                seed=1, backward=False),
    2: Workload("bf16 B4 H16 N8192 d128 C256", "bf16", 4, 16, 8192, 128, 256, seed=2),
    3: Workload("bf16 B1 H32 N131072 d128 C256, M_in and M_out", "bf16", 1, 32, 131072,
                128, 256, seed=3, m_in_scale=0.01),
    4: Workload("bf16 B2 H16 N32768 d128 C256, per-head decay", "bf16", 2, 16, 32768, 128,
                256, seed=4, decay="lightning"),
    5: Workload("bf16 packed 8 x U[1024,16384] H32 d64 C128", "bf16", 1, 32, 0, 64, 128,
                seed=5, len_range=(8, 1024, 16384)),
}

# The gated (GLA-style) form at the long-sequence shape, with the chunk length
# the gated kernels use.
GATED = Workload("bf16 B1 H32 N131072 d128 C64, GLA gates, M_in and M_out", "bf16", 1, 32,
                 131072, 128, 64, seed=6, gates="gla", m_in_scale=0.01)


def small(name, dtype="bf16", B=1, H=2, N=300, d=64, chunk=64, seed=0, lengths=None,
          decay="none", m_in_scale=None, dm_out_scale=None, backward=True,
          gates="none") -> Workload:
    """A reduced workload for parity tests."""
    return Workload(name, dtype, B, H, N, d, chunk, seed,
                    lengths=None if lengths is None else tuple(lengths), decay=decay,
                    gates=gates, m_in_scale=m_in_scale, dm_out_scale=dm_out_scale,
                    backward=backward)
