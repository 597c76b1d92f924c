"""CPU oracle for chunked causal linear attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link or
execute anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

Sources (cited by page title and section / equation / algorithm):
  [LASP]   "Linear Attention Sequence Parallelism" (arXiv 2404.02882), full text:
           Sec. 3.1 (Eqs. 2-3), Sec. 3.2 (Eqs. 4-23, Algorithms 2 and 3).
  [LASP-2] "LASP-2: Rethinking Sequence Parallelism for Linear Attention and Its
           Hybrid" (arXiv 2502.07563), review page: the memory state
           M_t = K_t^T V_t, its prefix sums and the masked intra/inter split.
  [LASP] Appendix A.4, Eq. 24 and Table 5 (GLA / GateLoop row): the gated
           recurrence with a per-token, per-key-channel gate.

Modules:
  lasp_oracle   numpy float64: the quadratic masked definition, the token
                recurrence, the chunked (intra/inter) form, row-sampled sums.
  gated_oracle  numpy float64: the gated recurrence, its unrolled closed form,
                its reverse-mode derivative and row-sampled prefix/suffix sums.
  crecurrent    a plain C float64 token recurrence (OpenMP over heads), used for
                full tensors at medium sizes and as the timed CPU baseline.
"""
from .lasp_oracle import *  # noqa: F401,F403
from .gated_oracle import *  # noqa: F401,F403
