"""Oracle: a plain, slow, float64 CPU implementation of the routed-expert MoE
MLP forward (route, expert-sorted padded permutation, GEMM1 + SwiGLU, GEMM2,
weighted combine) and of its FP8 / MX quantisers.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg may import it. The product path (the HIP library
and its Python binding) never imports, calls or links anything here, and the
two share no code: the seeded input generators live in their own package
(workloads/), which holds none of the method's arithmetic.

Modules:
  formats  bit-level codecs: bf16 RN, fp32 RN, OCP E4M3FN, OCP E2M1, E8M0
  moe      route, align_sort, quantisers, GEMM1+SwiGLU, GEMM2, combine, forward

Every function is pinned by a -m "not gpu" test (tests/test_oracle_*.py) to
something other than itself: brute force on tiny inputs, exhaustive format
tables, library casts, closed forms and invariants.
"""
from . import formats, moe  # noqa: F401
