"""Float64 CPU oracle for gated causal GQA attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
calls it and shares no code with it.

Modules:
  reference -- the plain definition in float64 NumPy (attention, per-chunk
               partials, the log-sum-exp merge, the KV append), plus the
               head-chunked evaluation order of the pages;
  brute     -- the same definition with Python loops, math.fsum and math.exp,
               for tiny inputs;
  plan      -- the head-chunk rule as the pages state it.

Parity status: every function is pinned by tests/test_oracle_*.py against
brute force, torch's CPU float64 SDPA, closed forms, invariants and the pages'
worked example; none is "parity unpinned".
"""

from . import brute, plan, reference  # noqa: F401
