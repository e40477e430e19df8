"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package draws random numbers and builds input structure (bf16/fp16 bit
patterns, near-tied score pairs, verify masks).  It holds none of the attention
arithmetic: neither the HIP path nor the oracle lives here, and this package
imports neither of them.
"""

from .inputs import *  # noqa: F401,F403
