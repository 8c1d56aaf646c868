"""CPU oracle for decode attention over a rotated, 2/4-bit quantized, paged KV cache.

TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the bench's CPU-baseline
leg may import this package; the GPU library and its Python binding never do.
See oracle/kvq_oracle.py for the definitions and their sources.
"""
from .kvq_oracle import *  # noqa: F401,F403
