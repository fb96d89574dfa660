"""KDA CPU oracle (float64) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.  It
shares no code with the HIP path and does not import the product package.
"""
from .kda_oracle import (brute_force, build, chunked, decode_step, default_threads, exact,
                         frontend, output_gate, recurrence)

__all__ = ["brute_force", "build", "chunked", "decode_step", "default_threads", "exact",
           "frontend", "output_gate", "recurrence"]
