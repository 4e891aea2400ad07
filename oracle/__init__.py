"""Float64 CPU oracle for sink attention (test infrastructure only).

Only the tests, the smoke entry point and the benchmark's CPU-baseline leg use
this package; the HIP path never imports it.
"""
from .sink_attn_oracle import *  # noqa: F401,F403
