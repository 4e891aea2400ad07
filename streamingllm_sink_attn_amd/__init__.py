"""Attention with a learnable sink for AMD MI355X (gfx950).

The compute lives in ``libsinkattn.so`` (HIP kernels behind a C ABI declared
in ``include/sink_attn.h``); :mod:`.binding` marshals torch tensors into it.
:mod:`.workloads` draws the seeded synthetic inputs.
"""
from .binding import SinkAttnError, bwd, debug_visit_map, decode, fwd, lib, prefill_path  # noqa: F401

__all__ = ["fwd", "bwd", "decode", "debug_visit_map", "prefill_path", "lib", "SinkAttnError"]
