"""Attention with a learnable sink for AMD MI355X (gfx950).

The compute lives in ``libsinkattn.so`` (HIP kernels behind a C ABI declared
in ``include/sink_attn.h``); :mod:`.binding` marshals torch tensors into it.
:mod:`.workloads` draws the seeded synthetic inputs.
"""
from .binding import (KvCache, SinkAttnError, bwd, debug_visit_map, decode, decode_noalloc,  # noqa: F401
                      fwd,
                      fwd_gated, head_importance, kvcache_append, kvcache_decode, kvcache_prefill, lib,
                      prefill_path)

__all__ = ["fwd", "fwd_gated", "head_importance", "bwd", "decode", "decode_noalloc", "KvCache", "kvcache_append",
           "kvcache_decode", "kvcache_prefill", "debug_visit_map", "prefill_path", "lib", "SinkAttnError"]
