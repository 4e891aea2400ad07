"""sink_attn_decode_noalloc through the C ABI against sink_attn_decode (the
same problem with a caller workspace): two calls in a row, the second on a
smaller input, with split partials in the static scratch; a problem larger
than the scratch is refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import binding as B
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import DEV, dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20        # SINK_ATTN_NOALLOC_SCRATCH_BYTES


def _announce(name):
    print(f"[case] {name}", flush=True)


def _args(wl):
    q = dev(wl.q, wl.dtype)
    kc, vc = dev(wl.k_cache, wl.dtype), dev(wl.v_cache, wl.dtype)
    csl = torch.from_numpy(wl.cache_seqlens).to(DEV) if wl.cache_seqlens is not None else None
    sink = torch.from_numpy(wl.sink).to(DEV) if wl.sink is not None else None
    return q, kc, vc, csl, sink


def _compare(wl, splits):
    q, kc, vc, csl, sink = _args(wl)
    desc = B.decode_desc(q, kc, wl.scale, csl, sink, splits)
    need = B.lib().sink_attn_decode_workspace_size(ctypes.byref(desc))
    want = sa.decode(q, kc, vc, csl, wl.scale, sink, num_splits=splits)
    B_, hq, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B_, hq), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.full((B_, hq), float("nan"), dtype=torch.float32, device=DEV)
    got = sa.decode_noalloc(q, kc, vc, csl, wl.scale, sink, num_splits=splits, o=o, lse=lse, s=s)
    torch.cuda.synchronize()
    for g, w, name in zip(got, want, ("o", "lse", "s")):
        assert torch.equal(g, w), f"{name} differs from sink_attn_decode"
    return need


def test_noalloc_decode_two_calls_second_smaller():
    wl1 = W.make_decode("noalloc1", 16, 2000, 32, 4, 128, seed=31,
                        cache_seqlens=[2000, 1, 1500, 777] * 4)
    wl2 = W.make_decode("noalloc2", 5, 700, 16, 2, 128, seed=32)
    _announce("decode_noalloc call 1: 16 x 2000 slots, 4 splits")
    n1 = _compare(wl1, 4)
    _announce("decode_noalloc call 2: 5 x 700 slots, 3 splits")
    n2 = _compare(wl2, 3)
    assert 0 < n2 < n1 <= SCRATCH_BYTES


def test_noalloc_decode_auto_splits_and_one_split():
    wl = W.make_decode("noalloc3", 3, 1200, 16, 2, 128, seed=33)
    _announce("decode_noalloc auto splits")
    _compare(wl, 0)
    _announce("decode_noalloc one split (no partials)")
    assert _compare(wl, 1) == 0


def test_noalloc_decode_refuses_beyond_scratch():
    """1024 sequences x 64 heads x 64 splits of (D + 2) float32 partials is
    2.2 GB: more than the 16 MiB scratch, refused on the host."""
    q = torch.zeros((1024, 64, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((1024, 64, 1, 128), dtype=torch.bfloat16, device=DEV)
    _announce("decode_noalloc too large")
    with pytest.raises(sa.SinkAttnError, match="static scratch") as e:
        sa.decode_noalloc(q, kc, kc, None, None, None, num_splits=64)
    assert e.value.status == B.WORKSPACE_TOO_SMALL
