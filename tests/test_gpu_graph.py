"""Graph capture of the hot path.  The library launches on the caller's stream
(the backward also on its own second stream, forked from and joined back into
the caller's through events, which capture turns into graph edges), allocates
and synchronises nothing, and clears its work-queue counters and split-tile
accumulators with kernels (no memset nodes), so a captured forward + backward
+ decode, replayed several times with eager work and synchronisations between
the replays, matches the eager results every time.  The eager step runs
first, so the backward's second stream exists when the capture starts."""
import pytest
import torch

import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import DEV, dev, prefill_args

pytestmark = pytest.mark.gpu

CASES = {
    "window": dict(lengths=(400, 77, 260), hq=8, hkv=2, n_sink=4, window=100),
    # key tiles split over several work items: float32 partials added
    # atomically and converted afterwards, so the accumulators must be cleared
    # again on every replay
    "split": dict(lengths=(1200, 70), hq=16, hkv=2),
    "blocks": dict(lengths=(700, 130), hq=8, hkv=2, block_lists=dict(n_random=3)),
}
# outputs of one step: o, lse, s, dq, dk, dv, dsink, decode o, lse, s
NAMES = ["o", "lse", "s", "dq", "dk", "dv", "dsink", "dec_o", "dec_lse", "dec_s"]
ATOMIC = {"dk", "dv"}           # split tiles sum their partials in no fixed order


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    print(f"[case] graph {name}", flush=True)
    c = dict(CASES[name])
    wl = W.make_prefill(name, c.pop("lengths"), c.pop("hq"), c.pop("hkv"), 128, seed=11, **c)
    q, k, v, cu, bi, sink = prefill_args(wl)
    do = dev(wl.do, wl.dtype)
    dc = W.make_decode("graph_decode", 3, 300, 8, 2, 128, seed=12)
    qd, kc, vc = dev(dc.q, "bf16"), dev(dc.k_cache, "bf16"), dev(dc.v_cache, "bf16")
    sd = torch.from_numpy(dc.sink).to(DEV)
    # max_seqlen is passed, so no call reads the device from the host
    args = (cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink)

    def step():
        o, lse, s = sa.fwd(q, k, v, *args)
        dq, dk, dv, dsink = sa.bwd(q, k, v, o, lse, do, *args)
        od, lsed, s_d = sa.decode(qd, kc, vc, None, dc.scale, sd)
        return [o, lse, s, dq, dk, dv, dsink, od, lsed, s_d]

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                       # warm-up on a side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for r in range(3):
        junk = torch.randn(1 << 16, device=DEV)     # eager work between replays
        junk.mul_(2.0).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        for nm, g, e in zip(NAMES, outs, eager):
            if nm in ATOMIC:
                assert torch.allclose(g.float(), e.float(), rtol=2.0 ** -7, atol=1e-3), \
                    f"replay {r}: {nm} differs"
            else:
                assert torch.equal(g, e), f"replay {r}: {nm} differs"


@pytest.mark.parametrize("quantized", [False, True])
def test_graph_cache_step_replays_match_eager(quantized):
    """A serving step on the rolling cache captured as one graph: restore the
    cache from a snapshot, chunked prefill, append the chunk, decode with two
    splits.  Every replay, with eager work between, matches the eager step bit
    for bit (outputs and the cache after the append)."""
    print(f"[case] graph cache step q={quantized}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(13)
    B, hq, hkv, d, n_sink, window, C = 3, 8, 2, 128, 4, 120, 48
    rnd = lambda *shape, s=1.0: (torch.randn(*shape, generator=g) * s).to(torch.bfloat16).to(DEV)
    cache = sa.KvCache(B, n_sink, window, hkv, d, quantized)
    seen0 = torch.tensor([0, 30, 200], dtype=torch.int32, device=DEV)
    sa.kvcache_append(cache, rnd(B, 200, hkv, d), rnd(B, 200, hkv, d), torch.zeros_like(seen0))
    seen = seen0                                    # positions of the chunk's first token
    state = [t for t in (cache.k, cache.v, cache.sink_k, cache.sink_v, cache.win_k, cache.win_v,
                         cache.win_k_scale, cache.win_v_scale) if t is not None]
    snap = [t.clone() for t in state]
    q, kn, vn = rnd(B, C, hq, d), rnd(B, C, hkv, d, s=0.7), rnd(B, C, hkv, d)
    q1 = rnd(B, hq, d)
    n_tokens = seen + C
    sink = torch.randn(hq, generator=g).to(DEV)

    def step():
        for t, s0 in zip(state, snap):
            t.copy_(s0)
        o, lse, s = sa.kvcache_prefill(cache, q, kn, vn, seen, 0.09, sink)
        sa.kvcache_append(cache, kn, vn, seen)
        od, ld, sd = sa.kvcache_decode(cache, q1, n_tokens, 0.09, sink, num_splits=2)
        return [o, lse, s, od, ld, sd] + state

    eager = [t.clone() for t in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = step()
    for r in range(3):
        junk = torch.randn(1 << 16, device=DEV)
        junk.mul_(2.0).sum().item()
        for t in state:                              # disturb the cache: the graph restores it
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, e) in enumerate(zip(outs, eager)):
            assert torch.equal(a, e), f"replay {r}: output {i} differs"
