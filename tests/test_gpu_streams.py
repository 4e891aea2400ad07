"""Calls on a stream other than the current one, and the debug precondition
checks on device inputs.

Outputs and workspace are allocated on the stream the kernels run on, so the
caching allocator cannot hand the workspace of an unfinished call to work on
the current stream: the backward and the cache decode run on a side stream
while the current stream allocates and fills buffers, and must still match
the oracle."""
import numpy as np
import pytest
import torch

import oracle
import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import (DEV, assert_dsink, assert_grad, assert_lse, assert_out, dev, host,
                         oracle_kwargs, prefill_args, tol_for)

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)


def _churn(nbytes, rounds=6):
    """Allocate and fill buffers on the current stream (would reuse a freed
    workspace of the side stream's call if the allocator allowed it)."""
    keep = []
    for r in range(rounds):
        t = torch.empty(nbytes // 4 + 1024 * r, dtype=torch.float32, device=DEV)
        t.fill_(float("nan"))
        keep.append(t)
    return keep


def test_side_stream_bwd():
    wl = W.make_prefill("side_bwd", [1500, 700], 8, 2, 128, n_sink=4, window=300, seed=21)
    _announce("bwd on a side stream")
    q, k, v, cu, bi, sink = prefill_args(wl)
    do = dev(wl.do, wl.dtype)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse, s = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink, stream=side)
    dq, dk, dv, dsink = sa.bwd(q, k, v, o, lse, do, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window,
                               bi, sink, stream=side)
    junk = _churn(64 << 20)
    torch.cuda.synchronize()
    del junk
    kw = oracle_kwargs(wl)
    rdq, rdk, rdv, rds = oracle.bwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, wl.do.f32, **kw)
    tol = tol_for(wl.dtype)
    assert_grad(host(dq), rdq, tol, "dQ")
    assert_grad(host(dk), rdk, tol, "dK")
    assert_grad(host(dv), rdv, tol, "dV")
    assert_dsink(host(dsink), rds, tol)


SCHEDULE_CASES = {
    # whole key tiles only: every output is written in a fixed order
    "window": dict(lengths=(1500, 700), hq=8, hkv=2, n_sink=4, window=300),
    # key tiles split over several work items (float32 partials added
    # atomically) and block lists
    "blocks_split": dict(lengths=(2600, 130), hq=16, hkv=2, block_lists=dict(n_random=5)),
}


@pytest.mark.parametrize("name", sorted(SCHEDULE_CASES))
def test_bwd_two_streams_match_one(name, monkeypatch):
    """The backward runs dQ on the library's second stream beside dK/dV on the
    caller's; SINK_ATTN_SERIAL_BWD=1 runs both on the caller's stream.  The
    kernels are the same, so dQ and dsink (fixed-order writes) are
    bit-identical, and dK/dV too where no key tile is split; every output also
    matches the oracle.  Run on a side stream of the caller's, with allocations
    on the current stream meanwhile."""
    _announce(f"bwd two streams vs one {name}")
    c = dict(SCHEDULE_CASES[name])
    wl = W.make_prefill(name, c.pop("lengths"), c.pop("hq"), c.pop("hkv"), 128, seed=23, **c)
    q, k, v, cu, bi, sink = prefill_args(wl)
    do = dev(wl.do, wl.dtype)
    args = (cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink)
    o, lse, s = sa.fwd(q, k, v, *args)
    outs = {}
    for mode in ("two", "one", "two"):
        if mode == "one":
            monkeypatch.setenv("SINK_ATTN_SERIAL_BWD", "1")
        else:
            monkeypatch.delenv("SINK_ATTN_SERIAL_BWD", raising=False)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        got = sa.bwd(q, k, v, o, lse, do, *args, stream=side)
        junk = _churn(16 << 20)
        torch.cuda.synchronize()
        del junk
        outs.setdefault(mode, []).append([t.clone() for t in got])
    monkeypatch.delenv("SINK_ATTN_SERIAL_BWD", raising=False)
    one = outs["one"][0]
    atomic = "split" in name
    for two in outs["two"]:
        for nm, a, b in zip(("dq", "dk", "dv", "dsink"), two, one):
            if atomic and nm in ("dk", "dv"):
                assert torch.allclose(a.float(), b.float(), rtol=2.0 ** -7, atol=1e-3), nm
            else:
                assert torch.equal(a, b), f"{nm} differs between the schedules"
    kw = oracle_kwargs(wl)
    rdq, rdk, rdv, rds = oracle.bwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, wl.do.f32, **kw)
    tol = tol_for(wl.dtype)
    dq, dk, dv, dsink = outs["two"][1]
    assert_grad(host(dq), rdq, tol, "dQ")
    assert_grad(host(dk), rdk, tol, "dK")
    assert_grad(host(dv), rdv, tol, "dV")
    assert_dsink(host(dsink), rds, tol)


def test_bwd_concurrent_threads():
    """Two host threads call the backward at once, each on its own stream and
    with its own inputs (ctypes releases the GIL during the call), so their
    calls contend for the device's second stream and its events: every result
    equals the same call made alone (the window case has no split key tiles,
    so every output is written in a fixed order)."""
    import threading
    _announce("bwd from two threads at once")
    cases = []
    for i, lengths in enumerate(((1500, 700), (900, 1300, 260))):
        wl = W.make_prefill(f"thr{i}", list(lengths), 8, 2, 128, n_sink=4, window=300, seed=31 + i)
        q, k, v, cu, bi, sink = prefill_args(wl)
        do = dev(wl.do, wl.dtype)
        args = (cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink)
        o, lse, _ = sa.fwd(q, k, v, *args)
        ref = [t.clone() for t in sa.bwd(q, k, v, o, lse, do, *args)]
        cases.append((q, k, v, o, lse, do, args, ref))
    torch.cuda.synchronize()
    errors = []

    def worker(c):
        q, k, v, o, lse, do, args, ref = c
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.default_stream())
        try:
            for _ in range(6):
                got = sa.bwd(q, k, v, o, lse, do, *args, stream=st)
                st.synchronize()
                for nm, a, b in zip(("dq", "dk", "dv", "dsink"), got, ref):
                    if not torch.equal(a, b):
                        errors.append(f"{nm} differs")
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors[:4]


def test_side_stream_kvcache_decode():
    _announce("cache decode on a side stream")
    rng = np.random.default_rng(5)
    B, n_sink, win, hkv, hq, d = 6, 4, 400, 2, 16, 128
    cache = sa.KvCache(B, n_sink, win, hkv, d)
    kn = torch.from_numpy(rng.standard_normal((B, 300, hkv, d)).astype(np.float32)).to(DEV).bfloat16()
    vn = torch.from_numpy(rng.standard_normal((B, 300, hkv, d)).astype(np.float32)).to(DEV).bfloat16()
    seen = torch.zeros(B, dtype=torch.int32, device=DEV)
    sa.kvcache_append(cache, kn, vn, seen)
    q = torch.from_numpy(rng.standard_normal((B, hq, d)).astype(np.float32)).to(DEV).bfloat16()
    nt = torch.full((B,), 300, dtype=torch.int32, device=DEV)
    sink = torch.from_numpy(rng.standard_normal(hq).astype(np.float32)).to(DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse, s = sa.kvcache_decode(cache, q, nt, None, sink, num_splits=3, stream=side)
    junk = _churn(8 << 20)
    torch.cuda.synchronize()
    del junk
    kc = cache.k.float().cpu().numpy()[:, :n_sink + 296]
    vc = cache.v.float().cpu().numpy()[:, :n_sink + 296]
    ro, rl, rs = oracle.decode(q.float().cpu().numpy(), kc, vc, 1.0 / np.sqrt(d),
                               sink=sink.cpu().numpy())
    tol = tol_for("bf16")
    assert_out(host(o), ro, tol)
    assert_lse(host(lse), rl, tol["lse"])
    assert float(np.max(np.abs(host(s) - rs))) <= tol["s"]


def test_debug_checks_on_device_inputs(monkeypatch):
    """SINK_ATTN_DEBUG=1: valid device inputs run as before; a broken
    cu_seqlens is reported before anything is launched."""
    monkeypatch.setenv("SINK_ATTN_DEBUG", "1")
    wl = W.make_prefill("debug", [130, 64], 4, 2, 128, n_sink=4, window=50, seed=2)
    _announce("debug checks")
    q, k, v, cu, bi, sink = prefill_args(wl)
    o, lse, s = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.fwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, **oracle_kwargs(wl))
    assert_out(host(o), ro, tol_for("bf16"))
    bad = torch.tensor([0, 140, 120], dtype=torch.int32, device=DEV)
    with pytest.raises(sa.SinkAttnError, match="decreases"):
        sa.fwd(q[:120], k[:120], v[:120], bad, 140, wl.scale, wl.n_sink, wl.window, None, sink)
    with pytest.raises(sa.SinkAttnError, match="cache_seqlens"):
        kc = torch.zeros((2, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
        sa.decode(q[:2], kc, kc, torch.tensor([3, 17], dtype=torch.int32, device=DEV))
