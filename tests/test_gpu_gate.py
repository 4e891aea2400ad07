"""GPU parity of the gate statistics ("Paper notes: Attention Sink and the
native MoE in attention layers", s2, s4, s5): the first-token gate of
sink_attn_fwd_gated against the float64 oracle, the gated call's other outputs
against the plain forward (bit for bit), and the head importance against the
mean of the same gate."""
import numpy as np
import pytest
import torch

import oracle
import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import DEV, dev, host, prefill_args, run_fwd

pytestmark = pytest.mark.gpu

GATE_TOL = 1e-3          # the gate is a share of the softmax, like s
IMP_TOL = 1e-5           # importance of the kernel's own gate: a float32 sum of T rows

CASES = {
    "dense_g4": dict(lengths=(200, 64, 1, 129), hq=8, hkv=2),
    "dense_g16": dict(lengths=(140, 33), hq=32, hkv=2),
    "window_sink4": dict(lengths=(400, 77, 260), hq=8, hkv=2, n_sink=4, window=100),
    # no kept first token: rows past the window cannot see it (gate 1)
    "window_nosinktok": dict(lengths=(333,), hq=4, hkv=1, n_sink=0, window=50),
    "window_one": dict(lengths=(200, 65), hq=4, hkv=1, n_sink=4, window=1),
    "blocks_g4": dict(lengths=(700, 130), hq=8, hkv=2, block_lists=dict(n_random=3)),
    # block 0 not always selected: rows without the first key
    "blocks_nodiag": dict(lengths=(300,), hq=4, hkv=1,
                          block_lists=dict(n_random=2, diagonal=False, always_first=False)),
    "stress_sink": dict(lengths=(260,), hq=4, hkv=1, n_sink=4, window=64, sink_shift=4.0),
    "no_sink": dict(lengths=(250, 99), hq=8, hkv=2, sink=False),
    "d64_generic": dict(lengths=(150, 40), hq=4, hkv=2, d=64),
}


def _wl(name):
    c = dict(CASES[name])
    d = c.pop("d", 128)
    return W.make_prefill(name, c.pop("lengths"), c.pop("hq"), c.pop("hkv"), d, seed=5, **c)


def _gate_kwargs(wl):
    return dict(n_sink=wl.n_sink, window=wl.window, block_indices=wl.block_indices,
                block_size=wl.block_size)


def _run_gated(wl):
    q, k, v, cu, bi, sink = prefill_args(wl)
    out = sa.fwd_gated(q, k, v, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink)
    torch.cuda.synchronize()
    return out


def _check(wl):
    o, lse, s, gate = _run_gated(wl)
    # the gate changes nothing else the forward writes
    o1, lse1, s1 = run_fwd(wl)
    assert torch.equal(o, o1) and torch.equal(lse, lse1) and torch.equal(s, s1)
    want = oracle.first_token_gate(wl.q.f32, wl.k.f32, wl.cu_seqlens, wl.scale, **_gate_kwargs(wl))
    got = host(gate).astype(np.float64)
    err = np.abs(got - want)
    assert err.max() <= GATE_TOL, f"gate max err {err.max():.3e}"
    # exact values where the gate is decided by the mask alone
    empty = ~np.isfinite(host(lse))
    assert np.all(got[empty] == 0.0)
    imp = host(sa.head_importance(gate)).astype(np.float64)
    np.testing.assert_allclose(imp, got.mean(axis=0), rtol=IMP_TOL, atol=IMP_TOL)
    assert np.max(np.abs(imp - oracle.head_importance(want))) <= GATE_TOL
    # the sink gate of the same call: importance of s
    imp_s = host(sa.head_importance(s)).astype(np.float64)
    np.testing.assert_allclose(imp_s, host(s).astype(np.float64).mean(axis=0), rtol=IMP_TOL,
                               atol=IMP_TOL)
    return got, want


@pytest.mark.parametrize("name", sorted(CASES))
def test_gate_variants(name):
    print(f"[case] gate {name}", flush=True)
    wl = _wl(name)
    got, _ = _check(wl)
    if name == "window_nosinktok":
        # rows at or past the window see no first token: exactly 1
        assert np.all(got[50:, :] == 1.0)
    # each sample's first query sees only its first key: exactly 0
    for b in range(wl.batch):
        t0 = int(wl.cu_seqlens[b])
        if int(wl.cu_seqlens[b + 1]) > t0 and wl.block_indices is None:
            assert np.all(got[t0, :] == 0.0)


def test_gate_tiny_f32_generic():
    print("[case] gate tiny_f32", flush=True)
    _check(W.tiny_f32())


def test_head_importance_shapes():
    print("[case] head importance shapes", flush=True)
    rng = np.random.default_rng(7)
    for rows, heads in [(1, 1), (63, 5), (64, 300), (1000, 32), (0, 4)]:
        g = torch.from_numpy(rng.random((rows, heads), dtype=np.float32)).to(DEV)
        imp = host(sa.head_importance(g)).astype(np.float64)
        want = oracle.head_importance(host(g))
        np.testing.assert_allclose(imp, want, rtol=1e-5, atol=1e-7)
        # fixed-order reduction: the same bits every call
        assert torch.equal(sa.head_importance(g), sa.head_importance(g))


@pytest.mark.timeout(600)
def test_gate_fullsize_gqa_sampled_rows():
    """The GQA prefill workload (4 x 4096, Hq=32, Hkv=8) in one gated call,
    checked on sampled rows the oracle evaluates one by one."""
    print("[case] gate fullsize gqa", flush=True)
    wl = W.gqa_prefill()
    o, lse, s, gate = _run_gated(wl)
    rng = np.random.default_rng(8)
    rows = [(int(t), int(h)) for t, h in zip(rng.integers(0, wl.total, 200),
                                              rng.integers(0, wl.hq, 200))]
    rows += [(int(wl.cu_seqlens[b]), 3) for b in range(wl.batch)]
    want = oracle.first_token_gate_rows(wl.q.f32, wl.k.f32, wl.cu_seqlens, wl.scale, rows)
    hg = host(gate)
    got = np.array([hg[t, h] for t, h in rows], dtype=np.float64)
    assert np.max(np.abs(got - want)) <= GATE_TOL
    imp = host(sa.head_importance(gate)).astype(np.float64)
    np.testing.assert_allclose(imp, hg.astype(np.float64).mean(axis=0), rtol=IMP_TOL, atol=IMP_TOL)
