"""Parity at the full benchmark sizes, in the launch configuration bench.py
times: the HIP path on the whole workload, compared with the float64 oracle on
sampled output rows it computes one by one, and with properties that hold at
any size (valid-set counts with Q = 0; dsink as a sum of per-row terms)."""
import numpy as np
import pytest
import torch

import oracle
import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import (DEV, TOL_BF16, assert_dsink_per_head, assert_grad, assert_lse, dev,
                         dsink_storage_floor, host)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _announce(name):
    print(f"[case] {name}", flush=True)


def _sample_rows(wl, n, seed):
    """Sampled (token, head) pairs: random ones plus every sample's first and
    last token, and the ragged tail of the packed tensor."""
    rng = np.random.default_rng(seed)
    rows = [(int(t), int(h)) for t, h in zip(rng.integers(0, wl.total, n), rng.integers(0, wl.hq, n))]
    for b in range(wl.batch):
        t0, t1 = int(wl.cu_seqlens[b]), int(wl.cu_seqlens[b + 1])
        rows += [(t0, int(rng.integers(wl.hq))), (t1 - 1, int(rng.integers(wl.hq)))]
    rows.append((wl.total - 1, wl.hq - 1))
    return rows


def _dev_args(wl):
    q, k, v = dev(wl.q, "bf16"), dev(wl.k, "bf16"), dev(wl.v, "bf16")
    cu = torch.from_numpy(wl.cu_seqlens).to(DEV)
    bi = torch.from_numpy(wl.block_indices).to(DEV) if wl.block_indices is not None else None
    sink = torch.from_numpy(wl.sink).to(DEV) if wl.sink is not None else None
    return q, k, v, cu, bi, sink


def _check_fwd_rows(wl, o, lse, s, rows):
    kw = dict(n_sink=wl.n_sink, window=wl.window, block_indices=wl.block_indices,
              block_size=wl.block_size, sink=wl.sink)
    ro, rl, rs = oracle.fwd_rows(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, rows, **kw)
    ho, hl, hs = host(o), host(lse), host(s)
    got_o = np.stack([ho[t, h] for t, h in rows])
    err = np.abs(got_o - ro)
    assert err.max() <= TOL_BF16["o_max"], f"O max err {err.max():.3e}"
    assert err.mean() <= TOL_BF16["o_mean"], f"O mean err {err.mean():.3e}"
    assert_lse(np.array([hl[t, h] for t, h in rows]), rl, TOL_BF16["lse"])
    assert np.max(np.abs(np.array([hs[t, h] for t, h in rows]) - rs)) <= TOL_BF16["s"]


def _dsink_property(wl, o, lse, do, dsink):
    """dsink_h = -sum_i Delta_ih p_sink_ih with Delta from the kernel's own bf16
    O and dO and p_sink = sigma(a_h - L_orig), in float64 on the host."""
    O = host(o)
    dO = host(do)
    L = host(lse)
    delta = np.einsum("thd,thd->th", O, dO)
    a = wl.sink.astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        p_sink = 1.0 / (1.0 + np.exp(L - a))
    want = -np.sum(delta * p_sink, axis=0)
    got = host(dsink)
    rel = np.max(np.abs(got - want)) / np.max(np.abs(want))
    assert rel <= 1e-3, f"dsink vs its per-row terms: rel err {rel:.3e}"


def test_gqa_prefill_full():
    wl = W.gqa_prefill()
    _announce("gqa prefill fwd full")
    q, k, v, cu, bi, sink = _dev_args(wl)
    o, lse, s = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, None, sink)
    torch.cuda.synchronize()
    _check_fwd_rows(wl, o, lse, s, _sample_rows(wl, 96, 1))


def _check_kv_rows(wl, dk, dv, kv_rows, kw):
    """dK / dV key rows against the oracle, every (query row, head) that sees
    the key summed in float64."""
    rdk, rdv = oracle.bwd_kv_rows(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, wl.do.f32,
                                  kv_rows, **kw)
    hdk, hdv = host(dk), host(dv)
    got_k = np.stack([hdk[t, g] for t, g in kv_rows])
    got_v = np.stack([hdv[t, g] for t, g in kv_rows])
    assert_grad(got_k, rdk, TOL_BF16, f"dK rows {kv_rows}")
    assert_grad(got_v, rdv, TOL_BF16, f"dV rows {kv_rows}")


def _check_dsink_heads(wl, dsink, heads, kw):
    """dsink of whole heads against the oracle's sum over every row of the
    head, head by head (bound: 1e-2 relative plus the bf16 storage of O)."""
    ro, rl, _, _, rds = oracle.fwd_bwd_heads(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale,
                                             wl.do.f32, heads, **kw)
    floor = dsink_storage_floor(ro, wl.do.f32[:, heads], rl, wl.sink[heads], "bf16")
    assert_dsink_per_head(host(dsink)[heads], rds, TOL_BF16, floor)


def test_streaming_prefill_full_fwd_bwd():
    wl = W.streaming_prefill()
    _announce("streaming prefill fwd+bwd full")
    q, k, v, cu, bi, sink = _dev_args(wl)
    do = dev(wl.do, "bf16")
    o, lse, s = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, None, sink)
    dq, dk, dv, dsink = sa.bwd(q, k, v, o, lse, do, cu, wl.max_seqlen, wl.scale, wl.n_sink,
                               wl.window, None, sink)
    torch.cuda.synchronize()
    rows = _sample_rows(wl, 64, 2)
    _check_fwd_rows(wl, o, lse, s, rows)
    kw = dict(n_sink=wl.n_sink, window=wl.window, sink=wl.sink)
    rdq, _, _ = oracle.bwd_rows(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, wl.do.f32,
                                rows[:24], **kw)
    hdq = host(dq)
    assert_grad(np.stack([hdq[t, h] for t, h in rows[:24]]), rdq, TOL_BF16, "dQ rows")
    # Keys: in every sample a kept first token and another key of the first
    # 64-key tile (seen by every query of the sample: the split tiles whose
    # float32 partials are added atomically), plus a window key; and the last
    # key of the packed tensor.
    c = wl.cu_seqlens
    kv_rows = []
    for b in range(wl.batch):
        g = b % wl.hkv
        L = int(c[b + 1] - c[b])
        kv_rows += [(int(c[b]) + b % wl.n_sink, g), (int(c[b]) + 5 + 7 * b, g),
                    (int(c[b]) + L // 2 + b, g)]
    kv_rows.append((int(c[wl.batch]) - 1, wl.hkv - 1))
    _check_kv_rows(wl, dk, dv, kv_rows, kw)
    _dsink_property(wl, o, lse, do, dsink)
    _check_dsink_heads(wl, dsink, [3, 30], kw)


def test_streaming_prefill_full_visited_counts():
    """Q = 0: e^{lse} equals the closed-form size of every row's valid set."""
    wl = W.streaming_prefill()
    _announce("streaming prefill q=0 counts full")
    q, k, v, cu, bi, sink = _dev_args(wl)
    q.zero_()
    _, lse, _ = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, None, sink)
    counts = np.exp(host(lse))
    want = np.concatenate([np.minimum(np.arange(L) + 1, 1024 + np.minimum(4, np.maximum(0, np.arange(L) + 1 - 1024)))
                           for L in wl.lengths]).astype(np.float64)
    np.testing.assert_allclose(counts, np.repeat(want[:, None], wl.hq, 1), rtol=4e-6)


def test_block_sparse_full_fwd_bwd():
    wl = W.block_sparse()
    _announce("block sparse fwd+bwd full")
    q, k, v, cu, bi, sink = _dev_args(wl)
    do = dev(wl.do, "bf16")
    o, lse, s = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, bi, sink)
    dq, dk, dv, dsink = sa.bwd(q, k, v, o, lse, do, cu, wl.max_seqlen, wl.scale, 0, 0, bi, sink)
    torch.cuda.synchronize()
    rows = _sample_rows(wl, 48, 3)
    _check_fwd_rows(wl, o, lse, s, rows)
    kw = dict(block_indices=wl.block_indices, block_size=64, sink=wl.sink)
    rdq, _, _ = oracle.bwd_rows(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, wl.do.f32,
                                rows[:16], **kw)
    hdq = host(dq)
    assert_grad(np.stack([hdq[t, h] for t, h in rows[:16]]), rdq, TOL_BF16, "dQ rows")
    # Keys: block 0 of every sample (selected by every query block: the most
    # split key tiles) and keys of randomly selected blocks, one KV head per
    # sample.
    c = wl.cu_seqlens
    kv_rows = []
    for b in range(wl.batch):
        g = (2 * b + 1) % wl.hkv
        kv_rows += [(int(c[b]), g), (int(c[b]) + 37, g), (int(c[b]) + 63, g),
                    (int(c[b]) + 64 * (60 + 50 * b) + 5 * b, g), (int(c[b]) + 64 * (250 - 3 * b) + 63, g)]
    _check_kv_rows(wl, dk, dv, kv_rows, kw)
    _dsink_property(wl, o, lse, do, dsink)
    _check_dsink_heads(wl, dsink, [7, 60], kw)


def test_block_sparse_full_visited_counts():
    """Q = 0 with the full block lists: e^{lse} = 64 min(16, qb) + r + 1."""
    wl = W.block_sparse()
    _announce("block sparse q=0 counts full")
    q, k, v, cu, bi, sink = _dev_args(wl)
    q.zero_()
    _, lse, _ = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, bi, sink)
    counts = np.exp(host(lse))
    L = int(wl.lengths[0])
    r = np.arange(L)
    per = (64 * np.minimum(16, r // 64) + r % 64 + 1).astype(np.float64)
    np.testing.assert_allclose(counts, np.repeat(np.tile(per, wl.batch)[:, None], wl.hq, 1), rtol=4e-6)


def test_streaming_decode_full():
    wl = W.streaming_decode()
    _announce("streaming decode full")
    q = dev(wl.q, "bf16")
    kc, vc = dev(wl.k_cache, "bf16"), dev(wl.v_cache, "bf16")
    sink = torch.from_numpy(wl.sink).to(DEV)
    o, lse, s = sa.decode(q, kc, vc, None, wl.scale, sink)
    torch.cuda.synchronize()
    ho, hl, hs = host(o), host(lse), host(s)
    for b in (0, 37, 64, 127):
        ro, rl, rs = oracle.decode(wl.q.f32[b:b + 1], wl.k_cache.f32[b:b + 1], wl.v_cache.f32[b:b + 1],
                                   wl.scale, sink=wl.sink)
        err = np.abs(ho[b] - ro[0])
        assert err.max() <= TOL_BF16["o_max"] and err.mean() <= TOL_BF16["o_mean"]
        assert_lse(hl[b], rl[0], TOL_BF16["lse"])
        assert np.max(np.abs(hs[b] - rs[0])) <= TOL_BF16["s"]
