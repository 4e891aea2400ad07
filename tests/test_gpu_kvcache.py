"""GPU parity of the rolling KV cache ("What is Attention Sink? ...
StreamingLLM" (model.playoffer.cn), core idea and engineering notes;
"Attention Sink" (lijianxiong.space), H2O circular queue): appends bit for bit
against the oracle's placement and 8-bit quantisation, and decode over the
bf16 and the 8-bit cache against the oracle's decode of the same slots."""
import numpy as np
import pytest
import torch

import streamingllm_sink_attn_amd as sa
from oracle import kvcache_oracle as KO
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import DEV, TOL_BF16, assert_lse, host

pytestmark = pytest.mark.gpu


def _bf16(rng, shape, scale=1.0):
    """bf16-exact float32 values and the matching device tensor."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    t = torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    return t.float().cpu().numpy(), t


def _state(cache):
    """Device cache arrays as numpy (bf16 as float32)."""
    if not cache.quantized:
        return dict(k=host(cache.k.float()), v=host(cache.v.float()))
    return dict(sink_k=host(cache.sink_k.float()), sink_v=host(cache.sink_v.float()),
                win_k=host(cache.win_k), win_v=host(cache.win_v),
                win_k_scale=host(cache.win_k_scale), win_v_scale=host(cache.win_v_scale))


def _stream(rng, B, hkv, d, n_sink, window, quantized, chunks, start=None, kscale=1.0):
    """Append the chunks on the GPU and in the oracle; compare after each."""
    cache = sa.KvCache(B, n_sink, window, hkv, d, quantized)
    ref = KO.new_cache(B, n_sink, window, hkv, d, quantized)
    seen = np.zeros(B, np.int32) if start is None else np.array(start, np.int32)
    toks = []
    for c in chunks:
        k, kt = _bf16(rng, (B, c, hkv, d), kscale)
        v, vt = _bf16(rng, (B, c, hkv, d))
        sa.kvcache_append(cache, kt, vt, torch.from_numpy(seen).to(DEV))
        torch.cuda.synchronize()
        KO.append(ref, k, v, seen, n_sink, window)
        got = _state(cache)
        for key, want in ref.items():
            if key == "quantized":
                continue
            assert np.array_equal(got[key], want), f"{key} differs after chunk {c}"
        seen = seen + c
        toks.append((k, v))
    return cache, ref, seen


@pytest.mark.parametrize("quantized", [False, True])
@pytest.mark.parametrize("n_sink,window,chunks", [(4, 40, [1, 7, 33, 2, 90, 1]), (0, 32, [5, 64]),
                                                  (6, 17, [3, 3, 40])])
def test_append_bit_exact(quantized, n_sink, window, chunks):
    print(f"[case] kvcache append q={quantized} {n_sink} {window} {chunks}", flush=True)
    rng = np.random.default_rng(11)
    _stream(rng, 3, 2, 128, n_sink, window, quantized, chunks, kscale=3.0)


def test_append_small_head_dim_and_offset_streams():
    """bf16 layout with D = 64 and sequences at different stream positions."""
    print("[case] kvcache append d64 offsets", flush=True)
    rng = np.random.default_rng(12)
    _stream(rng, 4, 1, 64, 4, 20, False, [5, 30, 2], start=[0, 3, 100, 17])


def _check_decode(cache, ref, seen, n_sink, window, hq, splits, rng, sink=True):
    B = cache.batch
    q, qt = _bf16(rng, (B, hq, cache.d))
    a = rng.standard_normal(hq).astype(np.float32) if sink else None
    at = torch.from_numpy(a).to(DEV) if sink else None
    nt = torch.from_numpy(np.asarray(seen, np.int32)).to(DEV)
    o, lse, s = sa.kvcache_decode(cache, qt, nt, 0.11, at, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl, rs = KO.cache_decode(q, ref, seen, n_sink, window, 0.11, sink=a)
    err = np.abs(host(o.float()) - ro)
    assert err.max() <= TOL_BF16["o_max"], f"O max err {err.max():.3e}"
    assert err.mean() <= TOL_BF16["o_mean"]
    assert_lse(host(lse), rl, TOL_BF16["lse"])
    assert np.max(np.abs(host(s) - rs)) <= TOL_BF16["s"]


@pytest.mark.parametrize("quantized", [False, True])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_over_cache(quantized, splits):
    print(f"[case] kvcache decode q={quantized} splits={splits}", flush=True)
    rng = np.random.default_rng(13)
    n_sink, window = 4, 300
    # fill levels: first tokens only, a partly filled ring, a wrapped ring
    for chunks in ([3], [3, 40], [3, 40, 280, 150]):
        cache, ref, seen = _stream(rng, 4, 2, 128, n_sink, window, quantized, chunks)
        _check_decode(cache, ref, seen, n_sink, window, 16, splits, rng)
    # shorter streams than written: the valid slots are the first
    # min(n, n_sink) first-token slots and the first ring slots
    _check_decode(cache, ref, np.array([2, 4, 10, 200], np.int32), n_sink, window, 16, splits, rng,
                  sink=False)


@pytest.mark.parametrize("quantized", [False, True])
def test_decode_over_cache_without_first_tokens(quantized):
    """n_sink = 0: the cache is the ring alone (no first-token chunk)."""
    print(f"[case] kvcache decode n_sink=0 q={quantized}", flush=True)
    rng = np.random.default_rng(16)
    for chunks in ([3], [50, 90]):
        cache, ref, seen = _stream(rng, 2, 2, 128, 0, 64, quantized, chunks)
        for splits in (0, 3):
            _check_decode(cache, ref, seen, 0, 64, 8, splits, rng)


@pytest.mark.parametrize("quantized", [False, True])
def test_decode_over_cache_odd_window_and_groups(quantized):
    """A ring length that is not a multiple of 4 (the 8-bit decode then reads
    scales one slot at a time), 5 first tokens, and 3 query heads per KV head."""
    print(f"[case] kvcache decode odd window q={quantized}", flush=True)
    rng = np.random.default_rng(15)
    n_sink, window = 5, 301
    for chunks in ([4], [9, 100], [9, 100, 400]):
        cache, ref, seen = _stream(rng, 3, 2, 128, n_sink, window, quantized, chunks)
        for splits in (0, 2):
            _check_decode(cache, ref, seen, n_sink, window, 6, splits, rng)


@pytest.mark.parametrize("quantized", [False, True])
def test_decode_ignores_unwritten_slots(quantized):
    """Ring slots not yet written may hold anything: NaN codes, values and
    scales there change nothing."""
    print(f"[case] kvcache unwritten slots q={quantized}", flush=True)
    rng = np.random.default_rng(14)
    n_sink, window = 4, 300
    cache, ref, seen = _stream(rng, 3, 2, 128, n_sink, window, quantized, [3, 40])
    nw = int(seen[0]) - n_sink                       # ring slots written so far (same for all)
    if not quantized:
        cache.k[:, n_sink + nw:] = float("nan")
        cache.v[:, n_sink + nw:] = float("nan")
    else:
        cache.win_k[:, nw:] = 0x7F                   # the e4m3 NaN code
        cache.win_v[:, nw:] = 0x7F
        cache.win_k_scale[:, :, nw:] = float("nan")
        cache.win_v_scale[:, :, nw:] = float("inf")
    for splits in (0, 1, 3):
        _check_decode(cache, ref, seen, n_sink, window, 16, splits, rng)


@pytest.mark.timeout(600)
def test_decode_q8_fullsize_sampled():
    """128 sequences x (4 first tokens + 4092-token 8-bit ring), Hq=64,
    Hkv=8: the bench workload, filled with random codes and scales, checked
    on sampled sequences against the oracle's decode of the dequantised
    slots."""
    print("[case] kvcache q8 fullsize", flush=True)
    B, n_sink, window, hq, hkv, d = 128, 4, 4092, 64, 8, 128
    wl = W.kvcache_q8_decode(B, n_sink, window, hq, hkv, d, seed=3)
    cache = sa.KvCache(B, n_sink, window, hkv, d, quantized=True)
    cache.sink_k.copy_(torch.from_numpy(wl.sink_k).to(torch.bfloat16))
    cache.sink_v.copy_(torch.from_numpy(wl.sink_v).to(torch.bfloat16))
    cache.win_k.copy_(torch.from_numpy(wl.win_k))
    cache.win_v.copy_(torch.from_numpy(wl.win_v))
    cache.win_k_scale.copy_(torch.from_numpy(wl.win_k_scale))
    cache.win_v_scale.copy_(torch.from_numpy(wl.win_v_scale))
    qt = torch.from_numpy(wl.q).to(DEV).to(torch.bfloat16)
    nt = torch.from_numpy(wl.n_tokens).to(DEV)
    at = torch.from_numpy(wl.sink).to(DEV)
    o, lse, s = sa.kvcache_decode(cache, qt, nt, wl.scale, at)
    torch.cuda.synchronize()
    ho, hl, hs = host(o.float()), host(lse), host(s)
    q = qt.float().cpu().numpy()
    for b in (0, 1, 77, 127):
        one = {key: (val[b:b + 1] if isinstance(val, np.ndarray) else val)
               for key, val in dict(quantized=True, sink_k=wl.sink_k, sink_v=wl.sink_v, win_k=wl.win_k,
                                    win_v=wl.win_v, win_k_scale=wl.win_k_scale,
                                    win_v_scale=wl.win_v_scale).items()}
        ro, rl, rs = KO.cache_decode(q[b:b + 1], one, wl.n_tokens[b:b + 1], n_sink, window, wl.scale,
                                     sink=wl.sink)
        err = np.abs(ho[b] - ro[0])
        assert err.max() <= TOL_BF16["o_max"], f"seq {b}: O max err {err.max():.3e}"
        assert_lse(hl[b], rl[0], TOL_BF16["lse"])
        assert np.max(np.abs(hs[b] - rs[0])) <= TOL_BF16["s"]


# ---------------------------------------------------------------------------
# Chunked prefill against the cache
# ---------------------------------------------------------------------------

def _check_prefill_rows(got, want, rows=None):
    o, lse, s = (host(x.float()) if x.dtype == torch.bfloat16 else host(x) for x in got)
    ro, rl, rs = want
    if rows is not None:
        idx = tuple(np.array(rows).T)
        o, lse, s, ro, rl, rs = o[idx], lse[idx], s[idx], ro[idx], rl[idx], rs[idx]
    err = np.abs(o - ro)
    assert err.max() <= TOL_BF16["o_max"], f"O max err {err.max():.3e}"
    assert err.mean() <= TOL_BF16["o_mean"]
    assert_lse(lse, rl, TOL_BF16["lse"])
    assert np.max(np.abs(s - rs)) <= TOL_BF16["s"]


def _prefill_stream(rng, B, hq, hkv, d, n_sink, window, quantized, chunks, start=None, sink=True):
    """Each chunk: prefill against the cache (GPU and oracle, compared), then
    append it to both caches."""
    cache = sa.KvCache(B, n_sink, window, hkv, d, quantized)
    ref = KO.new_cache(B, n_sink, window, hkv, d, quantized)
    seen = np.zeros(B, np.int32) if start is None else np.array(start, np.int32)
    a = rng.standard_normal(hq).astype(np.float32) if sink else None
    at = torch.from_numpy(a).to(DEV) if sink else None
    for c in chunks:
        q, qt = _bf16(rng, (B, c, hq, d))
        k, kt = _bf16(rng, (B, c, hkv, d), 0.7)
        v, vt = _bf16(rng, (B, c, hkv, d))
        st = torch.from_numpy(seen).to(DEV)
        got = sa.kvcache_prefill(cache, qt, kt, vt, st, 0.09, at)
        torch.cuda.synchronize()
        _check_prefill_rows(got, KO.cache_prefill(q, ref, k, v, seen, n_sink, window, 0.09, sink=a))
        sa.kvcache_append(cache, kt, vt, st)
        KO.append(ref, k, v, seen, n_sink, window)
        seen = seen + c
    return cache, ref, seen


@pytest.mark.parametrize("quantized", [False, True])
@pytest.mark.parametrize("n_sink,window,chunks,start", [(4, 40, [1, 7, 33, 2, 90, 1], [0, 3, 50]),
                                                        (0, 32, [5, 64], None),
                                                        (6, 17, [3, 3, 40], [0, 0, 9])])
def test_prefill_over_cache(quantized, n_sink, window, chunks, start):
    print(f"[case] kvcache prefill q={quantized} {n_sink} {window} {chunks} {start}", flush=True)
    rng = np.random.default_rng(21)
    _prefill_stream(rng, 3, 8, 2, 128, n_sink, window, quantized, chunks, start)


@pytest.mark.parametrize("n_sink,window,chunks,start", [(70, 200, [150, 70, 64, 300], [0, 77, 500]),
                                                        (0, 256, [64, 200, 129, 511], [0, 3, 1000]),
                                                        (4, 130, [64, 1, 127, 130], [2, 66, 131])])
def test_prefill_over_cache_tiles_in_place(n_sink, window, chunks, start):
    """bf16 cache, D = 128: key tiles read from the cache and the chunk where
    they lie (first tokens over more than one tile, ring runs before and
    after the wrap, chunk runs) and seam tiles staged, at several ring
    offsets per stream."""
    print(f"[case] kvcache prefill in place {n_sink} {window} {chunks} {start}", flush=True)
    rng = np.random.default_rng(26)
    _prefill_stream(rng, 3, 8, 2, 128, n_sink, window, False, chunks, start)


@pytest.mark.parametrize("quantized", [False, True])
def test_prefill_over_cache_three_heads_per_group(quantized):
    """3 query heads per KV head (one head per workgroup, 256-row position
    tiles) and an odd window."""
    print(f"[case] kvcache prefill G=3 q={quantized}", flush=True)
    rng = np.random.default_rng(24)
    _prefill_stream(rng, 2, 6, 2, 128, 5, 301, quantized, [7, 300, 260], start=[0, 40])


def test_prefill_over_cache_d64_and_no_sink():
    """bf16 layout with D = 64 (the generic forward) and without a sink."""
    print("[case] kvcache prefill d64 / no sink", flush=True)
    rng = np.random.default_rng(22)
    _prefill_stream(rng, 2, 4, 1, 64, 4, 20, False, [5, 30, 2], start=[0, 11])
    _prefill_stream(rng, 2, 8, 2, 128, 4, 20, False, [9, 30], sink=False)


@pytest.mark.timeout(600)
def test_prefill_fullsize_sampled():
    """8 streams x 1024-token chunks against (4 + 1024)-slot caches, Hq=32,
    Hkv=8: the bench workload, checked on sampled rows."""
    print("[case] kvcache prefill fullsize", flush=True)
    wl = W.kvcache_prefill()
    cache = sa.KvCache(wl.batch, wl.n_sink, wl.window, wl.hkv, wl.d, quantized=False)
    cache.k.copy_(torch.from_numpy(wl.k_cache).to(torch.bfloat16))
    cache.v.copy_(torch.from_numpy(wl.v_cache).to(torch.bfloat16))
    dev_ = lambda x: torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    got = sa.kvcache_prefill(cache, dev_(wl.q), dev_(wl.k_new), dev_(wl.v_new),
                             torch.from_numpy(wl.n_seen).to(DEV), wl.scale, torch.from_numpy(wl.sink).to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(23)
    rows = [(int(b), int(c)) for b, c in zip(rng.integers(0, wl.batch, 10), rng.integers(0, wl.chunk, 10))]
    rows += [(0, 0), (wl.batch - 1, wl.chunk - 1), (3, 63), (3, 64)]
    ref = dict(quantized=False, k=wl.k_cache, v=wl.v_cache)
    want = KO.cache_prefill(wl.q, ref, wl.k_new, wl.v_new, wl.n_seen, wl.n_sink, wl.window, wl.scale,
                            sink=wl.sink, rows=rows)
    _check_prefill_rows(got, want, rows)


@pytest.mark.timeout(600)
def test_prefill_fullsize_q8_sampled():
    """The bench's chunked prefill against the 8-bit cache (random e4m3 ring
    codes, row scales of unit-normal size, the same chunk), sampled rows."""
    print("[case] kvcache prefill fullsize q8", flush=True)
    wl = W.kvcache_prefill()
    rng = np.random.default_rng(25)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ref = KO.new_cache(wl.batch, wl.n_sink, wl.window, wl.hkv, wl.d, quantized=True)
    ref["sink_k"][:] = wl.k_cache[:, :wl.n_sink]
    ref["sink_v"][:] = wl.v_cache[:, :wl.n_sink]
    for name in ("win_k", "win_v"):
        ref[name][:] = finite[rng.integers(0, len(finite), size=ref[name].shape)]
    for name in ("win_k_scale", "win_v_scale"):
        ref[name][:] = (rng.uniform(2.0, 4.0, size=ref[name].shape) / 448.0).astype(np.float32)
    cache = sa.KvCache(wl.batch, wl.n_sink, wl.window, wl.hkv, wl.d, quantized=True)
    for name in ("sink_k", "sink_v"):
        getattr(cache, name).copy_(torch.from_numpy(ref[name]).to(torch.bfloat16))
    for name in ("win_k", "win_v", "win_k_scale", "win_v_scale"):
        getattr(cache, name).copy_(torch.from_numpy(ref[name]))
    dev_ = lambda x: torch.from_numpy(x).to(DEV).to(torch.bfloat16)
    got = sa.kvcache_prefill(cache, dev_(wl.q), dev_(wl.k_new), dev_(wl.v_new),
                             torch.from_numpy(wl.n_seen).to(DEV), wl.scale, torch.from_numpy(wl.sink).to(DEV))
    torch.cuda.synchronize()
    rows = [(int(b), int(c)) for b, c in zip(rng.integers(0, wl.batch, 8), rng.integers(0, wl.chunk, 8))]
    rows += [(0, 0), (wl.batch - 1, wl.chunk - 1)]
    want = KO.cache_prefill(wl.q, ref, wl.k_new, wl.v_new, wl.n_seen, wl.n_sink, wl.window, wl.scale,
                            sink=wl.sink, rows=rows)
    _check_prefill_rows(got, want, rows)


@pytest.mark.parametrize("d", [128, 64])
def test_cache_calls_without_s(d):
    """s is optional (a NULL pointer at the C ABI): the other outputs are the
    same bits with and without it, for chunked prefill (the matrix-core and
    the generic forward) and decode."""
    print(f"[case] kvcache calls without s d={d}", flush=True)
    rng = np.random.default_rng(26)
    B, hq, hkv, n_sink, window, C = 2, 4, 2, 4, 40, 30
    cache = sa.KvCache(B, n_sink, window, hkv, d, quantized=False)
    seen = torch.tensor([5, 70], dtype=torch.int32, device=DEV)
    _, kt = _bf16(rng, (B, 80, hkv, d))
    _, vt = _bf16(rng, (B, 80, hkv, d))
    sa.kvcache_append(cache, kt, vt, torch.zeros_like(seen))
    _, qt = _bf16(rng, (B, C, hq, d))
    _, knt = _bf16(rng, (B, C, hkv, d))
    _, vnt = _bf16(rng, (B, C, hkv, d))
    sink = torch.from_numpy(rng.standard_normal(hq).astype(np.float32)).to(DEV)
    o1, l1, s1 = sa.kvcache_prefill(cache, qt, knt, vnt, seen, 0.1, sink)
    o2, l2, s2 = sa.kvcache_prefill(cache, qt, knt, vnt, seen, 0.1, sink, return_s=False)
    assert s2 is None and s1 is not None
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    if d == 128:
        _, q1 = _bf16(rng, (B, hq, d))
        a = sa.kvcache_decode(cache, q1, seen, 0.1, sink)
        b = sa.kvcache_decode(cache, q1, seen, 0.1, sink, return_s=False)
        assert b[2] is None and torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Seeded random streams: every call of the cache API on one stream
# ---------------------------------------------------------------------------

def _random_stream_case(i):
    rng = np.random.default_rng(9100 + i)
    quantized = bool(i % 2)
    B = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2, 3, 4, 8]))
    d = 128 if quantized else int(rng.choice([128, 128, 64]))
    n_sink = int(rng.choice([0, 1, 3, 4, 6, 64]))
    window = int(rng.integers(1, 301))
    chunks = [int(x) for x in rng.integers(1, 201, size=int(rng.integers(1, 5)))]
    start = [int(x) for x in rng.integers(0, 501, size=B)] if rng.random() < 0.5 else None
    return rng, quantized, B, hkv * G, hkv, d, n_sink, window, chunks, start


@pytest.mark.parametrize("i", range(12))
def test_random_streams(i):
    """Random cache shapes and chunk sequences: each chunk's prefill against
    the cache and its append compared with the oracle, then a decode over
    the final cache with a random split count."""
    rng, quantized, B, hq, hkv, d, n_sink, window, chunks, start = _random_stream_case(i)
    print(f"[case] kvcache random stream {i}: q={quantized} B={B} hq={hq} hkv={hkv} d={d} "
          f"n_sink={n_sink} window={window} chunks={chunks} start={start}", flush=True)
    cache, ref, seen = _prefill_stream(rng, B, hq, hkv, d, n_sink, window, quantized, chunks, start)
    _check_decode(cache, ref, seen, n_sink, window, hq, int(rng.choice([0, 1, 3])), rng)
