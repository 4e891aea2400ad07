"""CPU pins of the rolling KV-cache oracle and its 8-bit window ("What is
Attention Sink? ... StreamingLLM" (model.playoffer.cn), "StreamingLLM core
idea" and "Other engineering implications"; "Attention Sink"
(lijianxiong.space), H2O circular queue).  Each check ties the oracle to the
format's definition, to brute force, or to the prefill oracle's StreamingLLM
mask rather than to itself."""
import numpy as np
import pytest

import oracle
from oracle import kvcache_oracle as KO


# ---------------------------------------------------------------------------
# e4m3: the code table and rounding, from the format's definition
# ---------------------------------------------------------------------------

def test_e4m3_table_landmarks():
    v = KO.e4m3_decode(np.arange(256))
    assert v[0x00] == 0.0 and np.signbit(v[0x80])             # +0 and -0
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0              # largest finite
    assert v[0x08] == 2.0 ** -6                                # smallest normal
    assert v[0x01] == 2.0 ** -9                                # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9                            # largest subnormal
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])             # the only NaNs
    assert np.sum(np.isnan(v)) == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                            # codes 0..0x7E increase
    # consecutive normal values differ by 2^(e-7) / 8 (3 mantissa bits)
    for c in range(0x08, 0x7E):
        e = c >> 3
        assert pos[c + 1] - pos[c] == 2.0 ** (e - 7) / 8


def test_e4m3_encode_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = KO.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(KO.e4m3_encode(vals), codes)          # every finite code (and -0)
    pos = KO.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):                                       # every midpoint: the even code
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        want = c if c % 2 == 0 else c + 1
        assert KO.e4m3_encode(mid) == want, c
        assert KO.e4m3_encode(np.nextafter(mid, np.float32(0))) == c
        assert KO.e4m3_encode(np.nextafter(mid, np.float32(1e9))) == c + 1
    assert KO.e4m3_encode(np.float32(1000.0)) == 0x7E           # saturation
    assert KO.e4m3_encode(np.float32(-1000.0)) == 0xFE
    assert KO.e4m3_encode(np.float32(2.0 ** -11)) == 0          # below half the subnormal step


def test_quantize_rows_error_bound_and_extremes():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((300, 128)) * np.exp(rng.uniform(-8, 8, (300, 1)))).astype(np.float32)
    codes, scale = KO.quantize_rows(x)
    xh = KO.dequantize(codes, scale)
    amax = np.abs(x).max(axis=1)
    # each row's largest magnitude lands on 448 exactly
    assert np.all(np.abs(KO.e4m3_decode(codes)).max(axis=1) == 448.0)
    np.testing.assert_allclose(scale, amax / np.float32(448), rtol=1e-7)
    # rounding error: half a step, i.e. 2^-4 relative in the normal range and
    # half the smallest subnormal step (2^-10 scale) below it
    err = np.abs(xh - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None].astype(np.float64) * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
    # zero row: zero scale and codes
    c0, s0 = KO.quantize_rows(np.zeros((2, 128), np.float32))
    assert np.all(c0 == 0) and np.all(s0 == 0)


# ---------------------------------------------------------------------------
# Ring placement: what StreamingLLM keeps, by brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n_sink,window,chunks", [(4, 7, [3, 1, 5, 9, 2, 30]), (0, 5, [1] * 13),
                                                  (6, 3, [2, 2, 1, 8]), (2, 16, [40])])
def test_append_keeps_first_tokens_and_recent_window(n_sink, window, chunks):
    """Stream tokens whose K carries their position; after every chunk the
    cache holds exactly the first n_sink and the last W positions."""
    d = 8
    cache = KO.new_cache(1, n_sink, window, 1, d, quantized=False)
    seen = 0
    for c in chunks:
        k = np.zeros((1, c, 1, d), np.float32)
        k[0, :, 0, 0] = np.arange(seen, seen + c)             # position tag
        KO.append(cache, k, k, [seen], n_sink, window)
        seen += c
        kept = KO.kept_positions(seen, n_sink, window)
        valid = min(seen, n_sink) + min(max(seen - n_sink, 0), window)
        held = sorted(cache["k"][0, :valid, 0, 0].astype(int).tolist())
        assert held == sorted(kept)
        # brute force: first n_sink, and the most recent W of the rest
        later = [p for p in range(seen) if p >= n_sink]
        assert sorted(kept) == sorted(list(range(min(seen, n_sink))) + later[-window:])


def test_cache_decode_equals_prefill_streaming_row():
    """Decoding the newest token over the cache equals row T-1 of the prefill
    oracle with the StreamingLLM mask (n_sink first tokens + window W): the
    cache content is that mask."""
    rng = np.random.default_rng(3)
    T, hq, hkv, d, n_sink, window = 57, 4, 2, 16, 3, 20
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d)).astype(np.float32)
    v = rng.standard_normal((T, hkv, d)).astype(np.float32)
    sink = rng.standard_normal(hq)
    cache = KO.new_cache(1, n_sink, window, hkv, d, quantized=False)
    seen = 0
    for c in (5, 1, 30, 21):
        KO.append(cache, k[None, seen:seen + c], v[None, seen:seen + c], [seen], n_sink, window)
        seen += c
    assert seen == T
    o, lse, s = KO.cache_decode(q[None, T - 1], cache, [T], n_sink, window, 0.3, sink=sink)
    po, plse, ps = oracle.fwd(q, k, v, [0, T], 0.3, n_sink=n_sink, window=window, sink=sink)
    np.testing.assert_allclose(o[0], po[T - 1], atol=1e-12)
    np.testing.assert_allclose(lse[0], plse[T - 1], atol=1e-12)
    np.testing.assert_allclose(s[0], ps[T - 1], atol=1e-12)


def test_quantized_cache_decode_is_decode_of_dequantized_values():
    """The 8-bit cache decodes as the bf16 cache holding the dequantised
    window values (sinks untouched), and stays within the quantisation error
    of the exact cache."""
    rng = np.random.default_rng(4)
    B, hq, hkv, d, n_sink, window = 3, 4, 2, 32, 4, 12
    qc = KO.new_cache(B, n_sink, window, hkv, d, quantized=True)
    bc = KO.new_cache(B, n_sink, window, hkv, d, quantized=False)
    n = np.array([2, 9, 40])
    for b in range(B):
        kk = rng.standard_normal((1, n[b], hkv, d)).astype(np.float32)
        vv = rng.standard_normal((1, n[b], hkv, d)).astype(np.float32)
        # views of sequence b: the appends write through them
        one = lambda c: {key: (val[b:b + 1] if isinstance(val, np.ndarray) else val)
                         for key, val in c.items()}
        KO.append(one(qc), kk, vv, [0], n_sink, window)
        KO.append(one(bc), kk, vv, [0], n_sink, window)
    q = rng.standard_normal((B, hq, d))
    o_q, lse_q, _ = KO.cache_decode(q, qc, n, n_sink, window, 0.2)
    # the same slots, dequantised into a plain cache
    deq = KO.new_cache(B, n_sink, window, hkv, d, quantized=False)
    deq["k"][:, :n_sink] = qc["sink_k"]
    deq["v"][:, :n_sink] = qc["sink_v"]
    deq["k"][:, n_sink:] = KO.dequantize(qc["win_k"], np.swapaxes(qc["win_k_scale"], 1, 2))
    deq["v"][:, n_sink:] = KO.dequantize(qc["win_v"], np.swapaxes(qc["win_v_scale"], 1, 2))
    o_d, lse_d, _ = KO.cache_decode(q, deq, n, n_sink, window, 0.2)
    np.testing.assert_allclose(o_q, o_d, atol=1e-6)
    np.testing.assert_allclose(lse_q, lse_d, atol=1e-6)
    # sequence 0 has only sink tokens: no quantisation at all
    o_b, _, _ = KO.cache_decode(q, bc, n, n_sink, window, 0.2)
    np.testing.assert_array_equal(o_q[0], o_b[0])
    assert np.max(np.abs(o_q - o_b)) < 0.1


# ---------------------------------------------------------------------------
# Chunked prefill against the cache
# ---------------------------------------------------------------------------

def test_bf16_round_ties_and_library():
    import torch
    one = np.float32(1.0)
    assert KO.bf16_round(np.float32(1 + 2.0 ** -8)) == one                    # tie -> even
    assert KO.bf16_round(np.float32(1 + 3 * 2.0 ** -8)) == np.float32(1 + 2.0 ** -6)
    assert KO.bf16_round(np.float32(1 + 2.0 ** -8 + 2.0 ** -20)) == np.float32(1 + 2.0 ** -7)
    x = (np.random.default_rng(5).standard_normal(10000) * 100).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(KO.bf16_round(x), want)


@pytest.mark.parametrize("n_sink,window,chunks", [(3, 20, [2, 5, 1, 30, 21, 4]), (0, 9, [4, 4, 13]),
                                                  (4, 40, [50, 7])])
def test_cache_prefill_equals_whole_stream_prefill(n_sink, window, chunks):
    """Every chunk's rows, computed from the cache before the chunk is
    appended, equal the rows of the prefill oracle over the whole stream with
    the StreamingLLM mask: first tokens still to come, a ring still filling,
    a wrapped ring and chunks longer than the window."""
    rng = np.random.default_rng(6)
    T, hq, hkv, d = sum(chunks), 4, 2, 8
    q = rng.standard_normal((T, hq, d))
    k = rng.standard_normal((T, hkv, d)).astype(np.float32)
    v = rng.standard_normal((T, hkv, d)).astype(np.float32)
    sink = rng.standard_normal(hq)
    po, plse, ps = oracle.fwd(q, k, v, [0, T], 0.4, n_sink=n_sink, window=window, sink=sink)
    cache = KO.new_cache(1, n_sink, window, hkv, d, quantized=False)
    seen = 0
    for c in chunks:
        sl = slice(seen, seen + c)
        o, lse, s = KO.cache_prefill(q[None, sl], cache, k[None, sl], v[None, sl], [seen], n_sink, window,
                                     0.4, sink=sink)
        np.testing.assert_allclose(o[0], po[sl], atol=1e-12)
        np.testing.assert_allclose(lse[0], plse[sl], atol=1e-12)
        np.testing.assert_allclose(s[0], ps[sl], atol=1e-12)
        KO.append(cache, k[None, sl], v[None, sl], [seen], n_sink, window)
        seen += c


def test_cache_prefill_chunk_of_one_is_decode():
    """A one-token chunk is a decode step: the same row as decoding over the
    cache after appending the token."""
    rng = np.random.default_rng(7)
    B, hq, hkv, d, n_sink, window = 3, 4, 2, 8, 2, 6
    for quantized in (False, True):
        cache = KO.new_cache(B, n_sink, window, hkv, d, quantized)
        seen = np.array([0, 3, 11])
        for b in range(B):
            n = int(seen[b])
            one = {key: (val[b:b + 1] if isinstance(val, np.ndarray) else val) for key, val in cache.items()}
            KO.append(one, rng.standard_normal((1, n, hkv, d)), rng.standard_normal((1, n, hkv, d)), [0],
                      n_sink, window)
        q = rng.standard_normal((B, 1, hq, d))
        kn = rng.standard_normal((B, 1, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((B, 1, hkv, d)).astype(np.float32)
        if quantized:
            kn, vn = KO.bf16_round(kn), KO.bf16_round(vn)
        o, lse, s = KO.cache_prefill(q, cache, kn, vn, seen, n_sink, window, 0.3)
        KO.append(cache, kn, vn, seen, n_sink, window)
        if quantized:
            # the decode oracle reads the exact dequantised ring; the prefill
            # reads it rounded to bfloat16: compare on a plain cache holding
            # the rounded values
            plain = KO.new_cache(B, n_sink, window, hkv, d, False)
            plain["k"][:, :n_sink] = cache["sink_k"]
            plain["v"][:, :n_sink] = cache["sink_v"]
            for name, sc in (("k", "win_k_scale"), ("v", "win_v_scale")):
                deq = KO.e4m3_decode(cache["win_" + name]).astype(np.float32) * \
                    np.swapaxes(cache[sc], 1, 2)[..., None].astype(np.float32)
                plain[name][:, n_sink:] = KO.bf16_round(deq)
            # the newest token is in the ring too, quantised: put its chunk value back
            for b in range(B):
                p = int(seen[b])
                kind, slot = KO.slot_of(p, n_sink, window)
                i = slot if kind == "sink" else n_sink + slot
                plain["k"][b, i], plain["v"][b, i] = kn[b, 0], vn[b, 0]
            cache = plain
        do, dl, ds = KO.cache_decode(q[:, 0], cache, seen + 1, n_sink, window, 0.3)
        np.testing.assert_allclose(o[:, 0], do, atol=1e-12)
        np.testing.assert_allclose(lse[:, 0], dl, atol=1e-12)
        np.testing.assert_allclose(s[:, 0], ds, atol=1e-12)


def test_cache_prefill_q8_with_exact_values_equals_bf16():
    """Rows whose values are e4m3 codes times a power of two (largest code
    448) quantise without error, so the 8-bit cache prefills exactly as the
    bf16 cache holding the same values."""
    rng = np.random.default_rng(8)
    B, C, hq, hkv, d, n_sink, window = 2, 5, 4, 2, 16, 2, 7
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])

    def exact_rows(n):
        codes = rng.choice(finite, size=(B, n, hkv, d))
        codes[..., 0] = 0x7E                                    # amax code 448 in every row
        return (KO.e4m3_decode(codes) * 2.0 ** rng.integers(-8, -4, size=(B, n, hkv, 1))).astype(np.float32)

    qc = KO.new_cache(B, n_sink, window, hkv, d, quantized=True)
    bc = KO.new_cache(B, n_sink, window, hkv, d, quantized=False)
    kk, vv = exact_rows(12), exact_rows(12)
    for c in (qc, bc):
        KO.append(c, kk, vv, [0, 0], n_sink, window)
    assert np.array_equal(KO.dequantize(qc["win_k"], np.swapaxes(qc["win_k_scale"], 1, 2)),
                          bc["k"][:, n_sink:])
    q = rng.standard_normal((B, C, hq, d))
    kn, vn = exact_rows(C), exact_rows(C)
    a = KO.cache_prefill(q, qc, kn, vn, [12, 12], n_sink, window, 0.25, sink=np.zeros(hq))
    b_ = KO.cache_prefill(q, bc, kn, vn, [12, 12], n_sink, window, 0.25, sink=np.zeros(hq))
    for x, y in zip(a, b_):
        np.testing.assert_array_equal(x, y)
