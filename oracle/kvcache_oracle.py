"""Plain CPU oracle for the StreamingLLM rolling KV cache and its sink-aware
8-bit variant.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke entry point and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP path and imports nothing from it.

Sources (cited by title and section):
  [QA]   "What is Attention Sink? How does StreamingLLM use it to handle long
         streaming input?" (model.playoffer.cn), "StreamingLLM core idea":
         the cache is a fixed segment of the first tokens (4 recommended) plus
         a sliding window of the most recent N; a new token enters the window
         and the oldest window token (never a first token) leaves.
         "Other engineering implications": KV-cache quantisers keep the first
         tokens, which carry a large attention share, in high precision and
         the other positions in low precision.
  [Blog] "Attention Sink" (lijianxiong.space), H2O section: the recent part is
         a circular queue whose oldest entry the new token replaces.

Readings where the pages leave a step open:
  * Placement: the token at stream position p lives in sink slot p when
    p < n_sink, else in ring slot (p - n_sink) mod W of the window segment.
    After T tokens the cache holds positions [0, min(T, n_sink)) and
    [max(n_sink, T - W), T): exactly StreamingLLM's kept set.
  * Low precision: 8-bit floating point e4m3 in the OCP layout (1 sign, 4
    exponent bits with bias 7, 3 mantissa bits; 448 the largest finite value;
    exponent 15 with mantissa 7 is NaN; no infinities), one float32 scale per
    (token, KV head) row: scale = amax / 448, code = e4m3(x * (448 / amax))
    rounded to nearest, ties to even, |values| above 448 saturating to 448.
    A row of zeros gets scale 0 and zero codes.  The first n_sink tokens stay
    bfloat16.
  * Decode over the cache: the current token is already appended; the valid
    slots are every slot a position was written to; no causal or window mask
    beyond that (the cache content is the mask).
  * Chunked prefill against the cache: chunk row c of a stream that has
    appended P0 tokens is position p = P0 + c and sees key position k when
    k <= p and (k < n_sink or p - k < W), the prefill mask of StreamingLLM
    ([QA] core idea) over the stream; keys before P0 come from the cache as
    it is before the chunk is appended, the others from the chunk.  The
    8-bit ring enters as bfloat16(float32(code value) * scale), rounded to
    nearest even: the prefill consumes bfloat16 keys and values.
"""
from __future__ import annotations

import numpy as np

from .sink_attn_oracle import decode as _decode

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "quantize_rows", "dequantize", "slot_of",
    "new_cache", "append", "kept_positions", "cache_decode", "bf16_round", "cache_prefill",
]

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """Value of each 8-bit code (OCP e4m3): (-1)^s 2^(e-7) (1 + m/8), or
    (-1)^s 2^-6 m/8 for e = 0; e = 15 with m = 7 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * (m / 8.0) * 2.0 ** -6
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


_POS_CODES = np.arange(0x7F)                 # 0x00 .. 0x7E: the finite non-negative codes
_POS_VALUES = e4m3_decode(_POS_CODES)        # increasing


def e4m3_encode(x):
    """Nearest e4m3 code of each value (float32 inputs), ties to the even
    code (the one with an even mantissa), magnitudes above 448 saturating."""
    v = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    # index of the largest representable value <= a, and the next one up
    lo = np.clip(np.searchsorted(_POS_VALUES, a, side="right") - 1, 0, len(_POS_VALUES) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.int64)
    neg = np.signbit(v)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def quantize_rows(x):
    """Per-row (last axis) 8-bit quantisation, in float32 as a kernel computes
    it: amax, scale = amax / 448, code = e4m3(x * (448 / amax)).  Returns
    (codes uint8, scale float32); a zero row gets scale 0."""
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    scale = np.where(zero, np.float32(0.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
    v = (xf * inv[..., None]).astype(np.float32)
    codes = e4m3_encode(v)
    codes = np.where(zero[..., None], np.uint8(0), codes).astype(np.uint8)
    return codes, scale


def dequantize(codes, scale):
    """code value times the row's scale, in float64."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def slot_of(p, n_sink, window):
    """("sink", p) for p < n_sink, else ("win", (p - n_sink) mod W)."""
    if p < n_sink:
        return "sink", p
    return "win", (p - n_sink) % window


def new_cache(batch, n_sink, window, hkv, d, quantized):
    """An empty cache as a dict of numpy arrays (the same layout as the
    library's): bf16 values are held as float32 here."""
    if not quantized:
        return dict(quantized=False, k=np.zeros((batch, n_sink + window, hkv, d), np.float32),
                    v=np.zeros((batch, n_sink + window, hkv, d), np.float32))
    return dict(quantized=True,
                sink_k=np.zeros((batch, n_sink, hkv, d), np.float32),
                sink_v=np.zeros((batch, n_sink, hkv, d), np.float32),
                win_k=np.zeros((batch, window, hkv, d), np.uint8),
                win_v=np.zeros((batch, window, hkv, d), np.uint8),
                win_k_scale=np.zeros((batch, hkv, window), np.float32),
                win_v_scale=np.zeros((batch, hkv, window), np.float32))


def append(cache, k_new, v_new, n_seen, n_sink, window):
    """Write chunk tokens (k_new, v_new [B, C, Hkv, D], positions n_seen[b] +
    c) into the cache in stream order: each token overwrites whatever its
    slot held, so the oldest window token leaves ([QA] core idea; [Blog]
    circular queue)."""
    k_new = np.asarray(k_new, np.float32)
    v_new = np.asarray(v_new, np.float32)
    B, C = k_new.shape[:2]
    for b in range(B):
        for c in range(C):
            p = int(n_seen[b]) + c
            kind, s = slot_of(p, n_sink, window)
            if not cache["quantized"]:
                slot = s if kind == "sink" else n_sink + s
                cache["k"][b, slot] = k_new[b, c]
                cache["v"][b, slot] = v_new[b, c]
            elif kind == "sink":
                cache["sink_k"][b, s] = k_new[b, c]
                cache["sink_v"][b, s] = v_new[b, c]
            else:
                kc, ks = quantize_rows(k_new[b, c])          # [Hkv, D] rows
                vc, vs = quantize_rows(v_new[b, c])
                cache["win_k"][b, s] = kc
                cache["win_v"][b, s] = vc
                cache["win_k_scale"][b, :, s] = ks
                cache["win_v_scale"][b, :, s] = vs
    return cache


def kept_positions(total, n_sink, window):
    """Stream positions StreamingLLM keeps after `total` tokens."""
    first = list(range(min(total, n_sink)))
    recent = list(range(max(n_sink, total - window), total))
    return first + recent


def _dense(cache, n_sink, window):
    """The cache as [B, n_sink + W, Hkv, D] float64 values, sinks first."""
    if not cache["quantized"]:
        return np.asarray(cache["k"], np.float64), np.asarray(cache["v"], np.float64)
    kw = dequantize(cache["win_k"], np.swapaxes(cache["win_k_scale"], 1, 2))
    vw = dequantize(cache["win_v"], np.swapaxes(cache["win_v_scale"], 1, 2))
    k = np.concatenate([np.asarray(cache["sink_k"], np.float64), kw], axis=1)
    v = np.concatenate([np.asarray(cache["sink_v"], np.float64), vw], axis=1)
    return k, v


def cache_decode(q, cache, n_tokens, n_sink, window, scale, sink=None):
    """Decode of one query per sequence over the slots written so far
    (n_tokens[b] tokens appended, the current one included): the plain decode
    definition on the dequantised values."""
    k, v = _dense(cache, n_sink, window)
    n = np.asarray(n_tokens, dtype=np.int64)
    valid = np.minimum(n, n_sink) + np.minimum(np.maximum(n - n_sink, 0), window)
    return _decode(q, k, v, scale, cache_seqlens=valid, sink=sink)


def bf16_round(x):
    """float32 values rounded to the nearest bfloat16, ties to even (finite
    inputs), returned as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _key_at(cache, b, pos, n_sink, window):
    """K and V rows [Hkv, D] (float64) the cache holds for stream position pos."""
    kind, slot = slot_of(pos, n_sink, window)
    if not cache["quantized"]:
        i = slot if kind == "sink" else n_sink + slot
        return np.asarray(cache["k"][b, i], np.float64), np.asarray(cache["v"][b, i], np.float64)
    if kind == "sink":
        return (np.asarray(cache["sink_k"][b, slot], np.float64),
                np.asarray(cache["sink_v"][b, slot], np.float64))
    out = []
    for codes, sc in ((cache["win_k"][b, slot], cache["win_k_scale"][b, :, slot]),
                      (cache["win_v"][b, slot], cache["win_v_scale"][b, :, slot])):
        vals = e4m3_decode(codes).astype(np.float32) * np.asarray(sc, np.float32)[:, None]
        out.append(bf16_round(vals).astype(np.float64))
    return out[0], out[1]


def cache_prefill(q, cache, k_new, v_new, n_seen, n_sink, window, scale, sink=None, rows=None):
    """Chunked prefill against the cache (reading above), row by row: each
    row's visible keys in position order, then the plain decode definition
    on them.  q [B, C, Hq, D], k_new / v_new [B, C, Hkv, D].  Returns o [B, C,
    Hq, D], lse and s [B, C, Hq]; with rows = [(b, c), ...] only those rows
    (the others stay zero)."""
    q = np.asarray(q, np.float64)
    B, C, hq, d = q.shape
    o = np.zeros((B, C, hq, d))
    lse = np.zeros((B, C, hq))
    s = np.zeros((B, C, hq))
    todo = rows if rows is not None else [(b, c) for b in range(B) for c in range(C)]
    for b, c in todo:
        p0 = int(n_seen[b])
        p = p0 + c
        vis = [k for k in range(p + 1) if k < n_sink or p - k < window]
        ks, vs = [], []
        for k in vis:
            if k < p0:
                kk, vv = _key_at(cache, b, k, n_sink, window)
            else:
                kk = np.asarray(k_new[b, k - p0], np.float64)
                vv = np.asarray(v_new[b, k - p0], np.float64)
            ks.append(kk)
            vs.append(vv)
        kd = np.stack(ks)[None]                     # [1, n_vis, Hkv, D]
        vd = np.stack(vs)[None]
        ro, rl, rs = _decode(q[b, c][None], kd, vd, scale, sink=sink)
        o[b, c], lse[b, c], s[b, c] = ro[0], rl[0], rs[0]
    return o, lse, s
