"""Seeded synthetic inputs for sink attention, shared by the HIP path and the oracle.

This module draws random numbers and lays them out; it holds none of the
attention arithmetic.  Every workload is drawn from one numpy
``Generator(PCG64(seed))`` in a fixed order: structure first (sample lengths,
block selections, slot permutations), then Q, K, V, the learnable sink logits
and dO.  Floating-point draws are float32 N(0, 1), rounded once to bfloat16
(round to nearest even) and then held two ways: as float32 arrays whose
values are exactly representable in bfloat16 (what the oracle upcasts to
float64) and as raw uint16 bit patterns (what the device receives).

The workload shapes follow the pages' settings: packed variable-length
samples (a ``cu_seqlens`` prefix array), grouped-query heads, a StreamingLLM
mask of ``n_sink`` first tokens plus a recent window, sparse block lists, and
a rolling decode cache whose slots are in no particular position order.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BLOCK = 64  # block size used by block-sparse workloads


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normal draws, so NaN/Inf handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


@dataclasses.dataclass
class Tensor:
    """A drawn tensor: float32 values and, for bf16 workloads, the raw bits."""
    f32: np.ndarray                 # values (bf16-exact when dtype == "bf16")
    bits: Optional[np.ndarray]      # uint16 bit patterns, or None for f32

    @property
    def shape(self):
        return self.f32.shape


def _draw(rng, shape, dtype: str, scale: float = 1.0) -> Tensor:
    x = _normal(rng, shape, scale)
    if dtype == "bf16":
        bits = round_to_bf16_bits(x)
        return Tensor(bf16_bits_to_f32(bits), bits)
    return Tensor(x, None)


@dataclasses.dataclass
class Prefill:
    name: str
    dtype: str                      # "bf16" or "f32"
    cu_seqlens: np.ndarray          # int32 [B+1]
    hq: int
    hkv: int
    d: int
    n_sink: int
    window: int                     # <= 0: no window
    block_size: int
    block_indices: Optional[np.ndarray]   # int32 [NQB, Hkv, KB] or None
    q: Tensor
    k: Tensor
    v: Tensor
    sink: Optional[np.ndarray]      # float32 [Hq] or None
    do: Optional[Tensor]
    scale: float

    @property
    def batch(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def total(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if self.batch else 0


@dataclasses.dataclass
class Decode:
    name: str
    dtype: str
    batch: int
    slots: int
    hq: int
    hkv: int
    d: int
    q: Tensor                       # [B, Hq, D]
    k_cache: Tensor                 # [B, S, Hkv, D]
    v_cache: Tensor                 # [B, S, Hkv, D]
    cache_seqlens: Optional[np.ndarray]   # int32 [B] or None (all slots valid)
    positions: np.ndarray           # int64 [B, S] slot -> stream position (tests only)
    sink: Optional[np.ndarray]
    scale: float


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def varlen_lengths(rng, n: int, lo: int, hi: int, total: int) -> np.ndarray:
    """n lengths, each uniform on {lo..hi}, conditioned on summing to ``total``.

    Draw n-1 lengths i.i.d., give the rest to the last sample, and redraw the
    whole set until the last one also falls in [lo, hi]; the accepted sets are
    uniform on the constrained set.
    """
    if not (n * lo <= total <= n * hi):
        raise ValueError("total not reachable with these bounds")
    while True:
        head = rng.integers(lo, hi + 1, size=n - 1)
        last = total - int(head.sum())
        if lo <= last <= hi:
            return np.concatenate([head, [last]]).astype(np.int64)


def sparse_block_lists(rng, lengths, hkv: int, n_random: int,
                       block: int = BLOCK, always_first: bool = True,
                       diagonal: bool = True) -> np.ndarray:
    """Block lists per (query block, KV head), packed over samples.

    For sample-local query block qb the list is {0} U R U {qb}, with R drawn
    uniformly without replacement from {1..qb-1}, |R| = min(n_random, qb-1);
    entries are sorted and padded with -1 to the fixed width.  Rows are
    ordered by sample, then by sample-local query block.
    """
    width = int(always_first) + n_random + int(diagonal)
    rows = []
    for L in lengths:
        nqb = -(-int(L) // block)
        for qb in range(nqb):
            for _g in range(hkv):
                sel = set()
                if always_first:
                    sel.add(0)
                if qb > 1 and n_random > 0:
                    r = min(n_random, qb - 1)
                    sel.update((1 + rng.choice(qb - 1, size=r, replace=False)).tolist())
                if diagonal:
                    sel.add(qb)
                row = sorted(sel)
                row = row + [-1] * (width - len(row))
                rows.append(row)
    nq = len(rows) // hkv if hkv else 0
    return np.asarray(rows, dtype=np.int32).reshape(nq, hkv, width)


def make_prefill(name: str, lengths, hq: int, hkv: int, d: int, dtype: str = "bf16",
                 n_sink: int = 0, window: int = 0, sink: bool = True,
                 with_do: bool = True, k_scale: float = 1.0, seed: int = 0,
                 block_lists: Optional[dict] = None, sink_shift: float = 0.0,
                 rng: Optional[np.random.Generator] = None) -> Prefill:
    """Draw a packed prefill workload.

    ``block_lists``: None for dense/window masks, else kwargs for
    :func:`sparse_block_lists` (drawn right after the lengths).
    ``sink_shift`` is added to every drawn sink logit (stress variants that
    push the real-token share s towards 0.5).
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    bi = None
    if block_lists is not None:
        bi = sparse_block_lists(rng, lengths, hkv, **block_lists)
    q = _draw(rng, (T, hq, d), dtype)
    k = _draw(rng, (T, hkv, d), dtype, scale=k_scale)
    v = _draw(rng, (T, hkv, d), dtype)
    a = rng.standard_normal(size=hq, dtype=np.float32) if sink else None
    if a is not None and sink_shift:
        a = (a + np.float32(sink_shift)).astype(np.float32)
    do = _draw(rng, (T, hq, d), dtype) if with_do else None
    return Prefill(name=name, dtype=dtype, cu_seqlens=cu, hq=hq, hkv=hkv, d=d,
                   n_sink=n_sink, window=window, block_size=BLOCK, block_indices=bi,
                   q=q, k=k, v=v, sink=a, do=do, scale=1.0 / float(np.sqrt(d)))


def make_decode(name: str, batch: int, slots: int, hq: int, hkv: int, d: int,
                dtype: str = "bf16", sink: bool = True, seed: int = 0,
                cache_seqlens=None, stream_len: Optional[int] = None,
                n_sink: int = 4) -> Decode:
    """Draw a rolling-cache decode workload.

    Each sequence has ``slots`` cache slots holding n_sink kept first tokens
    and the most recent tokens of a stream of ``stream_len`` tokens; which slot
    holds which position is a random permutation (a ring buffer has no
    position order).  The positions are recorded for tests; the kernel never
    sees them.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    stream_len = stream_len if stream_len is not None else 4 * slots
    recent = slots - n_sink
    pos_pool = np.concatenate([np.arange(n_sink),
                               np.arange(stream_len - recent, stream_len)]).astype(np.int64)
    positions = np.stack([pos_pool[rng.permutation(slots)] for _ in range(batch)])
    q = _draw(rng, (batch, hq, d), dtype)
    kc = _draw(rng, (batch, slots, hkv, d), dtype)
    vc = _draw(rng, (batch, slots, hkv, d), dtype)
    a = rng.standard_normal(size=hq, dtype=np.float32) if sink else None
    csl = None if cache_seqlens is None else np.asarray(cache_seqlens, dtype=np.int32)
    return Decode(name=name, dtype=dtype, batch=batch, slots=slots, hq=hq, hkv=hkv, d=d,
                  q=q, k_cache=kc, v_cache=vc, cache_seqlens=csl, positions=positions,
                  sink=a, scale=1.0 / float(np.sqrt(d)))


@dataclasses.dataclass
class KvDecodeQ8:
    """A filled 8-bit rolling cache and one query per sequence.  The ring
    holds e4m3 codes drawn directly (uniform over the 254 non-NaN codes) with
    per-(sequence, KV head, slot) scales near those of unit-normal rows; no
    quantisation is computed here."""
    batch: int
    n_sink: int
    window: int
    hq: int
    hkv: int
    d: int
    q: np.ndarray            # float32 (bf16-exact) [B, Hq, D]
    sink_k: np.ndarray       # float32 (bf16-exact) [B, n_sink, Hkv, D]
    sink_v: np.ndarray
    win_k: np.ndarray        # uint8 [B, window, Hkv, D]
    win_v: np.ndarray
    win_k_scale: np.ndarray  # float32 [B, Hkv, window]
    win_v_scale: np.ndarray
    n_tokens: np.ndarray     # int32 [B]: stream lengths (>= n_sink + window: full caches)
    sink: np.ndarray         # float32 [Hq]
    scale: float


def kvcache_q8_decode(batch: int = 128, n_sink: int = 4, window: int = 4092, hq: int = 64,
                      hkv: int = 8, d: int = 128, seed: int = 0) -> KvDecodeQ8:
    rng = np.random.Generator(np.random.PCG64(seed))
    valid = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)

    def codes(shape):
        return valid[rng.integers(0, len(valid), size=shape, dtype=np.uint8)]

    def scales(shape):
        return (rng.uniform(2.0, 4.0, size=shape) / 448.0).astype(np.float32)

    q = _draw(rng, (batch, hq, d), "bf16").f32
    sk = _draw(rng, (batch, n_sink, hkv, d), "bf16").f32
    sv = _draw(rng, (batch, n_sink, hkv, d), "bf16").f32
    wk, wv = codes((batch, window, hkv, d)), codes((batch, window, hkv, d))
    ks, vs = scales((batch, hkv, window)), scales((batch, hkv, window))
    n_tokens = rng.integers(n_sink + window, 4 * (n_sink + window), size=batch).astype(np.int32)
    a = rng.standard_normal(size=hq, dtype=np.float32)
    return KvDecodeQ8(batch, n_sink, window, hq, hkv, d, q, sk, sv, wk, wv, ks, vs, n_tokens, a,
                      1.0 / float(np.sqrt(d)))



@dataclasses.dataclass
class KvPrefill:
    """A filled bf16 rolling cache (first tokens + a wrapped ring) and one
    chunk of new tokens per stream, each stream at its own position."""
    batch: int
    n_sink: int
    window: int
    chunk: int
    hq: int
    hkv: int
    d: int
    k_cache: np.ndarray      # float32 (bf16-exact) [B, n_sink + window, Hkv, D]
    v_cache: np.ndarray
    q: np.ndarray            # float32 (bf16-exact) [B, chunk, Hq, D]
    k_new: np.ndarray        # float32 (bf16-exact) [B, chunk, Hkv, D]
    v_new: np.ndarray
    n_seen: np.ndarray       # int32 [B]: tokens cached before the chunk (>= n_sink + window)
    sink: np.ndarray         # float32 [Hq]
    scale: float

    def valid_pairs(self) -> int:
        """(query row, key) pairs the StreamingLLM mask keeps, over all heads."""
        total = 0
        for p0 in self.n_seen:
            p = int(p0) + np.arange(self.chunk)
            lo = np.maximum(p - self.window + 1, 0)              # window keys [lo, p]
            win = p - lo + 1
            first = np.minimum(self.n_sink, lo)                  # first tokens below the window
            total += int(np.sum(win + first))
        return total * self.hq


def kvcache_prefill(batch: int = 8, n_sink: int = 4, window: int = 1024, chunk: int = 1024, hq: int = 32,
                    hkv: int = 8, d: int = 128, seed: int = 0) -> KvPrefill:
    """Streams of the StreamingLLM prefill shape (4 first tokens, a
    1024-token window, Hq=32, Hkv=8, D=128) taking their next 1024-token
    chunk at positions past the first window."""
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = n_sink + window
    kc = _draw(rng, (batch, slots, hkv, d), "bf16").f32
    vc = _draw(rng, (batch, slots, hkv, d), "bf16").f32
    q = _draw(rng, (batch, chunk, hq, d), "bf16").f32
    kn = _draw(rng, (batch, chunk, hkv, d), "bf16", 0.5).f32
    vn = _draw(rng, (batch, chunk, hkv, d), "bf16").f32
    kc[:, n_sink:] *= np.float32(0.5)                             # K scaled as in the prefill workloads
    kc[:, :n_sink] *= np.float32(0.5)
    n_seen = rng.integers(slots, 8 * slots, size=batch).astype(np.int32)
    a = rng.standard_normal(size=hq, dtype=np.float32)
    return KvPrefill(batch, n_sink, window, chunk, hq, hkv, d, kc, vc, q, kn, vn, n_seen, a,
                     1.0 / float(np.sqrt(d)))

# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def tiny_f32(seed: int = 0) -> Prefill:
    """One sequence T=64, Hq=2, Hkv=1, D=16, fp32, causal, n_sink=4, window=16."""
    return make_prefill("tiny_f32", [64], hq=2, hkv=1, d=16, dtype="f32",
                        n_sink=4, window=16, seed=seed)


def gqa_prefill(seed: int = 0, seq: int = 4096, batch: int = 4) -> Prefill:
    """batch x seq packed, Hq=32, Hkv=8, D=128, bf16, causal, K scaled by 0.5."""
    return make_prefill("gqa_prefill", [seq] * batch, hq=32, hkv=8, d=128,
                        k_scale=0.5, with_do=False, seed=seed)


def streaming_lengths(seed: int = 0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng, varlen_lengths(rng, 8, 2048, 8192, 32768)


def streaming_prefill(seed: int = 0) -> Prefill:
    """8 varlen samples (2048..8192, sum 32768), Hq=32, Hkv=8, D=128, bf16,
    causal + n_sink=4 + window=1024, with dO."""
    rng, lengths = streaming_lengths(seed)
    return make_prefill("streaming_prefill", lengths, hq=32, hkv=8, d=128,
                        n_sink=4, window=1024, rng=rng)


def streaming_decode(seed: int = 0, batch: int = 128, slots: int = 4096) -> Decode:
    """128 sequences x 1 query, 4096-slot rolling cache (4 sink + 4092 recent),
    Hq=64, Hkv=8, D=128, bf16."""
    return make_decode("streaming_decode", batch, slots, hq=64, hkv=8, d=128, seed=seed)


def block_sparse(seed: int = 0, seq: int = 16384, batch: int = 4) -> Prefill:
    """batch x seq packed, Hq=64, Hkv=8, D=128, bf16, block 64; per (q block,
    KV head): block 0 + 15 random causal blocks + the diagonal block."""
    return make_prefill("block_sparse", [seq] * batch, hq=64, hkv=8, d=128,
                        block_lists=dict(n_random=15), seed=seed)
