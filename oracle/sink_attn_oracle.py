"""Plain, slow, float64 CPU oracle for attention with a learnable sink.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke entry point and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP path (no kernels, headers, helpers or tables) and imports nothing
from it.

Sources (cited by title and section throughout):
  [Notes]  "Attention Sink, Learnable Sink and dsink: from the meaning of the
           output to the backward gradient" (notes.kuangjux.top), sections 1-10.
  [QA]     "What is Attention Sink? How does StreamingLLM use it to handle long
           streaming input?" (model.playoffer.cn), "StreamingLLM core idea".
  [MoE]    "Paper notes: Attention Sink and the native MoE in attention layers"
           (lvdousha26.github.io), sections 2 and 5.

What is computed, per packed sample b, query head h, KV head g = g(h):
  x_ij   = alpha * <Q_ih, K_jg>                    [Notes] s1, definition of x
  valid  = causal, same sample, StreamingLLM window with kept first tokens,
           optional selected blocks                [Notes] s1-2; [QA] core idea
  L_orig = log sum_{j valid} e^{x_ij}              [Notes] s4, definition of Z, L_orig
  L_new  = log(e^{L_orig} + e^{a_h})               [Notes] s4, L_new
  P_ij   = e^{x_ij - L_new}                        [Notes] s4, O_new sum
  O_ih   = sum_j P_ij V_jg                         [Notes] s1, definition of O
  s_ih   = e^{L_orig - L_new}                      [Notes] s4, the four forms of s
Backward:
  Delta_ih = sum_d dO_ihd O_ihd                    [Notes] s7, definition of Delta
  dx_ij    = P_ij (<dO_ih, V_jg> - Delta_ih)       [Notes] s8, score gradient
  dsink_h  = -sum_i Delta_ih (1 - s_ih)            [Notes] s7, boxed equation
Gate statistics:
  G_ih     = sigma(LSE_not0 - x_i0)                [MoE] s5, vanilla attention
             (the first token of the sample plays the sink: G = 1 - A_0, s2)
  Imp_h    = (1/|T|) sum_i G_ih                    [MoE] s4, head importance

Readings where the pages leave a step open:
  * g(h) = h // (Hq / Hkv): contiguous groups of query heads share a KV head.
  * window W > 0: key j is in the window of query i iff i - j < W (the query
    itself counts); the first n_sink tokens of each sample stay visible.
    n_sink only matters when a window is set.
  * block_indices: int32 [NQB, Hkv, KB]; rows ordered by sample then by
    sample-local query block of ``block_size`` rows; entries are sample-local
    KV block ids, -1 is padding, each row is a set.  The selected blocks are
    further narrowed by causal order, the window and the sample boundary.
  * the sink logit is not multiplied by alpha and uses the natural base
    ([Notes] s7, second pitfall).
  * returned lse is L_orig (the real-token log-sum-exp); ``sink=None`` means
    no sink (s = 1); an empty valid set gives O = 0, lse = -inf and s = 0 with
    a sink (s = 1 without).
  * dsink is a plain sum over every query row of the call, with no mean.
  * first-token gate: the sink of vanilla attention is the sample's first
    token; G = 1 when that token is not a valid key of the row (no term to
    remove), 0 for a row with no valid key at all.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kv_head", "sample_mask", "fwd", "fwd_virtual_key", "bwd", "decode",
    "fwd_rows", "bwd_rows", "bwd_kv_rows", "logsumexp_rows", "first_token_gate",
    "first_token_gate_rows", "head_importance", "mask_rows", "fwd_bwd_heads",
]


def kv_head(h: int, hq: int, hkv: int) -> int:
    """g(h): the KV head read by query head h ([Notes] s1, GQA map)."""
    return h // (hq // hkv)


def _q_block_offsets(cu_seqlens, block_size):
    """First block_indices row of each sample (rows are packed by sample)."""
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    nqb = -(-lengths // block_size)
    return np.concatenate([[0], np.cumsum(nqb)]).astype(np.int64)


def sample_mask(L, n_sink, window, blocks=None, block_size=64):
    """Valid-key mask [L, L] for one sample and one KV head ([Notes] s1-2).

    ``blocks``: None, or an int array [nqb, KB] of selected sample-local KV
    block ids per sample-local query block (-1 = padding).
    """
    return mask_rows(0, L, np.arange(L), n_sink, window, blocks, block_size)


def mask_rows(i0, i1, cols, n_sink, window, blocks=None, block_size=64):
    """The valid-key predicate of sample_mask for sample-local query rows
    [i0, i1) and the sample-local key indices ``cols``: [i1 - i0, len(cols)]."""
    i = np.arange(i0, i1)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    m = j <= i                                   # causal order
    if window > 0:                               # kept first tokens + recent window
        m = m & ((j < n_sink) | (i - j < window))
    if blocks is not None:                       # sparse block selection
        sel = np.zeros(m.shape, dtype=bool)
        for qb in range(i0 // block_size, (i1 - 1) // block_size + 1):
            r0, r1 = max(i0, qb * block_size) - i0, min(i1, (qb + 1) * block_size) - i0
            for kb in blocks[qb]:
                if kb >= 0:
                    sel[r0:r1] |= (j[0] // block_size) == kb
        m = m & sel
    return m


def logsumexp_rows(x):
    """log sum_j e^{x_j} per row; rows with no finite entry give -inf."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, initial=-np.inf)
    safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        out = safe + np.log(np.sum(np.exp(x - safe[..., None]), axis=-1))
    return np.where(np.isfinite(m), out, -np.inf)


def _sink_terms(lorig, a):
    """L_new, s and p_sink from L_orig and the sink logit ([Notes] s4).

    a is None: no sink, L_new = L_orig, s = 1, p_sink = 0.
    """
    if a is None:
        return lorig.copy(), np.ones_like(lorig), np.zeros_like(lorig)
    lnew = np.logaddexp(lorig, a)                       # log(Z + e^a)
    s = np.exp(lorig - lnew)                            # Z / (Z + e^a)
    p_sink = np.exp(a - lnew)                           # e^a / (Z + e^a)
    return lnew, s, p_sink


def _as64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _blocks_of(block_indices, qoff, b, g):
    if block_indices is None:
        return None
    return np.asarray(block_indices)[qoff[b]:qoff[b + 1], g, :]


def fwd(q, k, v, cu_seqlens, scale, n_sink=0, window=0, block_indices=None,
        block_size=64, sink=None):
    """Forward: returns (O [T,Hq,D], lse = L_orig [T,Hq], s [T,Hq]) in float64.

    Materialises the full score matrix of each (sample, head), masks it and
    normalises with the extra e^{a_h} term in the denominator ([Notes] s1, s4).
    """
    q, k, v, a = _as64(q), _as64(k), _as64(v), _as64(sink)
    T, hq, D = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    o = np.zeros((T, hq, D))
    lse = np.full((T, hq), -np.inf)
    s_out = np.ones((T, hq))
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        L = t1 - t0
        if L == 0:
            continue
        for g in range(hkv):
            M = sample_mask(L, n_sink, window, _blocks_of(block_indices, qoff, b, g), block_size)
            for h in range(hq):
                if kv_head(h, hq, hkv) != g:
                    continue
                x = scale * (q[t0:t1, h, :] @ k[t0:t1, g, :].T)     # x_ij
                x = np.where(M, x, -np.inf)
                lorig = logsumexp_rows(x)
                lnew, s, _ = _sink_terms(lorig, None if a is None else a[h])
                safe = np.where(np.isfinite(lnew), lnew, 0.0)
                P = np.where(M, np.exp(x - safe[:, None]), 0.0)
                o[t0:t1, h, :] = P @ v[t0:t1, g, :]
                lse[t0:t1, h] = lorig
                s_out[t0:t1, h] = s
    return o, lse, s_out


def fwd_virtual_key(q, k, v, cu_seqlens, scale, n_sink=0, window=0, block_indices=None,
                    block_size=64, sink=None):
    """Second formulation: the sink as one extra key with logit a_h and V = 0.

    Softmax over [valid scores, a_h] taken as one vector; O is the weighted sum
    of the real values only; s is the total probability of the real keys
    ([Notes] s3, a value-free virtual position; [MoE] s2, G = 1 - A_sink).
    Returns (O, s).
    """
    q, k, v, a = _as64(q), _as64(k), _as64(v), _as64(sink)
    T, hq, D = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    o = np.zeros((T, hq, D))
    s_out = np.ones((T, hq))
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        L = t1 - t0
        for g in range(hkv):
            M = sample_mask(L, n_sink, window, _blocks_of(block_indices, qoff, b, g), block_size)
            for h in range(hq):
                if kv_head(h, hq, hkv) != g:
                    continue
                x = scale * (q[t0:t1, h, :] @ k[t0:t1, g, :].T)
                x = np.where(M, x, -np.inf)
                extra = np.full((L, 1), -np.inf if a is None else a[h])
                xa = np.concatenate([x, extra], axis=1)
                m = np.max(xa, axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(xa - m)
                den = e.sum(axis=1, keepdims=True)
                with np.errstate(invalid="ignore"):
                    p = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)
                o[t0:t1, h, :] = p[:, :L] @ v[t0:t1, g, :]
                s_out[t0:t1, h] = p[:, :L].sum(axis=1) if a is not None else 1.0
    return o, s_out


def first_token_gate(q, k, cu_seqlens, scale, n_sink=0, window=0, block_indices=None,
                     block_size=64):
    """Vanilla-attention gate G [T,Hq] in float64 ([MoE] s5, vanilla form).

    The sample's first token is the sink of vanilla attention; its share of
    the softmax is taken out through the log-sum-exp of the other valid keys:
    G = sigma(LSE_not0 - x_i0), where x_i0 = alpha <q_i, k_0> and LSE_not0 is
    the log-sum-exp over the valid keys other than the first.  By [MoE] s2 this
    is 1 - A_0, the output scale the first token imposes when its value is 0.
    A row whose first key is not valid gets 1; a row with no valid key gets 0.
    """
    q, k = _as64(q), _as64(k)
    T, hq, _ = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    gate = np.zeros((T, hq))
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        L = t1 - t0
        if L == 0:
            continue
        for g in range(hkv):
            M = sample_mask(L, n_sink, window, _blocks_of(block_indices, qoff, b, g), block_size)
            for h in range(hq):
                if kv_head(h, hq, hkv) != g:
                    continue
                x = scale * (q[t0:t1, h, :] @ k[t0:t1, g, :].T)
                x = np.where(M, x, -np.inf)
                x0 = x[:, 0].copy()                          # first-token score (-inf if not valid)
                rest = x.copy()
                rest[:, 0] = -np.inf
                lse_not0 = logsumexp_rows(rest)
                empty = ~np.isfinite(x0) & ~np.isfinite(lse_not0)
                with np.errstate(over="ignore", invalid="ignore"):
                    z = np.where(empty, 0.0, lse_not0 - np.where(np.isfinite(x0), x0, -np.inf))
                    G = 1.0 / (1.0 + np.exp(-z))             # sigma(LSE_not0 - x_i0)
                gate[t0:t1, h] = np.where(empty, 0.0, G)
    return gate


def head_importance(gate):
    """Imp_h = (1/|T|) sum_i G_ih: the mean gate of each head over the rows
    ([MoE] s4); 0 for no rows."""
    g = np.asarray(gate, dtype=np.float64)
    if g.shape[0] == 0:
        return np.zeros(g.shape[1])
    return g.sum(axis=0) / g.shape[0]


def bwd(q, k, v, cu_seqlens, scale, do, n_sink=0, window=0, block_indices=None,
        block_size=64, sink=None):
    """Backward: returns (dQ, dK, dV, dsink) in float64 (dsink None without sink).

    Re-runs the forward to get P (built from L_new, [Notes] s8) and O_new, then
    Delta = rowsum(dO * O_new) ([Notes] s7), the score gradient
    P * (dO V^T - Delta) ([Notes] s8), dQ = alpha dS K, dK = alpha dS^T Q and
    dV = P^T dO summed over the query heads of each KV group, and
    dsink_h = -sum_i Delta_ih (1 - s_ih) ([Notes] s7, boxed equation).
    """
    q, k, v, do, a = _as64(q), _as64(k), _as64(v), _as64(do), _as64(sink)
    T, hq, D = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta_all = np.zeros((T, hq))
    s_all = np.ones((T, hq))
    for b in range(len(cu) - 1):
        t0, t1 = int(cu[b]), int(cu[b + 1])
        L = t1 - t0
        if L == 0:
            continue
        for g in range(hkv):
            M = sample_mask(L, n_sink, window, _blocks_of(block_indices, qoff, b, g), block_size)
            for h in range(hq):
                if kv_head(h, hq, hkv) != g:
                    continue
                Q, K, V, dO = q[t0:t1, h], k[t0:t1, g], v[t0:t1, g], do[t0:t1, h]
                x = np.where(M, scale * (Q @ K.T), -np.inf)
                lorig = logsumexp_rows(x)
                lnew, s, _ = _sink_terms(lorig, None if a is None else a[h])
                safe = np.where(np.isfinite(lnew), lnew, 0.0)
                P = np.where(M, np.exp(x - safe[:, None]), 0.0)
                O = P @ V                                   # O_new
                delta = np.sum(dO * O, axis=1)              # Delta_ih
                dP = dO @ V.T                               # <dO_ih, V_jg>
                dS = P * (dP - delta[:, None])              # d loss / d x_ij
                dq[t0:t1, h] = scale * (dS @ K)
                dk[t0:t1, g] += scale * (dS.T @ Q)
                dv[t0:t1, g] += P.T @ dO
                delta_all[t0:t1, h] = delta
                s_all[t0:t1, h] = s
    dsink = None
    if a is not None:
        dsink = -np.sum(delta_all * (1.0 - s_all), axis=0)
    return dq, dk, dv, dsink


def decode(q, k_cache, v_cache, scale, cache_seqlens=None, sink=None):
    """One query per sequence against its rolling cache.

    q [B,Hq,D]; caches [B,S,Hkv,D].  The valid keys are the first
    cache_seqlens[b] slots (all S when None), in any position order: the cache
    keeps the first tokens plus a recent window ([QA] core idea; [Notes] s2),
    and the current token's K/V is already in it, so no causal or window mask
    applies.  Returns (O, lse = L_orig, s).
    """
    q, kc, vc, a = _as64(q), _as64(k_cache), _as64(v_cache), _as64(sink)
    B, hq, D = q.shape
    S, hkv = kc.shape[1], kc.shape[2]
    o = np.zeros((B, hq, D))
    lse = np.full((B, hq), -np.inf)
    s_out = np.ones((B, hq))
    for b in range(B):
        n = S if cache_seqlens is None else int(cache_seqlens[b])
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            x = scale * (kc[b, :n, g, :] @ q[b, h])
            lorig = logsumexp_rows(x[None, :])[0]
            lnew, s, _ = _sink_terms(np.array([lorig]), None if a is None else a[h])
            lnew, s = lnew[0], s[0]
            p = np.exp(x - lnew) if np.isfinite(lnew) else np.zeros(n)
            o[b, h] = p @ vc[b, :n, g, :]
            lse[b, h] = lorig
            s_out[b, h] = s
    return o, lse, s_out


# ---------------------------------------------------------------------------
# The same definitions evaluated for chosen output rows only (full-size checks)
# ---------------------------------------------------------------------------

def _row_keys(cu, qoff, t, g, n_sink, window, block_indices, block_size):
    """Packed indices of the keys valid for query token t and KV head g."""
    b = int(np.searchsorted(cu, t, side="right") - 1)
    t0, t1 = int(cu[b]), int(cu[b + 1])
    i = t - t0
    j = np.arange(i + 1)
    keep = np.ones(i + 1, dtype=bool)
    if window > 0:
        keep &= (j < n_sink) | (i - j < window)
    if block_indices is not None:
        row = np.asarray(block_indices)[qoff[b] + i // block_size, g]
        sel = np.zeros(i + 1, dtype=bool)
        for kb in row:
            if kb >= 0:
                sel |= (j // block_size) == kb
        keep &= sel
    return t0 + j[keep], b


def _row_state(q, k, v, cu, qoff, t, h, scale, n_sink, window, block_indices, block_size, a):
    """The forward quantities of query row (t, h), in float64 (only the rows
    read are converted)."""
    hq, hkv = q.shape[1], k.shape[1]
    g = kv_head(h, hq, hkv)
    keys, _ = _row_keys(cu, qoff, t, g, n_sink, window, block_indices, block_size)
    kk = np.asarray(k[keys, g, :], dtype=np.float64)
    x = scale * (kk @ np.asarray(q[t, h, :], dtype=np.float64))
    lorig = logsumexp_rows(x[None, :])[0]
    lnew, s, _ = _sink_terms(np.array([lorig]), None if a is None else float(a[h]))
    lnew, s = lnew[0], s[0]
    p = np.exp(x - lnew) if np.isfinite(lnew) else np.zeros(len(keys))
    o = p @ np.asarray(v[keys, g, :], dtype=np.float64)
    return keys, g, p, o, lorig, s


def fwd_rows(q, k, v, cu_seqlens, scale, rows, n_sink=0, window=0, block_indices=None,
             block_size=64, sink=None):
    """Forward for the given (token, head) pairs only: (O [n,D], lse [n], s [n])."""
    a = _as64(sink)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    outs, lses, ss = [], [], []
    for t, h in rows:
        _, _, _, o, lorig, s = _row_state(q, k, v, cu, qoff, int(t), int(h), scale,
                                          n_sink, window, block_indices, block_size, a)
        outs.append(o)
        lses.append(lorig)
        ss.append(s)
    return np.array(outs), np.array(lses), np.array(ss)


def first_token_gate_rows(q, k, cu_seqlens, scale, rows, n_sink=0, window=0, block_indices=None,
                          block_size=64):
    """First-token gate ([MoE] s5) for the given (token, head) pairs only [n]:
    sigma(LSE_not0 - x_i0) over the row's valid keys, 1 without a valid first
    key, 0 without any valid key (the same definition as first_token_gate)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    hq, hkv = q.shape[1], k.shape[1]
    out = []
    for t, h in rows:
        g = kv_head(int(h), hq, hkv)
        keys, b = _row_keys(cu, qoff, int(t), g, n_sink, window, block_indices, block_size)
        if len(keys) == 0:
            out.append(0.0)
            continue
        x = scale * (np.asarray(k[keys, g, :], dtype=np.float64)
                     @ np.asarray(q[int(t), int(h), :], dtype=np.float64))
        first = keys == cu[b]
        if not np.any(first):
            out.append(1.0)
            continue
        lse_not0 = logsumexp_rows(x[~first][None, :])[0]
        with np.errstate(over="ignore"):
            out.append(1.0 / (1.0 + np.exp(-(lse_not0 - x[first][0]))))
    return np.array(out)


def bwd_rows(q, k, v, cu_seqlens, scale, do, rows, n_sink=0, window=0, block_indices=None,
             block_size=64, sink=None):
    """dQ rows and the per-row dsink terms for the given (token, head) pairs.

    Returns (dQ [n,D], delta [n], one_minus_s [n]).
    """
    a = _as64(sink)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    dqs, deltas, oms = [], [], []
    for t, h in rows:
        t, h = int(t), int(h)
        keys, g, p, o, _, s = _row_state(q, k, v, cu, qoff, t, h, scale,
                                         n_sink, window, block_indices, block_size, a)
        dot = np.asarray(do[t, h], dtype=np.float64)
        delta = float(dot @ o)
        dp = np.asarray(v[keys, g, :], dtype=np.float64) @ dot
        ds = p * (dp - delta)
        dqs.append(scale * (ds @ np.asarray(k[keys, g, :], dtype=np.float64)))
        deltas.append(delta)
        oms.append(1.0 - s)
    return np.array(dqs), np.array(deltas), np.array(oms)


def _slab_columns(i0, i1, n_sink, window, blocks, block_size):
    """Sample-local keys that rows [i0, i1) might see: the causal keys [0, i1),
    narrowed to the kept first tokens plus [i0 - window + 1, i1) with a window
    and to the rows' selected blocks with block lists.  Only a superset is
    needed: mask_rows is applied on top."""
    cols = np.arange(i1, dtype=np.int64)
    if window > 0:
        cols = cols[(cols < n_sink) | (cols > i0 - window)]
    if blocks is not None:
        sel = set()
        for qb in range(i0 // block_size, (i1 - 1) // block_size + 1):
            sel.update(int(kb) for kb in blocks[qb] if kb >= 0)
        cols = cols[np.isin(cols // block_size, np.array(sorted(sel), dtype=np.int64))]
    return cols


def _slab(q, k, v, do, t0, i0, i1, h, g, scale, n_sink, window, blocks, block_size, a):
    """The forward and backward quantities of sample-local query rows
    [i0, i1) of one head (the sample starting at packed row t0), over the keys
    they can see: the same steps as fwd and bwd on that slab of the masked
    score matrix.  Returns (cols, P, dS, O, L_orig, s, Delta)."""
    cols = _slab_columns(i0, i1, n_sink, window, blocks, block_size)
    M = mask_rows(i0, i1, cols, n_sink, window, blocks, block_size)
    Q = np.asarray(q[t0 + i0:t0 + i1, h], dtype=np.float64)
    K = np.asarray(k[t0 + cols, g], dtype=np.float64)
    V = np.asarray(v[t0 + cols, g], dtype=np.float64)
    x = np.where(M, scale * (Q @ K.T), -np.inf)
    lorig = logsumexp_rows(x)
    lnew, s, _ = _sink_terms(lorig, None if a is None else a[h])
    safe = np.where(np.isfinite(lnew), lnew, 0.0)
    P = np.where(M, np.exp(x - safe[:, None]), 0.0)
    O = P @ V
    dS = delta = None
    if do is not None:
        dO = np.asarray(do[t0 + i0:t0 + i1, h], dtype=np.float64)
        delta = np.sum(dO * O, axis=1)
        dS = P * (dO @ V.T - delta[:, None])
    return cols, P, dS, O, lorig, s, delta


def _slab_rows(block_indices):
    """Rows per slab: one query block with block lists (each block has its own
    selection), else 256."""
    return 64 if block_indices is not None else 256


def bwd_kv_rows(q, k, v, cu_seqlens, scale, do, kv_rows, n_sink=0, window=0,
                block_indices=None, block_size=64, sink=None):
    """dK and dV rows for the given (key token, KV head) pairs.

    Each is a sum over every (query row, query head of the group) that sees
    the key: dK_j = alpha sum dS_ij Q_i and dV_j = sum P_ij dO_i ([Notes] s8),
    with every query row from the key on evaluated in slabs of rows (_slab).
    """
    a = _as64(sink)
    hq, hkv, D = q.shape[1], k.shape[1], q.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    dks = np.zeros((len(kv_rows), D))
    dvs = np.zeros((len(kv_rows), D))
    groups = {}
    for n, (tj, g) in enumerate(kv_rows):
        b = int(np.searchsorted(cu, int(tj), side="right") - 1)
        groups.setdefault((b, int(g)), []).append((n, int(tj) - int(cu[b])))
    rows_per = _slab_rows(block_indices)
    for (b, g), items in groups.items():
        t0, L = int(cu[b]), int(cu[b + 1] - cu[b])
        blocks = _blocks_of(block_indices, qoff, b, g)
        jmin = min(j for _, j in items)
        for h in range(hq):
            if kv_head(h, hq, hkv) != g:
                continue
            for i0 in range(jmin - jmin % rows_per, L, rows_per):
                i1 = min(L, i0 + rows_per)
                cols, P, dS, _, _, _, _ = _slab(q, k, v, do, t0, i0, i1, h, g, scale, n_sink, window,
                                                blocks, block_size, a)
                Q = np.asarray(q[t0 + i0:t0 + i1, h], dtype=np.float64)
                dO = np.asarray(do[t0 + i0:t0 + i1, h], dtype=np.float64)
                for n, j in items:
                    c = np.searchsorted(cols, j)
                    if c < len(cols) and cols[c] == j:
                        dks[n] += scale * (dS[:, c] @ Q)
                        dvs[n] += P[:, c] @ dO
    return dks, dvs


def fwd_bwd_heads(q, k, v, cu_seqlens, scale, do, heads, n_sink=0, window=0, block_indices=None,
                  block_size=64, sink=None):
    """Every row of the given query heads: O_new, L_orig, s and Delta, and
    dsink_h = -sum_i Delta_ih (1 - s_ih) ([Notes] s7, boxed equation), the
    rows evaluated in slabs (_slab).  Returns (O [T,n,D], lse [T,n], s [T,n],
    delta [T,n], dsink [n] or None)."""
    a = _as64(sink)
    T, hq, D = q.shape
    hkv = k.shape[1]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    qoff = _q_block_offsets(cu, block_size)
    n = len(heads)
    o = np.zeros((T, n, D))
    lse = np.full((T, n), -np.inf)
    s_all = np.ones((T, n))
    delta_all = np.zeros((T, n))
    rows_per = _slab_rows(block_indices)
    for x, h in enumerate(heads):
        g = kv_head(int(h), hq, hkv)
        for b in range(len(cu) - 1):
            t0, L = int(cu[b]), int(cu[b + 1] - cu[b])
            blocks = _blocks_of(block_indices, qoff, b, g)
            for i0 in range(0, L, rows_per):
                i1 = min(L, i0 + rows_per)
                _, _, _, O, lorig, s, delta = _slab(q, k, v, do, t0, i0, i1, int(h), g, scale, n_sink,
                                                    window, blocks, block_size, a)
                o[t0 + i0:t0 + i1, x] = O
                lse[t0 + i0:t0 + i1, x] = lorig
                s_all[t0 + i0:t0 + i1, x] = s
                delta_all[t0 + i0:t0 + i1, x] = delta
    dsink = None if a is None else -np.sum(delta_all * (1.0 - s_all), axis=0)
    return o, lse, s_all, delta_all, dsink
