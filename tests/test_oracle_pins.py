"""Pins for the float64 oracle, checked against what the pages and mathematics fix.

Each test ties the oracle to something other than itself: numbers printed on
the pages (tests/golden/worked_examples.json), closed forms, a second
formulation, a library routine (torch's scaled_dot_product_attention in
float64), brute-force loops on tiny inputs, or finite differences.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from streamingllm_sink_attn_amd import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------

def _two_key_case():
    """One head, D=2, alpha=1: query 1 sees keys 0 and 1 with logits ln 3 and 0,
    i.e. weights [0.75, 0.25] (the section-1 example)."""
    q = np.zeros((2, 1, 2))
    q[1, 0] = [math.log(3.0), 0.0]
    k = np.array([[[1.0, 0.0]], [[0.0, 0.0]]])
    v = np.array(GOLDEN["output_weighted_sum"]["V"])[:, None, :]
    return q, k, v, np.array([0, 2])


def test_worked_example_output():
    q, k, v, cu = _two_key_case()
    o, lse, s = oracle.fwd(q, k, v, cu, 1.0)
    np.testing.assert_allclose(o[1, 0], GOLDEN["output_weighted_sum"]["O"], rtol=0, atol=1e-15)
    # Z = 3 + 1 = 4
    assert abs(lse[1, 0] - math.log(4.0)) < 1e-15
    assert s[1, 0] == 1.0


def test_worked_example_sink_scale():
    g = GOLDEN["sink_scale"]
    q, k, v, cu = _two_key_case()
    # s = Z / (Z + e^a) = 0.2 with Z = 4  =>  e^a = 16
    a = np.array([math.log(16.0)])
    o, lse, s = oracle.fwd(q, k, v, cu, 1.0, sink=a)
    assert abs(s[1, 0] - g["s"]) < 1e-15
    np.testing.assert_allclose(o[1, 0], g["O_new"], atol=1e-15)
    assert abs(lse[1, 0] - math.log(4.0)) < 1e-15          # lse stays the real-token LSE
    # probabilities: one-hot values read the weights straight out of O
    v1 = np.eye(2)[:, None, :]
    o1, _, _ = oracle.fwd(q, k, v1, cu, 1.0, sink=a)
    np.testing.assert_allclose(o1[1, 0], g["real_probs"], atol=1e-15)
    assert abs(1.0 - o1[1, 0].sum() - g["sink_prob"]) < 1e-15
    # the same through the virtual-key formulation
    o2, s2 = oracle.fwd_virtual_key(q, k, v, cu, 1.0, sink=a)
    np.testing.assert_allclose(o2[1, 0], g["O_new"], atol=1e-15)
    assert abs(s2[1, 0] - g["s"]) < 1e-15


def test_worked_example_renormalisation():
    """Dropping a real first token renormalises the rest (section 2)."""
    g = GOLDEN["renormalisation"]
    # query 2 sees keys 0,1,2 with logits ln 16, ln 3, 0 -> 0.80 / 0.15 / 0.05
    q = np.zeros((3, 1, 3))
    q[2, 0] = [math.log(16.0), math.log(3.0), 0.0]
    k = np.eye(3)[:, None, :]
    v = np.eye(3)[:, None, :]
    o, _, _ = oracle.fwd(q, k, v, [0, 3], 1.0)
    np.testing.assert_allclose(o[2, 0], g["with_first_token"], atol=1e-15)
    # window 2 with no kept first token drops key 0 for query 2
    o, _, _ = oracle.fwd(q, k, v, [0, 3], 1.0, n_sink=0, window=2)
    np.testing.assert_allclose(o[2, 0], [0.0] + g["first_token_removed"], atol=1e-15)
    # keeping it as a StreamingLLM first token restores it
    o, _, _ = oracle.fwd(q, k, v, [0, 3], 1.0, n_sink=1, window=2)
    np.testing.assert_allclose(o[2, 0], g["with_first_token"], atol=1e-15)


def test_dynamic_range_example():
    """+10 against 99 x -10 (the softmax example of the FlashAttention-sink page)."""
    g = GOLDEN["dynamic_range"]
    n = g["scores"]["n_others"] + 1
    x = np.array([g["scores"]["first"]] + [g["scores"]["others"]] * (n - 1))
    # one query, keys e_j, q = x: score_j = x_j; one-hot values give the weights
    q = np.zeros((n, 1, n))
    q[n - 1, 0] = x
    k = np.eye(n)[:, None, :]
    v = np.eye(n)[:, None, :]
    o, _, _ = oracle.fwd(q, k, v, [0, n], 1.0)
    assert abs(o[n - 1, 0, 0] - g["first_share"]) < 1e-12
    np.testing.assert_allclose(o[n - 1, 0, 1:], g["other_share"], rtol=1e-6)


# ---------------------------------------------------------------------------
# Identities of the sink (section 4) and the gate form ([MoE] s2, s5)
# ---------------------------------------------------------------------------

def _small_case(seed=1, lengths=(37, 64, 5), hq=4, hkv=2, d=8, sink=True):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    a = _rand(rng, hq) if sink else None
    return q, k, v, W.cu_from_lengths(lengths), a


@pytest.mark.parametrize("mask", [dict(), dict(n_sink=3, window=9)])
def test_four_forms_of_s_and_output_scale(mask):
    q, k, v, cu, a = _small_case()
    scale = 0.3
    o, lse, s = oracle.fwd(q, k, v, cu, scale, sink=a, **mask)
    o0, lse0, s0 = oracle.fwd(q, k, v, cu, scale, **mask)
    Z = np.exp(lse)
    ea = np.exp(a)[None, :]
    np.testing.assert_array_equal(lse, lse0)                       # scores untouched by the sink
    np.testing.assert_allclose(s, Z / (Z + ea), rtol=1e-14)         # Z/(Z+e^a)
    sig = 1.0 / (1.0 + np.exp(-(lse - a[None, :])))                 # sigma(L_orig - a)
    np.testing.assert_allclose(s, sig, rtol=1e-14)
    _, s_vk = oracle.fwd_virtual_key(q, k, v, cu, scale, sink=a, **mask)
    np.testing.assert_allclose(s, s_vk, rtol=1e-13)                 # 1 - p_sink
    np.testing.assert_allclose(o, s[..., None] * o0, atol=1e-14)    # O_new = s O_orig
    assert np.all(s0 == 1.0)


@pytest.mark.parametrize("mask", [dict(), dict(n_sink=2, window=5)])
def test_virtual_zero_value_key(mask):
    """The sink equals one extra key of logit a_h (not scaled) with V = 0."""
    q, k, v, cu, a = _small_case(seed=2)
    o, _, s = oracle.fwd(q, k, v, cu, 0.7, sink=a, **mask)
    o2, s2 = oracle.fwd_virtual_key(q, k, v, cu, 0.7, sink=a, **mask)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(s, s2, atol=1e-13)


def test_zero_sink_is_off_by_one():
    """a = 0 adds exactly 1 to the denominator (section 4; the Zero Sink)."""
    q, k, v, cu, _ = _small_case(seed=3)
    hq = q.shape[1]
    o, lse, s = oracle.fwd(q, k, v, cu, 0.5, sink=np.zeros(hq))
    o0, lse0, _ = oracle.fwd(q, k, v, cu, 0.5)
    Z = np.exp(lse0)
    np.testing.assert_allclose(o, o0 * (Z / (Z + 1.0))[..., None], atol=1e-14)
    np.testing.assert_allclose(s, Z / (Z + 1.0), rtol=1e-14)


def test_relative_probabilities_invariant():
    """Ratios between real-token probabilities do not change (section 4)."""
    rng = np.random.default_rng(4)
    L, hq, d = 20, 2, 20
    q = _rand(rng, L, hq, d)
    k = _rand(rng, L, 1, d)
    v = np.eye(L)[:, None, :]                      # one-hot: O row = probability row
    a = np.array([1.5, -2.0])
    p_sink, _, s = oracle.fwd(q, k, v, [0, L], 0.4, sink=a)
    p_plain, _, _ = oracle.fwd(q, k, v, [0, L], 0.4)
    np.testing.assert_allclose(p_sink, p_plain * s[..., None], atol=1e-15)
    nz = p_plain > 0
    ratio = np.where(nz, p_sink / np.where(nz, p_plain, 1.0), 0.0)
    np.testing.assert_allclose(ratio[nz], np.broadcast_to(s[..., None], ratio.shape)[nz], rtol=1e-13)


def test_extreme_sinks():
    q, k, v, cu, _ = _small_case(seed=5)
    hq = q.shape[1]
    o0, _, _ = oracle.fwd(q, k, v, cu, 0.5)
    o, _, s = oracle.fwd(q, k, v, cu, 0.5, sink=np.full(hq, -40.0))
    np.testing.assert_allclose(o, o0, atol=1e-12)
    assert np.all(s > 1 - 1e-12)
    o, _, s = oracle.fwd(q, k, v, cu, 0.5, sink=np.full(hq, 60.0))
    assert np.all(np.abs(o) < 1e-20) and np.all(s < 1e-20)


# ---------------------------------------------------------------------------
# Textbook reductions
# ---------------------------------------------------------------------------

def _sdpa_causal(q, k, v, cu, scale):
    """torch's scaled_dot_product_attention in float64, per sample, GQA by repeat."""
    hq, hkv = q.shape[1], k.shape[1]
    out = np.zeros_like(q)
    for b in range(len(cu) - 1):
        t0, t1 = cu[b], cu[b + 1]
        Q = torch.from_numpy(q[t0:t1]).permute(1, 0, 2)
        K = torch.from_numpy(k[t0:t1]).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        V = torch.from_numpy(v[t0:t1]).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)
        O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
        out[t0:t1] = O.permute(1, 0, 2).numpy()
    return out


def test_no_sink_equals_sdpa():
    q, k, v, cu, _ = _small_case(seed=6, lengths=(50, 1, 31))
    o, lse, s = oracle.fwd(q, k, v, cu, 0.35)
    np.testing.assert_allclose(o, _sdpa_causal(q, k, v, cu, 0.35), atol=1e-13)
    # lse against torch.logsumexp of the causal scores
    for b in range(len(cu) - 1):
        t0, t1 = cu[b], cu[b + 1]
        for h in range(q.shape[1]):
            g = h // (q.shape[1] // k.shape[1])
            x = torch.from_numpy(0.35 * q[t0:t1, h] @ k[t0:t1, g].T)
            x = x.masked_fill(torch.ones_like(x, dtype=torch.bool).triu(1), float("-inf"))
            np.testing.assert_allclose(lse[t0:t1, h], torch.logsumexp(x, 1).numpy(), atol=1e-13)


def test_gqa_equals_repeated_mha():
    q, k, v, cu, a = _small_case(seed=7, hq=6, hkv=2)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    for mask in (dict(), dict(n_sink=2, window=7)):
        o1, l1, s1 = oracle.fwd(q, k, v, cu, 0.5, sink=a, **mask)
        o2, l2, s2 = oracle.fwd(q, kr, vr, cu, 0.5, sink=a, **mask)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
    do = np.random.default_rng(0).standard_normal(q.shape)
    g1 = oracle.bwd(q, k, v, cu, 0.5, do, sink=a)
    g2 = oracle.bwd(q, kr, vr, cu, 0.5, do, sink=a)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
    np.testing.assert_allclose(g1[1], g2[1].reshape(-1, 2, 3, q.shape[2]).sum(2), atol=1e-13)
    np.testing.assert_allclose(g1[2], g2[2].reshape(-1, 2, 3, q.shape[2]).sum(2), atol=1e-13)
    np.testing.assert_allclose(g1[3], g2[3], atol=1e-13)


def test_wide_window_and_all_blocks_equal_causal():
    q, k, v, cu, a = _small_case(seed=8, lengths=(70, 129))
    ref = oracle.fwd(q, k, v, cu, 0.5, sink=a)
    win = oracle.fwd(q, k, v, cu, 0.5, sink=a, n_sink=4, window=200)
    for x, y in zip(ref, win):
        np.testing.assert_array_equal(x, y)
    # every causal block selected (block size 16)
    lengths = np.diff(cu)
    rows = []
    for L in lengths:
        nqb = -(-L // 16)
        for qb in range(nqb):
            rows.append([list(range(qb + 1)) + [-1] * (nqb - qb - 1)] * k.shape[1])
    width = max(len(r[0]) for r in rows)
    bi = np.array([[rr + [-1] * (width - len(rr)) for rr in r] for r in rows], dtype=np.int32)
    blk = oracle.fwd(q, k, v, cu, 0.5, sink=a, block_indices=bi, block_size=16)
    for x, y in zip(ref, blk):
        np.testing.assert_array_equal(x, y)


# ---------------------------------------------------------------------------
# The valid set: brute force and closed-form counts
# ---------------------------------------------------------------------------

def _brute_mask(L, n_sink, window, blocks, bs):
    m = np.zeros((L, L), dtype=bool)
    for i in range(L):
        for j in range(L):
            ok = j <= i
            if window > 0 and not (j < n_sink or i - j < window):
                ok = False
            if blocks is not None and (j // bs) not in set(int(x) for x in blocks[i // bs] if x >= 0):
                ok = False
            m[i, j] = ok
    return m


@pytest.mark.parametrize("L,n_sink,window", [(1, 0, 0), (33, 4, 8), (40, 0, 5), (17, 20, 3), (64, 4, 16)])
def test_mask_brute_force(L, n_sink, window):
    np.testing.assert_array_equal(oracle.sample_mask(L, n_sink, window),
                                  _brute_mask(L, n_sink, window, None, 8))


def test_block_mask_brute_force():
    rng = np.random.default_rng(9)
    bi = W.sparse_block_lists(rng, [45], 1, n_random=2, block=8)[:, 0, :]
    bi[3, 0] = bi[3, 1]                     # duplicates are harmless
    for n_sink, window in ((0, 0), (2, 11)):
        np.testing.assert_array_equal(oracle.sample_mask(45, n_sink, window, bi, 8),
                                      _brute_mask(45, n_sink, window, bi, 8))


def _window_count(i, n_sink, W_):
    return min(i + 1, W_ + min(n_sink, max(0, i + 1 - W_)))


def test_visible_counts_closed_form_q_zero():
    """With Q = 0 every score is 0 and e^{lse} is the size of the valid set."""
    wl = W.tiny_f32()
    q = np.zeros_like(wl.q.f32)
    _, lse, _ = oracle.fwd(q, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale,
                           n_sink=wl.n_sink, window=wl.window)
    counts = np.exp(lse)
    want = np.array([_window_count(i, 4, 16) for i in range(64)], dtype=np.float64)
    np.testing.assert_allclose(counts, np.stack([want, want], 1), rtol=1e-13)
    assert int(round(counts[:, 0].sum())) == 1090
    # the streaming configuration's per-head count does not depend on the lengths (all >= 1028)
    lens = W.streaming_lengths()[1]
    tot = sum(sum(_window_count(i, 4, 1024) for i in range(L)) for L in lens)
    assert tot == 29_462_480


def test_block_sparse_closed_form_count():
    rng = np.random.default_rng(0)
    L, bs = 16 * 24, 16
    bi = W.sparse_block_lists(rng, [L], 1, n_random=5, block=bs)
    q = np.zeros((L, 1, 4))
    k = rng.standard_normal((L, 1, 4))
    _, lse, _ = oracle.fwd(q, k, k, [0, L], 1.0, block_indices=bi, block_size=bs)
    counts = np.exp(lse[:, 0])
    want = [bs * min(5 + 1, qb) + r + 1 for qb in range(L // bs) for r in range(bs)]
    np.testing.assert_allclose(counts, want, rtol=1e-13)


def test_empty_rows():
    """Block lists that miss the diagonal leave rows with no valid key."""
    rng = np.random.default_rng(10)
    L = 16
    q, k, v = _rand(rng, L, 2, 4), _rand(rng, L, 1, 4), _rand(rng, L, 1, 4)
    bi = np.array([[[-1]], [[0]]], dtype=np.int32)      # block 0 selects nothing
    o, lse, s = oracle.fwd(q, k, v, [0, L], 1.0, block_indices=bi, block_size=8, sink=np.array([0.3, -1.0]))
    assert np.all(o[:8] == 0) and np.all(np.isneginf(lse[:8])) and np.all(s[:8] == 0)
    o, lse, s = oracle.fwd(q, k, v, [0, L], 1.0, block_indices=bi, block_size=8)
    assert np.all(o[:8] == 0) and np.all(np.isneginf(lse[:8])) and np.all(s[:8] == 1)
    do = _rand(rng, L, 2, 4)
    dq, dk, dv, dsink = oracle.bwd(q, k, v, [0, L], 1.0, do, block_indices=bi, block_size=8,
                                   sink=np.array([0.3, -1.0]))
    assert np.all(dq[:8] == 0) and np.all(np.isfinite(dsink))


# ---------------------------------------------------------------------------
# Gradients: finite differences of the forward
# ---------------------------------------------------------------------------

def _loss(q, k, v, cu, scale, do, a, mask):
    o, _, _ = oracle.fwd(q, k, v, cu, scale, sink=a, **mask)
    return float(np.sum(do * o))


@pytest.mark.parametrize("mask", [dict(n_sink=2, window=5), dict()])
def test_gradients_finite_differences(mask):
    """Central differences over every element of Q, K, V and every sink logit."""
    rng = np.random.default_rng(11)
    lengths = (9, 6)
    T, hq, hkv, d = sum(lengths), 4, 2, 3
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    a = _rand(rng, hq)
    do = _rand(rng, T, hq, d)
    cu = W.cu_from_lengths(lengths)
    scale = 0.6
    dq, dk, dv, dsink = oracle.bwd(q, k, v, cu, scale, do, sink=a, **mask)
    eps = 1e-6

    def fd(arr, idx, which):
        args = dict(q=q, k=k, v=v, a=a)
        plus, minus = arr.copy(), arr.copy()
        plus[idx] += eps
        minus[idx] -= eps
        args[which] = plus
        lp = _loss(args["q"], args["k"], args["v"], cu, scale, do, args["a"], mask)
        args[which] = minus
        lm = _loss(args["q"], args["k"], args["v"], cu, scale, do, args["a"], mask)
        return (lp - lm) / (2 * eps)

    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("a", a, dsink)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            num[idx] = fd(arr, idx, name)
        tol = 1e-6 * (1 + np.max(np.abs(grad)))
        assert np.max(np.abs(num - grad)) < tol, name


def test_dsink_forms_and_sign():
    """dsink = -sum Delta (1 - s) = -sum Delta p_sink, and d O / d a = -(1 - s) O_new."""
    q, k, v, cu, a = _small_case(seed=12)
    do = np.random.default_rng(1).standard_normal(q.shape)
    _, _, _, dsink = oracle.bwd(q, k, v, cu, 0.5, do, sink=a, n_sink=3, window=6)
    o, lse, s = oracle.fwd(q, k, v, cu, 0.5, sink=a, n_sink=3, window=6)
    delta = np.sum(do * o, axis=-1)
    p_sink = np.exp(a[None, :] - np.logaddexp(lse, a[None, :]))
    np.testing.assert_allclose(dsink, -np.sum(delta * p_sink, axis=0), rtol=1e-12)
    # dO/da by differences
    eps = 1e-6
    ap, am = a.copy(), a.copy()
    ap[0] += eps
    am[0] -= eps
    dO = (oracle.fwd(q, k, v, cu, 0.5, sink=ap, n_sink=3, window=6)[0][:, 0]
          - oracle.fwd(q, k, v, cu, 0.5, sink=am, n_sink=3, window=6)[0][:, 0]) / (2 * eps)
    np.testing.assert_allclose(dO, -(1 - s[:, 0:1]) * o[:, 0], atol=1e-8)
    # sign: one query with Delta > 0 gives a negative sink gradient
    do1 = np.zeros_like(q)
    do1[5, 0] = o[5, 0]                          # Delta_50 = |O|^2 > 0
    _, _, _, ds1 = oracle.bwd(q, k, v, cu, 0.5, do1, sink=a, n_sink=3, window=6)
    assert ds1[0] < 0 and np.all(ds1[1:] == 0)


# ---------------------------------------------------------------------------
# Decode and the row-wise evaluators
# ---------------------------------------------------------------------------

def test_decode_matches_prefill_last_row_and_is_permutation_invariant():
    rng = np.random.default_rng(13)
    L, hq, hkv, d = 40, 4, 2, 8
    q, k, v = _rand(rng, L, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)
    a = _rand(rng, hq)
    n_sink, window = 3, 10
    o, lse, s = oracle.fwd(q, k, v, [0, L], 0.4, sink=a, n_sink=n_sink, window=window)
    keep = np.r_[0:n_sink, L - window:L]            # the rolling cache at step L-1
    perm = rng.permutation(len(keep))
    kc = k[keep][perm][None]
    vc = v[keep][perm][None]
    od, ld, sd = oracle.decode(q[L - 1][None], kc, vc, 0.4, sink=a)
    np.testing.assert_allclose(od[0], o[L - 1], atol=1e-13)
    np.testing.assert_allclose(ld[0], lse[L - 1], atol=1e-13)
    np.testing.assert_allclose(sd[0], s[L - 1], atol=1e-13)
    # cache_seqlens: only the first n slots count
    od2, _, _ = oracle.decode(q[L - 1][None], np.concatenate([kc, kc], 1), np.concatenate([vc, vc * 9], 1),
                              0.4, cache_seqlens=[len(keep)], sink=a)
    np.testing.assert_allclose(od2[0], o[L - 1], atol=1e-13)


def test_row_evaluators_match_full():
    rng = np.random.default_rng(14)
    lengths = (70, 45)
    T, hq, hkv, d = sum(lengths), 4, 2, 8
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    do = _rand(rng, T, hq, d)
    a = _rand(rng, hq)
    cu = W.cu_from_lengths(lengths)
    bi = W.sparse_block_lists(rng, lengths, hkv, n_random=2, block=16)
    for mask in (dict(n_sink=2, window=9), dict(block_indices=bi, block_size=16), dict()):
        o, lse, s = oracle.fwd(q, k, v, cu, 0.5, sink=a, **mask)
        dq, dk, dv, dsink = oracle.bwd(q, k, v, cu, 0.5, do, sink=a, **mask)
        rows = [(0, 0), (5, 3), (69, 1), (70, 2), (114, 3), (100, 0)]
        ro, rl, rs = oracle.fwd_rows(q, k, v, cu, 0.5, rows, sink=a, **mask)
        rdq, rdelta, rom = oracle.bwd_rows(q, k, v, cu, 0.5, do, rows, sink=a, **mask)
        for n, (t, h) in enumerate(rows):
            np.testing.assert_allclose(ro[n], o[t, h], atol=1e-13)
            np.testing.assert_allclose(rl[n], lse[t, h], atol=1e-13)
            np.testing.assert_allclose(rs[n], s[t, h], atol=1e-13)
            np.testing.assert_allclose(rdq[n], dq[t, h], atol=1e-12)
        kv_rows = [(0, 0), (3, 1), (40, 0), (70, 1), (114, 0), (1, 0), (69, 1)]
        rdk, rdv = oracle.bwd_kv_rows(q, k, v, cu, 0.5, do, kv_rows, sink=a, **mask)
        for n, (t, g) in enumerate(kv_rows):
            np.testing.assert_allclose(rdk[n], dk[t, g], atol=1e-12)
            np.testing.assert_allclose(rdv[n], dv[t, g], atol=1e-12)
        heads = [3, 0, 2]
        ho, hl, hs, hdelta, hds = oracle.fwd_bwd_heads(q, k, v, cu, 0.5, do, heads, sink=a, **mask)
        for x, h in enumerate(heads):
            np.testing.assert_allclose(ho[:, x], o[:, h], atol=1e-13)
            np.testing.assert_allclose(hl[:, x], lse[:, h], atol=1e-13)
            np.testing.assert_allclose(hs[:, x], s[:, h], atol=1e-13)
            np.testing.assert_allclose(hdelta[:, x], np.sum(do[:, h] * o[:, h], axis=1), atol=1e-12)
            np.testing.assert_allclose(hds[x], dsink[h], rtol=1e-12, atol=1e-12)


def test_row_evaluators_match_full_long_rows():
    """Rows past one slab (256 rows; 64 with block lists): the slab evaluators
    against the full oracle, with windows, kept tokens and block lists."""
    rng = np.random.default_rng(15)
    lengths = (600, 290)
    T, hq, hkv, d = sum(lengths), 2, 1, 8
    q, k, v = _rand(rng, T, hq, d), _rand(rng, T, hkv, d), _rand(rng, T, hkv, d)
    do = _rand(rng, T, hq, d)
    a = _rand(rng, hq)
    cu = W.cu_from_lengths(lengths)
    bi = W.sparse_block_lists(rng, lengths, hkv, n_random=3, block=64)
    for mask in (dict(n_sink=4, window=100), dict(block_indices=bi, block_size=64),
                 dict(n_sink=0, window=300), dict()):
        _, dk, dv, dsink = oracle.bwd(q, k, v, cu, 0.5, do, sink=a, **mask)
        kv_rows = [(0, 0), (2, 0), (64, 0), (299, 0), (599, 0), (600, 0), (700, 0), (889, 0)]
        rdk, rdv = oracle.bwd_kv_rows(q, k, v, cu, 0.5, do, kv_rows, sink=a, **mask)
        for n, (t, g) in enumerate(kv_rows):
            np.testing.assert_allclose(rdk[n], dk[t, g], atol=1e-12)
            np.testing.assert_allclose(rdv[n], dv[t, g], atol=1e-12)
        *_, hds = oracle.fwd_bwd_heads(q, k, v, cu, 0.5, do, [1, 0], sink=a, **mask)
        np.testing.assert_allclose(hds, dsink[[1, 0]], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# First-token gate and head importance ("Paper notes: Attention Sink and the
# native MoE in attention layers", s2, s4, s5)
# ---------------------------------------------------------------------------

def test_first_token_gate_worked_example():
    """Section-1 weights [0.75, 0.25]: the first token takes 0.75, so the
    vanilla gate G = 1 - A_0 is 0.25; query 0 sees only the first token (0)."""
    q, k, _, cu = _two_key_case()
    g = oracle.first_token_gate(q, k, cu, 1.0)
    w = GOLDEN["output_weighted_sum"]["weights"]
    assert abs(g[1, 0] - (1.0 - w[0])) < 1e-15
    assert g[0, 0] == 0.0
    assert abs(oracle.head_importance(g)[0] - (1.0 - w[0]) / 2) < 1e-15


def _first_token_probe(rng, mask, hq=4, hkv=2, D=6, lengths=(37, 70, 1)):
    """V one-hot on each sample's first token: the forward's output column 0
    is then the attention weight A_0 of every row (no sink)."""
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = _rand(rng, T, hq, D)
    k = _rand(rng, T, hkv, D)
    v = np.zeros((T, hkv, D))
    v[cu[:-1], :, 0] = 1.0
    o, lse, _ = oracle.fwd(q, k, v, cu, 0.4, **mask)
    return q, k, cu, o[:, :, 0], lse


@pytest.mark.parametrize("mask", [dict(), dict(n_sink=3, window=9), dict(n_sink=0, window=5),
                                  "blocks"])
def test_first_token_gate_is_one_minus_first_token_weight(mask):
    """The LSE form sigma(LSE_not0 - x_0) of s5 equals 1 - A_0 of s2, A_0 read
    through the forward's P V with a one-hot first value."""
    rng = np.random.default_rng(21)
    if mask == "blocks":
        lengths = (130, 64)
        nqb = 3 + 1
        bi = np.full((nqb, 2, 2), -1, dtype=np.int32)
        bi[0, :, 0] = 0
        bi[1, 0, :] = [1, 0]          # head 0: both blocks; head 1: block 1 only (no first key)
        bi[1, 1, 0] = 1
        bi[2, :, 0] = 2               # diagonal only: no first key
        bi[3, :, 0] = 0
        mask = dict(block_indices=bi)
        q, k, cu, a0, lse = _first_token_probe(rng, mask, lengths=lengths)
    else:
        q, k, cu, a0, lse = _first_token_probe(rng, mask)
    g = oracle.first_token_gate(q, k, cu, 0.4, **mask)
    valid = np.isfinite(lse)
    np.testing.assert_allclose(g[valid], 1.0 - a0[valid], rtol=0, atol=1e-12)
    assert np.all(g[~valid] == 0.0)
    if mask.get("window", 0) > 0 and mask.get("n_sink", 0) == 0:
        # rows past the window cannot see the first token: G = 1 exactly
        L0 = 37
        assert np.all(g[5:L0] == 1.0)


def test_implicit_gate_identity():
    """s2: with a zero first value, vanilla attention equals G times the
    attention over the other tokens (the sample with its first token removed)."""
    rng = np.random.default_rng(22)
    L, hq, hkv, D = 29, 4, 2, 8
    q, k, v = _rand(rng, L, hq, D), _rand(rng, L, hkv, D), _rand(rng, L, hkv, D)
    v0 = v.copy()
    v0[0] = 0.0
    o, _, _ = oracle.fwd(q, k, v0, [0, L], 0.35)
    g = oracle.first_token_gate(q, k, [0, L], 0.35)
    o_rest, _, _ = oracle.fwd(q[1:], k[1:], v[1:], [0, L - 1], 0.35)
    np.testing.assert_allclose(o[1:], g[1:, :, None] * o_rest, rtol=0, atol=1e-12)
    assert np.all(o[0] == 0.0) and np.all(g[0] == 0.0)


def test_first_token_gate_rows_match_full():
    rng = np.random.default_rng(23)
    lengths = (150, 40)
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k = _rand(rng, T, 4, 8), _rand(rng, T, 2, 8)
    for mask in (dict(), dict(n_sink=2, window=30), dict(n_sink=0, window=30)):
        full = oracle.first_token_gate(q, k, cu, 0.3, **mask)
        rows = [(0, 0), (1, 3), (60, 1), (149, 2), (150, 0), (189, 3)]
        got = oracle.first_token_gate_rows(q, k, cu, 0.3, rows, **mask)
        np.testing.assert_allclose(got, [full[t, h] for t, h in rows], rtol=0, atol=1e-13)


def test_head_importance_is_the_mean_gate():
    g = np.array([[0.0, 1.0], [0.5, 1.0], [1.0, 0.25]])
    np.testing.assert_allclose(oracle.head_importance(g), [0.5, 0.75], atol=1e-15)
    assert np.all(oracle.head_importance(np.zeros((0, 3))) == 0.0)


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by one of the checks above
# ---------------------------------------------------------------------------

def test_planted_mistakes_are_caught(monkeypatch):
    """A wrong sign on the sink term, a sink multiplied by alpha or a dropped
    Delta each break a pin that the real oracle passes."""
    from oracle import sink_attn_oracle as so
    q, k, v, cu = _two_key_case()
    a = np.array([math.log(16.0)])
    real = so._sink_terms

    def wrong_sign(lorig, a_):
        return real(lorig, None if a_ is None else -a_)
    monkeypatch.setattr(so, "_sink_terms", wrong_sign)
    o, _, s = so.fwd(q, k, v, cu, 1.0, sink=a)
    assert abs(s[1, 0] - 0.2) > 0.1
    monkeypatch.setattr(so, "_sink_terms", real)
    # alpha applied to the sink logit: a different s for alpha != 1
    q2 = q * 2.0
    o, _, s = so.fwd(q2, k, v, cu, 0.5, sink=a)
    assert abs(s[1, 0] - 0.2) < 1e-15
    o_bad, _, s_bad = so.fwd(q2, k, v, cu, 0.5, sink=a * 0.5)
    assert abs(s_bad[1, 0] - 0.2) > 0.1
    # gate with the first token left inside the log-sum-exp: sigma(LSE - x_0)
    # = 1 / (1 + A_0) instead of 1 - A_0, far from the worked example's 0.25
    qg, kg, _, cug = _two_key_case()
    lse_all = math.log(4.0)
    wrong = 1.0 / (1.0 + math.exp(-(lse_all - math.log(3.0))))
    right = so.first_token_gate(qg, kg, cug, 1.0)[1, 0]
    assert abs(right - 0.25) < 1e-15 and abs(wrong - 0.25) > 0.3
