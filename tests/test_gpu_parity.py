"""GPU parity: the HIP path through the C ABI against the float64 oracle on the
same seeded inputs, element by element, at sizes that span several tiles and
ragged tails."""
import numpy as np
import pytest
import torch

import oracle
import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import (DEV, assert_dsink, assert_grad, assert_lse, assert_out, check_bwd_full,
                         check_fwd_full, dev, host, oracle_kwargs, prefill_args, run_bwd, run_fwd,
                         tol_for)

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)


# ---------------------------------------------------------------------------
# The tiny float32 workload: forward and backward, generic kernels
# ---------------------------------------------------------------------------

def test_tiny_f32_fwd_bwd():
    wl = W.tiny_f32()
    _announce("tiny_f32")
    out = run_fwd(wl)
    ro, rl, rs = check_fwd_full(wl, out)
    dq, dk, dv, dsink = run_bwd(wl, out[0], out[1])
    rdq, rdk, rdv, rds = oracle.bwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale,
                                    wl.do.f32, **oracle_kwargs(wl))
    tol = tol_for("f32")
    assert_grad(host(dq), rdq, tol, "dQ")
    assert_grad(host(dk), rdk, tol, "dK")
    assert_grad(host(dv), rdv, tol, "dV")
    assert_dsink(host(dsink), rds, tol)


# ---------------------------------------------------------------------------
# bf16 forward variants (MFMA path for D=128, generic otherwise)
# ---------------------------------------------------------------------------

FWD_CASES = {
    "dense_g4": dict(lengths=(200, 64, 1, 129), hq=8, hkv=2),
    "dense_g1": dict(lengths=(130, 257), hq=2, hkv=2),
    "dense_g2": dict(lengths=(300, 5), hq=4, hkv=2),
    "dense_g8": dict(lengths=(190,), hq=16, hkv=2),
    "dense_g3": dict(lengths=(150, 70), hq=6, hkv=2),
    # workgroup geometry: 8 heads per workgroup and two head groups per KV
    # head (G=16), one head of eight 32-row wavefronts (G=5), three head
    # groups of four heads (G=12)
    "dense_g16": dict(lengths=(140, 33), hq=32, hkv=2),
    "dense_g5": dict(lengths=(300,), hq=5, hkv=1),
    "window_g12": dict(lengths=(260, 90), hq=12, hkv=1, n_sink=4, window=70),
    "window_sink4": dict(lengths=(400, 77, 260), hq=8, hkv=2, n_sink=4, window=100),
    "window_nosinktok": dict(lengths=(333,), hq=4, hkv=1, n_sink=0, window=50),
    "window_bigsink": dict(lengths=(420,), hq=4, hkv=1, n_sink=70, window=10),
    "window_wide": dict(lengths=(300, 64), hq=4, hkv=2, n_sink=4, window=1000),
    "window_g2": dict(lengths=(390, 129), hq=4, hkv=2, n_sink=4, window=64),
    # a window of one key (the diagonal only, plus the kept tokens) and one
    # far longer than any sample (every causal key): the mask bounds' ends
    "window_one": dict(lengths=(200, 65), hq=4, hkv=1, n_sink=4, window=1),
    "window_huge": dict(lengths=(300, 70), hq=4, hkv=2, n_sink=4, window=2 ** 30),
    "blocks_g4": dict(lengths=(700, 130), hq=8, hkv=2, block_lists=dict(n_random=3)),
    "blocks_g1": dict(lengths=(513,), hq=2, hkv=2, block_lists=dict(n_random=2)),
    "blocks_window": dict(lengths=(640,), hq=4, hkv=1, n_sink=4, window=150,
                          block_lists=dict(n_random=4)),
    "blocks_nodiag": dict(lengths=(300,), hq=4, hkv=1,
                          block_lists=dict(n_random=2, diagonal=False, always_first=False)),
    "no_sink": dict(lengths=(250, 99), hq=8, hkv=2, sink=False),
    "stress_sink": dict(lengths=(260,), hq=4, hkv=1, n_sink=4, window=64, sink_shift=4.0),
    "d64_generic": dict(lengths=(150, 40), hq=4, hkv=2, d=64),
    # key tiles with more than 128 (head, query tile) iterations: the
    # backward splits them over several work items
    "dense_g8_long": dict(lengths=(1200, 70), hq=16, hkv=2),
    "window_split": dict(lengths=(2200,), hq=8, hkv=1, n_sink=4, window=256),
    "blocks_split": dict(lengths=(1500,), hq=16, hkv=2, block_lists=dict(n_random=4)),
    # empty samples between and after others (cu_seqlens repeats a value)
    "window_empty": dict(lengths=(130, 0, 70, 0), hq=4, hkv=2, n_sink=4, window=50),
    "blocks_empty": dict(lengths=(0, 130, 0, 70), hq=4, hkv=2, block_lists=dict(n_random=2)),
}


def _wl(name, seed=0, **over):
    c = dict(FWD_CASES[name])
    c.update(over)
    d = c.pop("d", 128)
    return W.make_prefill(name, c.pop("lengths"), c.pop("hq"), c.pop("hkv"), d, seed=seed, **c)


@pytest.mark.parametrize("name", sorted(FWD_CASES))
def test_fwd_bf16_variants(name):
    wl = _wl(name)
    _announce(f"fwd {name}")
    check_fwd_full(wl, run_fwd(wl))


@pytest.mark.parametrize("a", [0.0, 20.0, -20.0])
def test_fwd_fixed_sink_values(a):
    wl = _wl("window_sink4", seed=3)
    wl.sink = np.full(wl.hq, a, dtype=np.float32)
    _announce(f"fwd fixed sink {a}")
    check_fwd_full(wl, run_fwd(wl))


def test_fwd_dynamic_range_example():
    """+10 against 99 x -10 (the softmax example of the FlashAttention-sink
    page) through the MFMA path: scores built from one-hot keys."""
    n, d = 100, 128
    q = np.zeros((n, 1, d), np.float32)
    k = np.zeros((n, 1, d), np.float32)
    for j in range(n):
        k[j, 0, j] = 1.0
    q[n - 1, 0, 0] = 10.0
    q[n - 1, 0, 1:n] = -10.0
    v = np.zeros((n, 1, d), np.float32)
    for j in range(n):
        v[j, 0, j] = 1.0
    bits = lambda x: W.round_to_bf16_bits(x)
    wl = W.Prefill("dyn", "bf16", W.cu_from_lengths([n]), 1, 1, d, 0, 0, 64, None,
                   W.Tensor(q, bits(q)), W.Tensor(k, bits(k)), W.Tensor(v, bits(v)), None, None, 1.0)
    _announce("fwd dynamic range")
    o, lse, s = run_fwd(wl)
    row = host(o)[n - 1, 0]
    assert abs(row[0] - 0.9999997959) < 4e-3          # bf16 output rounding
    assert np.all(np.abs(row[1:n]) < 1e-6)


# ---------------------------------------------------------------------------
# The visited key set, bit for bit
# ---------------------------------------------------------------------------

VISIT_CASES = ["dense_g4", "dense_g2", "dense_g1", "window_sink4", "window_bigsink", "window_g2",
               "window_one", "window_huge", "blocks_g4", "blocks_g1", "blocks_window", "blocks_nodiag",
               "window_empty", "blocks_empty"]


@pytest.mark.parametrize("name", VISIT_CASES)
def test_visit_map_bit_exact(name):
    wl = _wl(name)
    _announce(f"visit map {name}")
    _check_visit_map(wl)


@pytest.mark.parametrize("window", [0, 150])
def test_visit_map_messy_block_lists(window):
    wl = _wl("blocks_g4", seed=9, window=window, n_sink=4 if window else 0)
    wl.block_indices = _messy_block_lists(np.random.default_rng(21), wl.lengths, wl.hkv)
    _announce(f"visit map messy block lists window={window}")
    _check_visit_map(wl)


def _check_visit_map(wl):
    q, k, v, cu, bi, sink = prefill_args(wl)
    got = sa.debug_visit_map(q, k, cu, wl.max_seqlen, wl.n_sink, wl.window, bi).cpu().numpy()
    qoff = np.concatenate([[0], np.cumsum(-(-wl.lengths // 64))])
    off = 0
    for b, L in enumerate(wl.lengths):
        L = int(L)
        for g in range(wl.hkv):
            blocks = None if wl.block_indices is None else wl.block_indices[qoff[b]:qoff[b + 1], g, :]
            want = oracle.sample_mask(L, wl.n_sink, wl.window, blocks, 64)
            m = got[off:off + L * L].reshape(L, L).astype(bool)
            assert np.array_equal(m, want), f"sample {b} head {g}: {np.sum(m != want)} mismatches"
            off += L * L


def test_q_zero_counts_closed_form():
    """Q = 0: every score is 0 and e^{lse} is the number of valid keys."""
    wl = W.make_prefill("qzero", [1500, 1100, 64], 8, 2, 128, n_sink=4, window=1024, seed=1)
    wl.q = W.Tensor(np.zeros_like(wl.q.f32), np.zeros_like(wl.q.bits))
    _announce("q=0 counts")
    o, lse, s = run_fwd(wl)
    counts = np.exp(host(lse))
    want = []
    for L in wl.lengths:
        for i in range(int(L)):
            want.append(min(i + 1, 1024 + min(4, max(0, i + 1 - 1024))))
    want = np.repeat(np.array(want, dtype=np.float64)[:, None], wl.hq, axis=1)
    np.testing.assert_allclose(counts, want, rtol=2e-6)


# ---------------------------------------------------------------------------
# Backward (bf16) on small shapes
# ---------------------------------------------------------------------------

BWD_CASES = ["dense_g4", "window_sink4", "blocks_g4", "no_sink", "dense_g2", "blocks_nodiag",
             "d64_generic", "dense_g8_long", "window_split", "blocks_split", "dense_g1", "window_g2",
             "window_bigsink", "window_nosinktok", "window_wide", "window_one", "window_huge",
             "blocks_window", "dense_g3", "dense_g8", "stress_sink", "blocks_g1", "dense_g16", "dense_g5",
             "window_g12", "window_empty", "blocks_empty"]


def _check_bwd(wl, max_seqlen=None):
    check_bwd_full(wl, max_seqlen)


@pytest.mark.parametrize("name", BWD_CASES)
def test_bwd_bf16_variants(name):
    wl = _wl(name)
    _announce(f"bwd {name}")
    _check_bwd(wl)


def _sink_values(kind, hq):
    if kind == "mixed":
        return np.array([(-20.0, 0.0, 20.0)[h % 3] for h in range(hq)], np.float32)
    return np.full(hq, float(kind), np.float32)


@pytest.mark.parametrize("kind", ["0", "20", "-20", "mixed"])
@pytest.mark.parametrize("name", ["window_sink4", "blocks_g4", "dense_g4", "d64_generic"])
def test_bwd_extreme_sinks(name, kind):
    """The backward where p_sink matters most ("Attention Sink, Learnable Sink
    and dsink" s10 lists an extreme sink among the cases to validate): a = 0,
    a = +20 (s -> 0, O -> 0, p_sink -> 1), a = -20 (s -> 1, where 1 - s
    cancels and p_sink = exp(a - L_new) keeps its precision), and the three
    mixed across heads; dsink checked head by head."""
    wl = _wl(name, seed=11)
    wl.sink = _sink_values(kind, wl.hq)
    _announce(f"bwd extreme sink {name} a={kind}")
    _check_bwd(wl)


def _messy_block_lists(rng, lengths, hkv, width=6):
    """Block lists the workload generator never draws but the mask accepts
    ([Notes] s9-10: a query block attends to the key blocks its row lists):
    entries in random order, one selected block listed twice, the block after
    the query block (causally invisible), -1 between entries."""
    rows = []
    for L in lengths:
        nqb = -(-int(L) // 64)
        for qb in range(nqb):
            for _g in range(hkv):
                sel = [int(x) for x in rng.choice(qb + 1, size=min(qb + 1, 3), replace=False)]
                sel.append(sel[0])
                if qb + 1 < nqb:
                    sel.append(qb + 1)
                sel = (sel + [-1] * width)[:width]
                rng.shuffle(sel)
                rows.append(sel)
    return np.asarray(rows, dtype=np.int32).reshape(-1, hkv, width)


@pytest.mark.parametrize("window", [0, 150])
def test_fwd_bwd_messy_block_lists(window):
    wl = _wl("blocks_g4", seed=9, window=window, n_sink=4 if window else 0)
    wl.block_indices = _messy_block_lists(np.random.default_rng(21), wl.lengths, wl.hkv)
    _announce(f"fwd+bwd messy block lists window={window}")
    check_fwd_full(wl, run_fwd(wl))
    _check_bwd(wl)


@pytest.mark.parametrize("name", ["window_sink4", "dense_g8_long", "blocks_g4", "d64_generic"])
def test_fwd_bwd_max_seqlen_above_every_sample(name):
    """max_seqlen is an upper bound on the lengths: with four times the
    longest sample, the workgroups and key tiles past every sample do no work
    and the results match the oracle as before."""
    wl = _wl(name, seed=4)
    ms = 4 * wl.max_seqlen
    _announce(f"fwd+bwd max_seqlen x4 {name}")
    check_fwd_full(wl, run_fwd(wl, max_seqlen=ms))
    _check_bwd(wl, max_seqlen=ms)


def test_bwd_is_repeatable():
    """dsink is reduced in a fixed order: two runs give identical bits."""
    wl = _wl("window_sink4", seed=5)
    args = prefill_args(wl)
    o, lse, _ = run_fwd(wl, args)
    g1 = run_bwd(wl, o, lse, args)
    g2 = run_bwd(wl, o, lse, args)
    assert torch.equal(g1[3], g2[3])


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------

DECODE_CASES = {
    "d128_g8": dict(batch=5, slots=300, hq=16, hkv=2, d=128),
    "d128_g4_lens": dict(batch=4, slots=257, hq=8, hkv=2, d=128, cache_seqlens=[257, 1, 100, 64]),
    # more than 16 query heads per KV head: two head groups per KV head (the
    # second one partly empty with 20)
    "d128_g20": dict(batch=2, slots=200, hq=40, hkv=2, d=128, cache_seqlens=[200, 37]),
    "d128_g32": dict(batch=2, slots=130, hq=32, hkv=1, d=128),
    "d64": dict(batch=3, slots=100, hq=4, hkv=1, d=64),
    "f32": dict(batch=2, slots=70, hq=4, hkv=2, d=16, dtype="f32"),
    "no_sink": dict(batch=3, slots=200, hq=8, hkv=1, d=128, sink=False),
}


def _dwl(name, seed=0):
    c = dict(DECODE_CASES[name])
    return W.make_decode(name, c.pop("batch"), c.pop("slots"), c.pop("hq"), c.pop("hkv"), c.pop("d"),
                         seed=seed, **c)


def run_decode(wl, num_splits=0, perm=None):
    q = dev(wl.q, wl.dtype)
    kc, vc = dev(wl.k_cache, wl.dtype), dev(wl.v_cache, wl.dtype)
    if perm is not None:
        kc, vc = kc[:, perm].contiguous(), vc[:, perm].contiguous()
    csl = torch.from_numpy(wl.cache_seqlens).to(DEV) if wl.cache_seqlens is not None else None
    sink = torch.from_numpy(wl.sink).to(DEV) if wl.sink is not None else None
    out = sa.decode(q, kc, vc, csl, wl.scale, sink, num_splits=num_splits)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_variants(name, splits):
    wl = _dwl(name)
    _announce(f"decode {name} splits={splits}")
    o, lse, s = run_decode(wl, splits)
    ro, rl, rs = oracle.decode(wl.q.f32, wl.k_cache.f32, wl.v_cache.f32, wl.scale,
                               cache_seqlens=wl.cache_seqlens, sink=wl.sink)
    tol = tol_for(wl.dtype)
    assert_out(host(o), ro, tol)
    assert_lse(host(lse), rl, tol["lse"])
    assert float(np.max(np.abs(host(s) - rs))) <= tol["s"]


@pytest.mark.parametrize("name", ["d128_g4_lens", "f32"])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_ignores_unused_slots(name, splits):
    """Slots at or past cache_seqlens may hold anything: NaN and Inf there
    change nothing (a zero probability times NaN would be NaN)."""
    c = dict(DECODE_CASES[name])
    if "cache_seqlens" not in c:
        c["cache_seqlens"] = [70, 33][:c["batch"]]
    wl = W.make_decode(name, c.pop("batch"), c.pop("slots"), c.pop("hq"), c.pop("hkv"), c.pop("d"),
                       seed=4, **c)
    _announce(f"decode unused slots {name} splits={splits}")
    q = dev(wl.q, wl.dtype)
    kc, vc = dev(wl.k_cache, wl.dtype), dev(wl.v_cache, wl.dtype)
    for b, n in enumerate(wl.cache_seqlens):
        kc[b, int(n):] = float("nan")
        vc[b, int(n):] = float("nan")
        if int(n) + 1 < wl.slots:
            vc[b, int(n) + 1] = float("inf")
    csl = torch.from_numpy(wl.cache_seqlens).to(DEV)
    sink = torch.from_numpy(wl.sink).to(DEV) if wl.sink is not None else None
    o, lse, s = sa.decode(q, kc, vc, csl, wl.scale, sink, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(wl.q.f32, wl.k_cache.f32, wl.v_cache.f32, wl.scale,
                               cache_seqlens=wl.cache_seqlens, sink=wl.sink)
    tol = tol_for(wl.dtype)
    assert np.all(np.isfinite(host(o)))
    assert_out(host(o), ro, tol)
    assert_lse(host(lse), rl, tol["lse"])
    assert float(np.max(np.abs(host(s) - rs))) <= tol["s"]


def test_decode_permutation_and_split_invariance():
    """Slots are an unordered set and the split merge is exact: permuting the
    cache or changing num_splits changes the result only by rounding."""
    wl = _dwl("d128_g8", seed=9)
    wl = W.make_decode("perm", 4, 1000, 16, 2, 128, seed=9)
    ro, rl, rs = oracle.decode(wl.q.f32, wl.k_cache.f32, wl.v_cache.f32, wl.scale, sink=wl.sink)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(wl.slots)).to(DEV)
    tol = tol_for("bf16")
    for splits in (1, 2, 4, 7, 8):
        for pm in (None, perm):
            _announce(f"decode invariance splits={splits} perm={pm is not None}")
            o, lse, s = run_decode(wl, splits, pm)
            assert_out(host(o), ro, tol)
            assert_lse(host(lse), rl, tol["lse"])
            assert float(np.max(np.abs(host(s) - rs))) <= tol["s"]
