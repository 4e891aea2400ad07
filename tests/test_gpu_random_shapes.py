"""Seeded sweep of random prefill and decode shapes against the float64
oracle: sample lengths from 0 to a few hundred (ragged tails, empty samples,
one-token samples), GQA groups of 1 to 4 query heads, head_dim 128 (matrix
core kernels) and 64 or 32 (generic kernels, bfloat16 or float32), causal /
kept first tokens + window / sparse block lists, and the sink off, moderate
or wide.  Each case checks O, LSE and s of the forward and dQ, dK, dV and
dsink of the backward ("Attention Sink, Learnable Sink and dsink" s1, s4,
s7-s8), or O, LSE and s of the decode with split-KV (s4, the LSE merge),
to the same tolerances as the named cases."""
import numpy as np
import pytest
import torch

import oracle
import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

from gpu_helpers import (DEV, assert_lse, assert_out, check_bwd_full, check_fwd_full, dev, host,
                         prefill_args, run_fwd, tol_for)

pytestmark = pytest.mark.gpu

N_PREFILL = 24
N_DECODE = 16


def _prefill_case(i):
    rng = np.random.default_rng(7000 + i)
    batch = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(0, 261, size=batch)]
    if max(lengths) == 0:
        lengths[0] = int(rng.integers(1, 261))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 3, 4]))
    kind = rng.choice(["mfma", "mfma", "generic_bf16", "generic_f32"])
    d, dtype = {"mfma": (128, "bf16"), "generic_bf16": (64, "bf16"), "generic_f32": (32, "f32")}[kind]
    mode = rng.choice(["causal", "window", "blocks"])
    n_sink = window = 0
    blocks = None
    if mode == "window":
        n_sink = int(rng.choice([0, 1, 4, 7, 64]))
        window = int(rng.choice([1, 5, 33, 64, 100, 200]))
    elif mode == "blocks":
        blocks = dict(n_random=int(rng.integers(0, 4)))
    sink = bool(rng.random() < 0.8)
    wl = W.make_prefill(f"rand{i}", lengths, hq=hkv * G, hkv=hkv, d=d, dtype=dtype, n_sink=n_sink,
                        window=window, sink=sink, block_lists=blocks, rng=rng)
    if sink and rng.random() < 0.3:
        wl.sink = (wl.sink * np.float32(8.0)).astype(np.float32)       # a over about +-20
    desc = (f"lengths={lengths} hq={hkv * G} hkv={hkv} d={d} {dtype} {mode} n_sink={n_sink} "
            f"window={window} blocks={blocks} sink={sink}")
    return wl, desc


@pytest.mark.parametrize("i", range(N_PREFILL))
def test_random_prefill_fwd_bwd(i):
    wl, desc = _prefill_case(i)
    print(f"[case] random prefill {i}: {desc}", flush=True)
    check_fwd_full(wl, run_fwd(wl, prefill_args(wl)))
    check_bwd_full(wl)


def _decode_case(i):
    rng = np.random.default_rng(8000 + i)
    batch = int(rng.integers(1, 6))
    slots = int(rng.integers(1, 700))
    hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 3, 4, 8, 16]))
    kind = rng.choice(["mfma", "mfma", "generic_f32"])
    d, dtype = (128, "bf16") if kind == "mfma" else (64, "f32")
    csl = [int(x) for x in rng.integers(1, slots + 1, size=batch)] if rng.random() < 0.7 else None
    sink = bool(rng.random() < 0.8)
    splits = int(rng.choice([0, 1, 2, 5]))
    wl = W.make_decode(f"rdec{i}", batch, slots, hkv * G, hkv, d, dtype=dtype, sink=sink, seed=8000 + i,
                       cache_seqlens=csl, n_sink=min(4, slots))
    desc = f"batch={batch} slots={slots} hq={hkv * G} hkv={hkv} d={d} {dtype} csl={csl} sink={sink} splits={splits}"
    return wl, splits, desc


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode(i):
    wl, splits, desc = _decode_case(i)
    print(f"[case] random decode {i}: {desc}", flush=True)
    q = dev(wl.q, wl.dtype)
    kc, vc = dev(wl.k_cache, wl.dtype), dev(wl.v_cache, wl.dtype)
    csl = torch.from_numpy(wl.cache_seqlens).to(DEV) if wl.cache_seqlens is not None else None
    sink = torch.from_numpy(wl.sink).to(DEV) if wl.sink is not None else None
    o, lse, s = sa.decode(q, kc, vc, csl, wl.scale, sink, num_splits=splits)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(wl.q.f32, wl.k_cache.f32, wl.v_cache.f32, wl.scale,
                               cache_seqlens=wl.cache_seqlens, sink=wl.sink)
    tol = tol_for(wl.dtype)
    assert_out(host(o), ro, tol)
    assert_lse(host(lse), rl, tol["lse"])
    assert float(np.max(np.abs(host(s) - rs))) <= tol["s"]
