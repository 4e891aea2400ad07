"""Benchmark of the sink-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--legs NAME]

Prints ONE JSON line.  The headline (``value``) is the GQA prefill forward:
4 packed samples x 4096 tokens, Hq=32, Hkv=8, D=128, bf16, causal, learnable
sink, in TFLOP/s counting only unmasked (query, key, head) pairs at 4*D FLOP
each.  The other workloads (StreamingLLM prefill fwd+bwd, StreamingLLM decode,
block-sparse fwd+bwd) are reported under ``also``.  Inputs are synthetic,
seeded, and resident in HBM before timing starts.  Kernel time is measured with
HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "sink-attn fwd/fwd+bwd TFLOP/s (% MFMA peak); decode KV GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# HBM bytes one launch of the forward kernel moves on the GQA prefill
# workload: rocprofv3 FETCH_SIZE and WRITE_SIZE passes (bench.py --legs
# headline --calibrate-copy), each scaled by what the same counter reads for a
# 1 GiB device-to-device copy (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); the
# summary is profiles/fwd_kernel_gqa_prefill_4x4096.md.  The figures hold for
# the kernel sources they were taken on: when those change, traffic is
# reported as null until the counters are taken again.
FWD_TRAFFIC = {
    "sources": ("fwd_mfma.hip", "qmajor.cuh", "common.cuh", "internal.h"),
    "sha256": "ec782dd1e70cb6d4a967fe652fb4da2d01055ae974c3a2013fd04ea708e86869",
    "read_bytes": 224755875,
    "write_bytes": 143030272,
}


def _fwd_traffic():
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "streamingllm_sink_attn_amd", "csrc")
    h = hashlib.sha256()
    try:
        for f in FWD_TRAFFIC["sources"]:
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    except OSError:
        return None
    if h.hexdigest() != FWD_TRAFFIC["sha256"]:
        return None
    return FWD_TRAFFIC["read_bytes"] + FWD_TRAFFIC["write_bytes"]


def _counts_window(lengths, n_sink, window):
    """Valid (query, key) pairs per head for causal + kept first tokens + window."""
    tot = 0
    for L in lengths:
        i = np.arange(int(L), dtype=np.int64)
        if window > 0:
            c = np.minimum(i + 1, window + np.minimum(n_sink, np.maximum(0, i + 1 - window)))
        else:
            c = i + 1
        tot += int(c.sum())
    return tot


def _counts_blocks(lengths, block_indices, hkv, hq, bs=64):
    """Valid pairs summed over query heads for block lists (+ causal)."""
    tot = 0
    row = 0
    G = hq // hkv
    for L in lengths:
        L = int(L)
        nqb = -(-L // bs)
        for qb in range(nqb):
            rows = min(bs, L - qb * bs)
            for g in range(hkv):
                sel = set(int(x) for x in block_indices[row + qb, g] if x >= 0 and x <= qb)
                n = 0
                for kb in sel:
                    if kb < qb:
                        n += bs * rows
                    else:                     # diagonal block: causal inside
                        n += rows * (rows + 1) // 2
                tot += n * G
        row += nqb
    return tot


def _dev_bf16(t, torch):
    return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()


class Timer:
    """HIP events on the current stream around a region, averaged per step."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall * 1e3 / steps


def bench_gqa_prefill(torch, sa, W, steps, warmup):
    wl = W.gqa_prefill()
    q, k, v = _dev_bf16(wl.q, torch), _dev_bf16(wl.k, torch), _dev_bf16(wl.v, torch)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    sink = torch.from_numpy(wl.sink).cuda()
    o = torch.empty_like(q)
    pairs = _counts_window(wl.lengths, 0, 0) * wl.hq
    flops = 4.0 * wl.d * pairs

    def step():
        sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, None, sink, return_s=True, out=o)

    ms, wall_ms = Timer(torch).run(step, steps, warmup)
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(workload="gqa_prefill_fwd", ms=ms, wall_ms=wall_ms, flops=flops, pairs=pairs,
                tflops=tflops, wl=wl)


def bench_gqa_gated(torch, sa, W, steps, warmup):
    """The GQA prefill forward with the first-token gate written, and the head
    importance of that gate.  Timed apart: the plain forward, the gated
    forward (its overhead is the gate's cost inside the kernel) and one head
    importance call ([T, Hq] float32 in, [Hq] out)."""
    wl = W.gqa_prefill()
    q, k, v = _dev_bf16(wl.q, torch), _dev_bf16(wl.k, torch), _dev_bf16(wl.v, torch)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    sink = torch.from_numpy(wl.sink).cuda()
    o = torch.empty_like(q)
    gate = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    imp = torch.empty(wl.hq, dtype=torch.float32, device="cuda")
    pairs = _counts_window(wl.lengths, 0, 0) * wl.hq
    flops = 4.0 * wl.d * pairs

    def plain():
        sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, None, sink, return_s=True, out=o)

    def gated():
        sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, None, sink, return_s=True, out=o,
               gate0=gate)

    ms_plain, _ = Timer(torch).run(plain, steps, warmup)
    ms, _ = Timer(torch).run(gated, steps, warmup)
    ms_imp, _ = Timer(torch).run(lambda: sa.head_importance(gate, out=imp), steps, warmup)
    return dict(workload="gqa_prefill_fwd_gated", unit="TFLOP/s",
                value=round(flops / (ms * 1e-3) / 1e12, 2), ms_per_step=round(ms, 4),
                plain_fwd_ms=round(ms_plain, 4), gate_overhead=round(ms / ms_plain - 1.0, 4),
                head_importance_ms=round(ms_imp, 4),
                note="forward with the first-token gate written (FLOPs: the forward's 4*D per "
                     "valid pair); head importance timed alone")


def _fwd_bwd_leg(torch, sa, wl, pairs, name, steps, warmup, cfg):
    """Times one forward + backward per step; FLOPs are 14*D per valid pair
    (4*D forward, 10*D backward), and fwd / bwd are also timed alone."""
    q, k, v = _dev_bf16(wl.q, torch), _dev_bf16(wl.k, torch), _dev_bf16(wl.v, torch)
    do = _dev_bf16(wl.do, torch)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    sink = torch.from_numpy(wl.sink).cuda()
    bi = torch.from_numpy(wl.block_indices).cuda() if wl.block_indices is not None else None
    o = torch.empty_like(q)
    state = {}

    def fwd():
        state["out"] = sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink,
                              return_s=True, out=o)

    def bwd():
        _, lse, _ = state["out"]
        sa.bwd(q, k, v, o, lse, do, cu, wl.max_seqlen, wl.scale, wl.n_sink, wl.window, bi, sink)

    def step():
        fwd()
        bwd()

    T = Timer(torch)
    ms, _ = T.run(step, steps, warmup)
    ms_f, _ = T.run(fwd, steps, 2)
    ms_b, _ = T.run(bwd, steps, 2)
    f_all, f_f, f_b = 14.0 * wl.d * pairs, 4.0 * wl.d * pairs, 10.0 * wl.d * pairs
    tf = f_all / (ms * 1e-3) / 1e12
    return {"workload": name, "unit": "TFLOP/s", "value": round(tf, 2),
            "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "ms_per_step": round(ms, 4),
            "flops_per_step": f_all, "valid_pairs": pairs,
            "fwd": {"ms": round(ms_f, 4), "tflops": round(f_f / (ms_f * 1e-3) / 1e12, 2)},
            "bwd": {"ms": round(ms_b, 4), "tflops": round(f_b / (ms_b * 1e-3) / 1e12, 2)},
            "config": cfg}


def bench_streaming_prefill(torch, sa, W, steps, warmup):
    """8 varlen samples (sum 32768), Hq=32, Hkv=8, D=128, n_sink=4, window=1024."""
    wl = W.streaming_prefill()
    pairs = _counts_window(wl.lengths, wl.n_sink, wl.window) * wl.hq
    return _fwd_bwd_leg(torch, sa, wl, pairs, "streaming_prefill_fwd_bwd", steps, warmup,
                        {"lengths": [int(x) for x in wl.lengths], "hq": wl.hq, "hkv": wl.hkv,
                         "head_dim": wl.d, "n_sink": wl.n_sink, "window": wl.window})


def bench_block_sparse(torch, sa, W, steps, warmup):
    """4 x 16384, Hq=64, Hkv=8, D=128, 64-token blocks: first + 15 random + diagonal."""
    wl = W.block_sparse()
    pairs = _counts_blocks(wl.lengths, wl.block_indices, wl.hkv, wl.hq)
    return _fwd_bwd_leg(torch, sa, wl, pairs, "block_sparse_fwd_bwd", steps, warmup,
                        {"batch": wl.batch, "seq_len": int(wl.lengths[0]), "hq": wl.hq,
                         "hkv": wl.hkv, "head_dim": wl.d, "blocks_per_row": 17})


def bench_decode(torch, sa, W, steps, warmup):
    """StreamingLLM decode: 128 sequences x 4096-slot cache, Hq=64, Hkv=8.
    Two cache copies alternate so no call finds the previous one's bytes in
    the on-die caches.  Bytes count each valid K/V slot once plus Q, O, lse, s."""
    wl = W.streaming_decode()
    q = _dev_bf16(wl.q, torch)
    kc = [_dev_bf16(wl.k_cache, torch)]
    vc = [_dev_bf16(wl.v_cache, torch)]
    kc.append(torch.roll(kc[0], 1, dims=1).contiguous())
    vc.append(torch.roll(vc[0], 1, dims=1).contiguous())
    sink = torch.from_numpy(wl.sink).cuda()
    o = torch.empty_like(q)
    nbytes = (2 * wl.batch * wl.slots * wl.hkv * wl.d * 2 + 2 * wl.batch * wl.hq * wl.d * 2
              + 2 * wl.batch * wl.hq * 4)
    it = [0]

    def step():
        i = it[0] & 1
        it[0] += 1
        sa.decode(q, kc[i], vc[i], None, wl.scale, sink, out=o)

    ms, wall_ms = Timer(torch).run(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "streaming_decode", "unit": "GB/s", "value": round(gbs, 1),
            "ms_per_step": round(ms, 4), "bytes_per_step": nbytes,
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "config": {"batch": wl.batch, "slots": wl.slots, "hq": wl.hq, "hkv": wl.hkv,
                       "head_dim": wl.d}}


def bench_kvcache_q8_decode(torch, sa, W, steps, warmup):
    """Decode over the 8-bit rolling cache: 128 sequences x (4 first tokens in
    bf16 + a 4092-token e4m3 ring), Hq=64, Hkv=8 (the bf16 decode's shape).
    Two cache copies alternate; bytes count each valid slot once (bf16 first
    tokens, 8-bit ring rows and their two scales) plus Q, O, lse, s."""
    wl = W.kvcache_q8_decode()
    caches = []
    for i in range(2):
        c = sa.KvCache(wl.batch, wl.n_sink, wl.window, wl.hkv, wl.d, quantized=True)
        c.sink_k.copy_(torch.from_numpy(wl.sink_k).to(torch.bfloat16))
        c.sink_v.copy_(torch.from_numpy(wl.sink_v).to(torch.bfloat16))
        c.win_k.copy_(torch.roll(torch.from_numpy(wl.win_k), i, dims=1))
        c.win_v.copy_(torch.roll(torch.from_numpy(wl.win_v), i, dims=1))
        c.win_k_scale.copy_(torch.from_numpy(wl.win_k_scale))
        c.win_v_scale.copy_(torch.from_numpy(wl.win_v_scale))
        caches.append(c)
    q = torch.from_numpy(wl.q).cuda().to(torch.bfloat16)
    nt = torch.from_numpy(wl.n_tokens).cuda()
    sink = torch.from_numpy(wl.sink).cuda()
    o = torch.empty_like(q)
    B, H, D = wl.batch, wl.hkv, wl.d
    nbytes = (2 * B * wl.n_sink * H * D * 2 + 2 * B * wl.window * H * D + 2 * B * H * wl.window * 4
              + 2 * B * wl.hq * D * 2 + 2 * B * wl.hq * 4)
    it = [0]

    def step():
        i = it[0] & 1
        it[0] += 1
        sa.kvcache_decode(caches[i], q, nt, wl.scale, sink, out=o)

    ms, _ = Timer(torch).run(step, steps, warmup)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "streaming_decode_q8", "unit": "GB/s", "value": round(gbs, 1),
            "ms_per_step": round(ms, 4), "bytes_per_step": nbytes,
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "config": {"batch": B, "n_sink": wl.n_sink, "window": wl.window, "hq": wl.hq,
                       "hkv": H, "head_dim": D, "ring": "e4m3 + per-row float32 scales"}}


def bench_kvcache_prefill(torch, sa, W, steps, warmup):
    """Chunked prefill against the rolling cache: 8 streams each taking a
    1024-token chunk against (4 first tokens + 1024-token window) bf16
    caches, Hq=32, Hkv=8, D=128, streams past their first window.  One step is
    the whole call (packing the cache and chunk, the forward, the copy of the
    chunk rows); FLOPs count the kept (row, key) pairs at 4*D."""
    wl = W.kvcache_prefill()
    cache = sa.KvCache(wl.batch, wl.n_sink, wl.window, wl.hkv, wl.d, quantized=False)
    cache.k.copy_(torch.from_numpy(wl.k_cache).to(torch.bfloat16))
    cache.v.copy_(torch.from_numpy(wl.v_cache).to(torch.bfloat16))
    dev = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)
    q, kn, vn = dev(wl.q), dev(wl.k_new), dev(wl.v_new)
    seen = torch.from_numpy(wl.n_seen).cuda()
    sink = torch.from_numpy(wl.sink).cuda()
    o = torch.empty_like(q)
    pairs = wl.valid_pairs()
    flops = 4.0 * wl.d * pairs

    def step():
        sa.kvcache_prefill(cache, q, kn, vn, seen, wl.scale, sink, out=o)

    ms, _ = Timer(torch).run(step, steps, warmup)
    tf = flops / (ms * 1e-3) / 1e12
    # the same call against the 8-bit cache (ring rows dequantised on the way
    # in): random codes and row scales of unit-normal size, the bf16 first tokens
    qc = sa.KvCache(wl.batch, wl.n_sink, wl.window, wl.hkv, wl.d, quantized=True)
    qc.sink_k.copy_(cache.k[:, :wl.n_sink])
    qc.sink_v.copy_(cache.v[:, :wl.n_sink])
    g = torch.Generator(device="cpu").manual_seed(1)
    for t in (qc.win_k, qc.win_v):
        t.copy_(torch.randint(0, 0x7F, tuple(t.shape), generator=g, dtype=torch.uint8)
                | (torch.randint(0, 2, tuple(t.shape), generator=g, dtype=torch.uint8) << 7))
    for t in (qc.win_k_scale, qc.win_v_scale):
        t.copy_(torch.rand(tuple(t.shape), generator=g) * (2.0 / 448) + 2.0 / 448)

    def step_q8():
        sa.kvcache_prefill(qc, q, kn, vn, seen, wl.scale, sink, out=o)

    ms8, _ = Timer(torch).run(step_q8, steps, warmup)
    # appending the same chunk afterwards (every token lands: chunk <= window);
    # bytes: the chunk's K, V read once, their slots written once
    rows = wl.batch * wl.chunk * wl.hkv
    app = {}
    for name, c_, wbytes in (("bf16", cache, rows * wl.d * 2 * 2), ("q8", qc, rows * (wl.d + 4) * 2)):
        ms_a, _ = Timer(torch).run(lambda: sa.kvcache_append(c_, kn, vn, seen), steps, warmup)
        nb = rows * wl.d * 2 * 2 + wbytes
        app[name] = {"ms": round(ms_a, 4), "GBs": round(nb / (ms_a * 1e-3) / 1e9, 1), "bytes": nb}
    return {"workload": "streaming_chunked_prefill", "unit": "TFLOP/s", "value": round(tf, 2),
            "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "ms_per_step": round(ms, 4),
            "q8_cache": {"ms": round(ms8, 4), "tflops": round(flops / (ms8 * 1e-3) / 1e12, 2)},
            "append": app,
            "valid_pairs": pairs,
            "config": {"batch": wl.batch, "chunk": wl.chunk, "n_sink": wl.n_sink, "window": wl.window,
                       "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "cache": "bf16"}}


def cpu_baseline(W, budget_s=15.0):
    """The float64 oracle on whole (sample, head) units of the same workload,
    until about budget_s seconds of CPU work; reported in TFLOP/s counted the
    same way as the GPU figure."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # noqa: BLE001
        threads = 1
    wl = W.gqa_prefill()
    L = int(wl.lengths[0])
    units = [(b, h) for b in range(wl.batch) for h in range(wl.hq)]
    done = 0
    start = time.perf_counter()
    for b, h in units:
        g = h // (wl.hq // wl.hkv)
        t0 = int(wl.cu_seqlens[b])
        sl = slice(t0, t0 + L)
        q = wl.q.f32[sl, h:h + 1]
        k = wl.k.f32[sl, g:g + 1]
        v = wl.v.f32[sl, g:g + 1]
        oracle.fwd(q, k, v, np.array([0, L]), wl.scale, sink=wl.sink[h:h + 1])
        done += 1
        if time.perf_counter() - start > budget_s:
            break
    el = time.perf_counter() - start
    pairs = L * (L + 1) // 2 * done
    flops = 4.0 * wl.d * pairs
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} (sample, head) units of {L}x{L} causal, fp64, {el:.1f}s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: the GPU reaches its steady clocks only after "
                         "tens of milliseconds of load")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", choices=("all", "headline", "decode", "streaming", "blocks", "gated",
                                       "decode_q8", "prefill_cache"),
                    default="all",
                    help="headline: only the GQA prefill forward (for profiler runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one 1 GiB device-to-device copy (a kernel of known "
                         "traffic for scaling hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                          "multi-GPU sharding is not implemented"}))
        sys.exit(2)

    import torch
    import streamingllm_sink_attn_amd as sa
    from streamingllm_sink_attn_amd import workloads as W

    sa.lib()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    single = {"decode": bench_decode, "streaming": bench_streaming_prefill,
              "blocks": bench_block_sparse, "gated": bench_gqa_gated,
              "decode_q8": bench_kvcache_q8_decode, "prefill_cache": bench_kvcache_prefill}
    if args.legs in single:
        print(json.dumps(single[args.legs](torch, sa, W, args.steps, args.warmup)), flush=True)
        return
    head = bench_gqa_prefill(torch, sa, W, args.steps, args.warmup)
    wl = head.pop("wl")
    roofline = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": head["tflops"] / PEAK_BF16_TFLOPS, "traffic": _fwd_traffic()}
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gqa_prefill_fwd", "batch": wl.batch, "seq_len": int(wl.lengths[0]),
                   "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "mask": "causal",
                   "sink": "learnable", "flops_per_step": head["flops"]},
        "roofline": roofline,
    }
    also = []
    legs = ((bench_streaming_prefill, bench_decode, bench_block_sparse, bench_gqa_gated,
             bench_kvcache_q8_decode, bench_kvcache_prefill) if args.legs == "all" else ())
    for fn in legs:
        try:
            also.append(fn(torch, sa, W, args.steps, args.warmup))
        except Exception as e:  # noqa: BLE001 - report, keep the headline
            also.append({"workload": fn.__name__, "error": repr(e)})
        torch.cuda.empty_cache()
    if also:
        line["also"] = also
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
