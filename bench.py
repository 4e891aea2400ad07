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
    "sources": ('fwd_mfma.hip', 'qmajor.cuh', 'common.cuh', 'internal.h', 'stream_rows.cuh'),
    "sha256": "722fb0cc38f342ca165612e25c9d061aa72f902cf3cd33e6d1d74e3f603e6250",
    "read_bytes": 231219194,
    "write_bytes": 142695419,
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


def _progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _dev_bf16(t, torch):
    return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).cuda()


class ClockSampler:
    """Samples the GPU's graphics clock on a host thread every 5 ms while a
    leg's timed region runs: the current level of the kernel driver's
    pp_dpm_sclk file, which follows the live clock (the firmware metrics
    table that amdsmi reads refreshes only about once a second).  Reports
    the median and range in MHz, or None where the file is not readable."""

    def __init__(self):
        import glob
        self.path = None
        self.samples = []
        self._stop = None
        self._thread = None
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            try:
                if self._parse(open(f).read()) is not None:
                    self.path = f
                    break
            except OSError:
                continue

    @staticmethod
    def _parse(text):
        for line in text.splitlines():
            if line.rstrip().endswith("*"):
                mhz = line.split(":", 1)[1].strip().rstrip("*").strip().lower().replace("mhz", "")
                return float(mhz)
        return None

    def start(self):
        import threading
        self.samples = []
        if self.path is None:
            return
        self._stop = threading.Event()

        def poll():
            while not self._stop.is_set():
                try:
                    with open(self.path) as fh:
                        v = self._parse(fh.read())
                    if v is not None:
                        self.samples.append(v)
                except OSError:
                    return
                self._stop.wait(0.005)

        self._thread = threading.Thread(target=poll, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        if not self.samples:
            return None
        x = np.array(self.samples)
        return {"median_mhz": round(float(np.median(x)), 1), "min_mhz": round(float(x.min()), 1),
                "max_mhz": round(float(x.max()), 1), "samples": int(x.size)}


class Timer:
    """HIP events on the current stream (the one the binding enqueues on).

    Warm-up runs at least `warmup` steps and at least MIN_WARM_MS of GPU time
    (a GPU coming out of idle raises its clock over about half a second of
    load: measured 355 MHz idle, ~1940 MHz after 250 ms, ~2070 MHz after
    450 ms of back-to-back forwards).  The timed region records one event between consecutive steps,
    with no host synchronisation inside it, so the stream stays busy and every
    step's time is its own; the median step is reported, the mean and range
    beside it."""

    MIN_WARM_MS = 600.0

    def __init__(self, torch, clock=None):
        self.torch = torch
        self.clock = clock

    def warm(self, fn, warmup):
        torch = self.torch
        st = torch.cuda.current_stream()
        done, gpu_ms = 0, 0.0
        while done < warmup or gpu_ms < self.MIN_WARM_MS:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(5):
                fn()
            e1.record(st)
            e1.synchronize()
            gpu_ms += e0.elapsed_time(e1)
            done += 5
            if done >= 100000:
                break
        return done

    def timed(self, fns, steps):
        """Runs steps rounds of the functions in `fns` (interleaved) and
        returns per-function lists of step times in ms, and the wall time."""
        torch = self.torch
        st = torch.cuda.current_stream()
        torch.cuda.synchronize()
        n = len(fns)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps * n + 1)]
        t0 = time.perf_counter()
        ev[0].record(st)
        for i in range(steps):
            for j, fn in enumerate(fns):
                fn()
                ev[i * n + j + 1].record(st)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        per = [[ev[i * n + j].elapsed_time(ev[i * n + j + 1]) for i in range(steps)] for j in range(n)]
        return per, wall

    def run(self, fn, steps, warmup, per_step=1):
        """Returns a dict: median, mean, min, max ms per call; wall ms per
        step; warm-up steps run; the clock during the timed region.  A step of
        `fn` holds `per_step` calls (a graph replay of several launches)."""
        return self.run_many([fn], steps, warmup, per_step)[0]

    def run_many(self, fns, steps, warmup, per_step=1):
        n_warm = 0
        for fn in fns:
            n_warm = max(n_warm, self.warm(fn, warmup))
        if self.clock is not None:
            self.clock.start()
        per, wall = self.timed(fns, steps)
        clk = self.clock.stop() if self.clock is not None else None
        out = []
        for times in per:
            x = np.array(times) / per_step
            out.append({"median": float(np.median(x)), "mean": float(x.mean()), "min": float(x.min()),
                        "max": float(x.max()), "wall": wall / steps, "warmup_steps": n_warm, "clock": clk})
        return out


def graphed(torch, fn, n):
    """n calls of fn captured in one HIP graph (torch.cuda.CUDAGraph); returns
    its replay.  For launches of ~10 us, whose eager calls are bound by the
    host's launch rate rather than the GPU."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g.replay


def _ms(r):
    """Rounded timing summary of one Timer result (median is the figure used)."""
    return {"median": round(r["median"], 4), "mean": round(r["mean"], 4), "min": round(r["min"], 4),
            "max": round(r["max"], 4)}


def bench_gqa_prefill(torch, sa, W, steps, warmup, clock=None):
    wl = W.gqa_prefill()
    q, k, v = _dev_bf16(wl.q, torch), _dev_bf16(wl.k, torch), _dev_bf16(wl.v, torch)
    cu = torch.from_numpy(wl.cu_seqlens).cuda()
    sink = torch.from_numpy(wl.sink).cuda()
    o = torch.empty_like(q)
    pairs = _counts_window(wl.lengths, 0, 0) * wl.hq
    flops = 4.0 * wl.d * pairs

    def step():
        sa.fwd(q, k, v, cu, wl.max_seqlen, wl.scale, 0, 0, None, sink, return_s=True, out=o)

    r = Timer(torch, clock).run(step, steps, warmup)
    return dict(workload="gqa_prefill_fwd", timing=r, flops=flops, pairs=pairs,
                tflops=flops / (r["median"] * 1e-3) / 1e12,
                tflops_mean=flops / (r["mean"] * 1e-3) / 1e12, wl=wl)


def bench_gqa_gated(torch, sa, W, steps, warmup, clock=None):
    """The GQA prefill forward with the first-token gate written, and the head
    importance of that gate.  The plain and the gated forward are timed
    interleaved (plain, gated, plain, gated, ...) so both see the same clocks;
    the gate's overhead is the ratio of their medians.  The head importance
    ([T, Hq] float32 in, [Hq] out) is timed alone."""
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

    T = Timer(torch, clock)
    r_plain, r_gated = T.run_many([plain, gated], steps, warmup)
    r_imp = T.run(graphed(torch, lambda: sa.head_importance(gate, out=imp), 16), steps, warmup, per_step=16)
    ms, ms_plain = r_gated["median"], r_plain["median"]
    return dict(workload="gqa_prefill_fwd_gated", unit="TFLOP/s",
                value=round(flops / (ms * 1e-3) / 1e12, 2), ms_per_step=round(ms, 4),
                plain_fwd_ms=round(ms_plain, 4), gate_overhead=round(ms / ms_plain - 1.0, 4),
                head_importance_ms=round(r_imp["median"], 4), head_importance_timing="HIP graph of 16 calls",
                timing=_ms(r_gated),
                timing_plain=_ms(r_plain), clock=r_gated["clock"],
                note="forward with the first-token gate written (FLOPs: the forward's 4*D per "
                     "valid pair), timed interleaved with the plain forward; head importance "
                     "timed alone")


def _fwd_bwd_leg(torch, sa, wl, pairs, name, steps, warmup, cfg, clock=None):
    """Times one forward + backward per step; FLOPs are 14*D per valid pair
    (4*D forward, 10*D backward).  The forward and the backward are also timed
    on their own, interleaved with each other."""
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

    T = Timer(torch, clock)
    r = T.run(step, steps, warmup)
    r_f, r_b = T.run_many([fwd, bwd], steps, 2)
    ms, ms_f, ms_b = r["median"], r_f["median"], r_b["median"]
    f_all, f_f, f_b = 14.0 * wl.d * pairs, 4.0 * wl.d * pairs, 10.0 * wl.d * pairs
    tf = f_all / (ms * 1e-3) / 1e12
    return {"workload": name, "unit": "TFLOP/s", "value": round(tf, 2),
            "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "ms_per_step": round(ms, 4),
            "timing": _ms(r), "clock": r["clock"], "flops_per_step": f_all, "valid_pairs": pairs,
            "fwd": {"ms": round(ms_f, 4), "tflops": round(f_f / (ms_f * 1e-3) / 1e12, 2)},
            "bwd": {"ms": round(ms_b, 4), "tflops": round(f_b / (ms_b * 1e-3) / 1e12, 2)},
            "config": cfg}


def bench_streaming_prefill(torch, sa, W, steps, warmup, clock=None):
    """8 varlen samples (sum 32768), Hq=32, Hkv=8, D=128, n_sink=4, window=1024."""
    wl = W.streaming_prefill()
    pairs = _counts_window(wl.lengths, wl.n_sink, wl.window) * wl.hq
    return _fwd_bwd_leg(torch, sa, wl, pairs, "streaming_prefill_fwd_bwd", steps, warmup,
                        {"lengths": [int(x) for x in wl.lengths], "hq": wl.hq, "hkv": wl.hkv,
                         "head_dim": wl.d, "n_sink": wl.n_sink, "window": wl.window}, clock)


def bench_block_sparse(torch, sa, W, steps, warmup, clock=None):
    """4 x 16384, Hq=64, Hkv=8, D=128, 64-token blocks: first + 15 random + diagonal."""
    wl = W.block_sparse()
    pairs = _counts_blocks(wl.lengths, wl.block_indices, wl.hkv, wl.hq)
    return _fwd_bwd_leg(torch, sa, wl, pairs, "block_sparse_fwd_bwd", steps, warmup,
                        {"batch": wl.batch, "seq_len": int(wl.lengths[0]), "hq": wl.hq,
                         "hkv": wl.hkv, "head_dim": wl.d, "blocks_per_row": 17}, clock)


MEASURED = {}      # measured_peaks() of this run, read by the decode legs


def measured_peaks(torch, sa, clock=None, steps=10):
    """The microbenchmarks of libsinkattn_peaks.so (include/sink_attn_peaks.h)
    timed like the legs: a 2 GiB streaming read, the dense bf16 MFMA rate and
    the v_exp_f32 rate, beside the nominal peaks (HBM 8 TB/s, bf16 MFMA 2.5
    PFLOP/s at 2.4 GHz)."""
    import ctypes
    P = sa.binding.peaks_lib()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    T = Timer(torch, clock)
    out = {}
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    red = torch.empty(8192, dtype=torch.int32, device="cuda")
    r = T.run(lambda: P.sink_attn_peaks_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                             ctypes.c_void_p(red.data_ptr()), 8192, st()), steps, 3)
    out["hbm_read"] = {"GBs": round(nbytes / (r["median"] * 1e-3) / 1e9, 1), "bytes": nbytes,
                       "ms": round(r["median"], 4), "clock": r["clock"]}
    del buf
    torch.cuda.empty_cache()
    grid, iters = 1024, 4096
    o = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    r = T.run(lambda: P.sink_attn_peaks_mfma(iters, ctypes.c_void_p(o.data_ptr()), grid, st()), steps, 3)
    fl = grid * 4 * 4 * iters * 32768.0
    tf = fl / (r["median"] * 1e-3) / 1e12
    out["mfma_bf16"] = {"TFLOPs": round(tf, 1), "ms": round(r["median"], 4), "clock": r["clock"]}
    if r["clock"]:
        out["mfma_bf16"]["flop_per_clk_per_cu"] = round(tf * 1e12 / (256 * r["clock"]["median_mhz"] * 1e6), 1)
    r = T.run(lambda: P.sink_attn_peaks_exp(iters, ctypes.c_void_p(o.data_ptr()), grid, st()), steps, 3)
    ne = grid * 256 * 8 * iters
    out["exp_f32"] = {"Gexp_per_s": round(ne / (r["median"] * 1e-3) / 1e9, 1), "ms": round(r["median"], 4),
                      "clock": r["clock"]}
    if r["clock"]:
        out["exp_f32"]["per_clk_per_cu"] = round(ne / (r["median"] * 1e-3) / (256 * r["clock"]["median_mhz"] * 1e6), 2)
    out["probes"] = probes(torch, sa)
    MEASURED.update(out)
    return out


def probes(torch, sa):
    """Cycle counts (s_memtime per wavefront, one 8-wavefront workgroup per
    CU) of the co-issue and LDS-rate probes of libsinkattn_peaks.so: 16
    MFMAs and/or 32 FMAs per iteration in one wavefront or split over the
    two wavefronts of a SIMD; 16 LDS reads per lane per iteration."""
    import ctypes
    P = sa.binding.peaks_lib()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    grid, iters = 256, 2000
    o = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    cyc = torch.zeros(grid * 8, dtype=torch.int64, device="cuda")
    res = {}
    names = {0: "16 mfma", 1: "32 fma", 2: "16 mfma + 32 fma, one wavefront",
             3: "16 mfma on wavefronts 0-3, 32 fma on 4-7 (same SIMDs)"}
    for mode, name in names.items():
        for _ in range(2):                             # the second launch is the measured one
            assert P.sink_attn_peaks_coissue(mode, iters, ctypes.c_void_p(o.data_ptr()),
                                             ctypes.c_void_p(cyc.data_ptr()), grid, st()) == 0
        torch.cuda.synchronize()
        c = cyc.view(grid, 8).double() / iters
        if mode == 3:
            res[name] = {"mfma_wave_cycles_per_iter": round(c[:, :4].mean().item(), 1),
                         "fma_wave_cycles_per_iter": round(c[:, 4:].mean().item(), 1)}
        else:
            res[name] = {"cycles_per_iter": round(c.mean().item(), 1), "max": round(c.max().item(), 1)}
    lo = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    for mode, (name, nb) in {0: ("ds_read_b128", 16), 1: ("ds_read_b64", 8), 2: ("ds_read_b64_tr_b16", 8)}.items():
        for _ in range(2):
            assert P.sink_attn_peaks_lds(mode, iters, ctypes.c_void_p(lo.data_ptr()),
                                         ctypes.c_void_p(cyc.data_ptr()), grid, st()) == 0
        torch.cuda.synchronize()
        slowest = cyc.view(grid, 8).max().item()
        res[name] = {"bytes_per_clk_per_cu": round(512 * iters * 16 * nb / slowest, 1)}
    return res


def bench_decode(torch, sa, W, steps, warmup, clock=None):
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

    r = Timer(torch, clock).run(step, steps, warmup)
    ms = r["median"]
    gbs = nbytes / (ms * 1e-3) / 1e9
    read = MEASURED.get("hbm_read", {}).get("GBs")
    return {"workload": "streaming_decode", "unit": "GB/s", "value": round(gbs, 1),
            "ms_per_step": round(ms, 4), "timing": _ms(r), "clock": r["clock"], "bytes_per_step": nbytes,
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "frac_of_measured_read": round(gbs / read, 4) if read else None,
            "config": {"batch": wl.batch, "slots": wl.slots, "hq": wl.hq, "hkv": wl.hkv,
                       "head_dim": wl.d}}


def bench_kvcache_q8_decode(torch, sa, W, steps, warmup, clock=None):
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

    r = Timer(torch, clock).run(step, steps, warmup)
    ms = r["median"]
    gbs = nbytes / (ms * 1e-3) / 1e9
    read = MEASURED.get("hbm_read", {}).get("GBs")
    return {"workload": "streaming_decode_q8", "unit": "GB/s", "value": round(gbs, 1),
            "ms_per_step": round(ms, 4), "timing": _ms(r), "clock": r["clock"], "bytes_per_step": nbytes,
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "frac_of_measured_read": round(gbs / read, 4) if read else None,
            "config": {"batch": B, "n_sink": wl.n_sink, "window": wl.window, "hq": wl.hq,
                       "hkv": H, "head_dim": D, "ring": "e4m3 + per-row float32 scales"}}


def bench_kvcache_prefill(torch, sa, W, steps, warmup, clock=None):
    """Chunked prefill against the rolling cache: 8 streams each taking a
    1024-token chunk against (4 first tokens + 1024-token window) bf16
    caches, Hq=32, Hkv=8, D=128, streams past their first window.  One step is
    the whole call; FLOPs count the kept (row, key) pairs at 4*D."""
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

    T = Timer(torch, clock)
    r = T.run(step, steps, warmup)
    ms = r["median"]
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

    ms8 = T.run(step_q8, steps, warmup)["median"]
    # appending the same chunk afterwards (every token lands: chunk <= window);
    # bytes: the chunk's K, V read once, their slots written once
    rows = wl.batch * wl.chunk * wl.hkv
    app = {}
    for name, c_, wbytes in (("bf16", cache, rows * wl.d * 2 * 2), ("q8", qc, rows * (wl.d + 4) * 2)):
        ms_a = T.run(graphed(torch, lambda: sa.kvcache_append(c_, kn, vn, seen), 16), steps, warmup,
                     per_step=16)["median"]
        nb = rows * wl.d * 2 * 2 + wbytes
        app[name] = {"ms": round(ms_a, 4), "GBs": round(nb / (ms_a * 1e-3) / 1e9, 1), "bytes": nb}
    return {"workload": "streaming_chunked_prefill", "unit": "TFLOP/s", "value": round(tf, 2),
            "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "ms_per_step": round(ms, 4),
            "timing": _ms(r), "clock": r["clock"],
            "q8_cache": {"ms": round(ms8, 4), "tflops": round(flops / (ms8 * 1e-3) / 1e12, 2)},
            "append": app, "append_timing": "HIP graph of 16 calls",
            "valid_pairs": pairs,
            "config": {"batch": wl.batch, "chunk": wl.chunk, "n_sink": wl.n_sink, "window": wl.window,
                       "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "cache": "bf16"}}


def _oracle_unit(kind, args):
    """One unit of the CPU baseline in a worker process (one BLAS thread)."""
    import oracle
    t = time.perf_counter()
    if kind == "fwd":
        oracle.fwd(*args[:4], args[4], sink=args[5])
    elif kind == "fwd_bwd":
        q, k, v, cu, scale, do, n_sink, window, sink = args
        oracle.bwd(q, k, v, cu, scale, do, n_sink=n_sink, window=window, sink=sink)
    else:
        q, kc, vc, scale, sink = args
        oracle.decode(q, kc, vc, scale, sink=sink)
    return time.perf_counter() - t


def _run_units(pool, units, budget_s):
    """Submits (kind, args, work) units to the pool, at most one per worker
    in flight, until budget_s has passed; returns (work done, wall seconds,
    units done)."""
    import concurrent.futures as cf
    start = time.perf_counter()
    it = iter(units)
    pending = {}
    done_work, done_units = 0.0, 0

    def submit():
        u = next(it, None)
        if u is not None:
            pending[pool.submit(_oracle_unit, u[0], u[1])] = u[2]
        return u is not None

    for _ in range(pool._max_workers):
        submit()
    while pending:
        finished, _ = cf.wait(list(pending), return_when=cf.FIRST_COMPLETED)
        for f in finished:
            f.result()
            done_work += pending.pop(f)
            done_units += 1
            if time.perf_counter() - start < budget_s:
                submit()
    return done_work, time.perf_counter() - start, done_units


def cpu_baseline(W, budget_s=12.0):
    """The float64 oracle on the host cores, on bounded samples of three
    workloads, each spread over a process pool with one BLAS thread per
    process (units are independent):
      * the GQA prefill forward (the headline), by (sample, query head) units
        of 4096 x 4096 causal, TFLOP/s counted as the GPU figure;
      * the StreamingLLM prefill forward + backward, by (sample, query head)
        units (the oracle's backward re-runs the forward), 14*D per pair;
      * the StreamingLLM decode, by sequence (4096 slots, Hq=64, Hkv=8) on 32
        sequences drawn with the decode recipe, GB/s of its algorithmic bytes.
    `cores` is the number of worker processes (the host cores this process
    may use, at most 16)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        pool = cf.ProcessPoolExecutor(max_workers=cores, mp_context=mp.get_context("spawn"))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    try:
        wl = W.gqa_prefill()
        L = int(wl.lengths[0])
        G = wl.hq // wl.hkv
        units = []
        for b in range(wl.batch):
            for h in range(wl.hq):
                t0 = int(wl.cu_seqlens[b])
                sl = slice(t0, t0 + L)
                args = (wl.q.f32[sl, h:h + 1], wl.k.f32[sl, h // G:h // G + 1], wl.v.f32[sl, h // G:h // G + 1],
                        np.array([0, L]), wl.scale, wl.sink[h:h + 1])
                units.append(("fwd", args, 4.0 * wl.d * L * (L + 1) // 2))
        flops, el, n = _run_units(pool, units, budget_s)
        head = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                "sample": f"{n} of {len(units)} (sample, head) units of {L}x{L} causal, fp64, "
                          f"{el:.1f}s on {cores} processes"}
        del wl, units

        wl = W.streaming_prefill()
        units = []
        for b in range(wl.batch):
            t0, t1 = int(wl.cu_seqlens[b]), int(wl.cu_seqlens[b + 1])
            Lb = t1 - t0
            i = np.arange(Lb)
            pairs = int(np.minimum(i + 1, wl.window + np.minimum(wl.n_sink, np.maximum(0, i + 1 - wl.window))).sum())
            for h in range(wl.hq):
                g = h // (wl.hq // wl.hkv)
                args = (wl.q.f32[t0:t1, h:h + 1], wl.k.f32[t0:t1, g:g + 1], wl.v.f32[t0:t1, g:g + 1],
                        np.array([0, Lb]), wl.scale, wl.do.f32[t0:t1, h:h + 1], wl.n_sink, wl.window,
                        wl.sink[h:h + 1])
                units.append(("fwd_bwd", args, 14.0 * wl.d * pairs))
        units.sort(key=lambda u: u[2])               # shortest samples first: more units per budget
        flops, el, n = _run_units(pool, units, budget_s * 0.75)
        streaming = {"workload": "streaming_prefill_fwd_bwd", "value": flops / el / 1e12, "unit": "TFLOP/s",
                     "sample": f"{n} of {len(units)} (sample, head) units, fp64 forward + backward, "
                               f"{el:.1f}s"}
        del wl, units

        wl = W.streaming_decode(batch=32)
        per_seq = (2 * wl.slots * wl.hkv * wl.d * 2 + 2 * wl.hq * wl.d * 2 + 2 * wl.hq * 4)
        units = [("decode", (wl.q.f32[b:b + 1], wl.k_cache.f32[b:b + 1], wl.v_cache.f32[b:b + 1], wl.scale,
                             wl.sink), per_seq) for b in range(wl.batch)]
        nbytes, el, n = _run_units(pool, units, budget_s * 0.4)
        decode = {"workload": "streaming_decode", "value": nbytes / el / 1e9, "unit": "GB/s",
                  "sample": f"{n} sequences of 4096 slots (Hq=64, Hkv=8) drawn with the decode recipe, "
                            f"{el:.1f}s"}
    finally:
        pool.shutdown()
    head["also"] = [streaming, decode]
    return head


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (at least this many, and at least 600 ms of GPU "
                         "time: the GPU raises its clock over about half a second of load)")
    ap.add_argument("--min-warm-ms", type=float, default=Timer.MIN_WARM_MS,
                    help="GPU time every leg's warm-up runs at least (profiler runs pass 0)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", choices=("all", "headline", "decode", "streaming", "blocks", "gated",
                                       "decode_q8", "prefill_cache", "peaks"),
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

    Timer.MIN_WARM_MS = args.min_warm_ms

    sa.lib()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    clock = ClockSampler()
    single = {"decode": bench_decode, "streaming": bench_streaming_prefill,
              "blocks": bench_block_sparse, "gated": bench_gqa_gated,
              "decode_q8": bench_kvcache_q8_decode, "prefill_cache": bench_kvcache_prefill}
    if args.legs in single:
        print(json.dumps(single[args.legs](torch, sa, W, args.steps, args.warmup, clock)), flush=True)
        return
    if args.legs == "peaks":
        print(json.dumps(measured_peaks(torch, sa, clock)), flush=True)
        return
    peaks = measured_peaks(torch, sa, clock) if args.legs == "all" else None
    if peaks:
        _progress(f"measured peaks: {json.dumps(peaks)}")
    head = bench_gqa_prefill(torch, sa, W, args.steps, args.warmup, clock)
    wl = head.pop("wl")
    r = head["timing"]
    # the dominant kernel is the forward kernel, one launch per step: its
    # average launch duration is the mean step time of the timed region
    roofline = {"bound": "mfma", "achieved": head["tflops_mean"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": head["tflops_mean"] / PEAK_BF16_TFLOPS,
                "traffic": _fwd_traffic()}
    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": r["warmup_steps"],
        "ms_per_step": round(r["median"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gqa_prefill_fwd", "batch": wl.batch, "seq_len": int(wl.lengths[0]),
                   "hq": wl.hq, "hkv": wl.hkv, "head_dim": wl.d, "mask": "causal",
                   "sink": "learnable", "flops_per_step": head["flops"]},
        "roofline": roofline,
        "timing": _ms(r),
        "clock": r["clock"],
    }
    if peaks:
        line["measured_peaks"] = peaks
    also = []
    legs = ((bench_streaming_prefill, bench_decode, bench_block_sparse, bench_gqa_gated,
             bench_kvcache_q8_decode, bench_kvcache_prefill) if args.legs == "all" else ())
    _progress(f"headline done: {line['value']} TFLOP/s")
    for fn in legs:
        t0 = time.perf_counter()
        try:
            also.append(fn(torch, sa, W, args.steps, args.warmup, clock))
        except Exception as e:  # noqa: BLE001 - report, keep the headline
            also.append({"workload": fn.__name__, "error": repr(e)})
        torch.cuda.empty_cache()
        _progress(f"{fn.__name__} done in {time.perf_counter() - t0:.1f}s")
    if also:
        line["also"] = also
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        line["cpu_baseline"] = cpu_baseline(W)
        _progress(f"cpu baseline done in {time.perf_counter() - t0:.1f}s")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
