"""Host-side checks of the benchmark's command line and of its FLOP/byte
counting helpers (no GPU)."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from streamingllm_sink_attn_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_window_pair_count_by_brute_force():
    """Kept (query, key) pairs of causal + first tokens + window, counted one
    by one on small samples."""
    for lengths, n_sink, window in (([37, 5, 64], 4, 10), ([100], 0, 7), ([20, 33], 3, 0)):
        want = 0
        for L in lengths:
            for i in range(L):
                for j in range(i + 1):
                    if window <= 0 or j < n_sink or i - j < window:
                        want += 1
        assert bench._counts_window(lengths, n_sink, window) == want


def test_chunked_prefill_pair_count_by_brute_force():
    wl = W.kvcache_prefill(batch=3, n_sink=4, window=16, chunk=9, hq=2, hkv=1, d=8, seed=1)
    want = 0
    for p0 in wl.n_seen:
        for c in range(wl.chunk):
            p = int(p0) + c
            want += sum(1 for k in range(p + 1) if k < wl.n_sink or p - k < wl.window)
    assert wl.valid_pairs() == want * wl.hq
    # a stream still inside its first window
    wl.n_seen[:] = np.array([0, 2, 5], np.int32)
    want = 0
    for p0 in wl.n_seen:
        for c in range(wl.chunk):
            p = int(p0) + c
            want += sum(1 for k in range(p + 1) if k < wl.n_sink or p - k < wl.window)
    assert wl.valid_pairs() == want * wl.hq
