"""The binding's host-side precondition checks (SINK_ATTN_DEBUG=1): each
device-side precondition the C ABI documents, broken once, is reported; valid
inputs pass.  Pure host code, no GPU."""
import numpy as np
import pytest

from streamingllm_sink_attn_amd import binding as B
from streamingllm_sink_attn_amd import workloads as W


def _raises(fn, *a, match, **kw):
    with pytest.raises(B.SinkAttnError, match=match) as e:
        fn(*a, **kw)
    assert e.value.status == B.INVALID_ARGUMENT


def test_debug_flag(monkeypatch):
    monkeypatch.delenv("SINK_ATTN_DEBUG", raising=False)
    assert not B.debug_enabled()
    monkeypatch.setenv("SINK_ATTN_DEBUG", "1")
    assert B.debug_enabled()
    monkeypatch.setenv("SINK_ATTN_DEBUG", "0")
    assert not B.debug_enabled()


def test_prefill_valid_inputs_pass():
    cu = W.cu_from_lengths([200, 1, 64, 129])
    B.check_prefill_preconditions(cu, 394, 200)
    B.check_prefill_preconditions(np.array([0], np.int32), 0, 0)       # no samples
    B.check_prefill_preconditions(np.array([0, 0, 5], np.int32), 5, 5)  # an empty sample
    rng = np.random.default_rng(0)
    bi = W.sparse_block_lists(rng, [200, 1, 64, 129], 2, n_random=2)
    B.check_prefill_preconditions(cu, 394, 200, bi)


def test_prefill_first_entry_not_zero():
    _raises(B.check_prefill_preconditions, np.array([1, 5, 9]), 9, 8, match=r"cu_seqlens\[0\] = 1")


def test_prefill_not_monotone():
    _raises(B.check_prefill_preconditions, np.array([0, 50, 40, 90]), 90, 60,
            match="decreases at sample 1")


def test_prefill_last_entry_not_total():
    _raises(B.check_prefill_preconditions, np.array([0, 50, 90]), 100, 50,
            match=r"cu_seqlens\[batch\] = 90 != total_tokens = 100")


def test_prefill_length_above_max_seqlen():
    _raises(B.check_prefill_preconditions, np.array([0, 50, 130]), 130, 64,
            match="sample 1 has length 80 > max_seqlen = 64")


def test_prefill_empty_cu():
    _raises(B.check_prefill_preconditions, np.array([], np.int32), 0, 0, match="empty")


def test_block_ids_out_of_range():
    cu = W.cu_from_lengths([130, 64])              # 3 + 1 query blocks
    bi = np.full((4, 1, 2), -1, np.int32)
    bi[:, 0, 0] = [0, 1, 2, 0]
    B.check_prefill_preconditions(cu, 194, 130, bi)
    bad = bi.copy()
    bad[3, 0, 1] = 1                               # sample 1 has one block
    _raises(B.check_prefill_preconditions, cu, 194, 130, bad, match=r"sample 1: block ids must be in \[-1, 1\)")
    bad = bi.copy()
    bad[0, 0, 1] = -2
    _raises(B.check_prefill_preconditions, cu, 194, 130, bad, match=r"sample 0: .*found \[-2, 2\]")


def test_block_rows_too_few():
    cu = W.cu_from_lengths([130, 64])
    _raises(B.check_prefill_preconditions, cu, 194, 130, np.zeros((3, 1, 1), np.int32),
            match="3 rows < sum_b ceil")
    _raises(B.check_prefill_preconditions, cu, 194, 130, np.zeros((4, 1), np.int32),
            match="must be")


def test_cache_seqlens_range():
    B.check_decode_preconditions(np.array([1, 300, 17]), 300)
    B.check_decode_preconditions(None, 300)
    _raises(B.check_decode_preconditions, np.array([5, 0, 3]), 300, match=r"cache_seqlens\[1\] = 0")
    _raises(B.check_decode_preconditions, np.array([5, 301, 3]), 300, match=r"cache_seqlens\[1\] = 301")


def test_stream_positions():
    B.check_stream_positions(np.array([0, 7, 2 ** 30]), "n_seen", 1024)
    _raises(B.check_stream_positions, np.array([3, -1]), "n_seen", match=r"n_seen\[1\] = -1 < 0")
    _raises(B.check_stream_positions, np.array([2 ** 31 - 10]), "n_seen", 16,
            match=r"n_seen\[0\] \+ chunk")
    _raises(B.check_stream_positions, np.array([-4]), "n_tokens", match="n_tokens")
