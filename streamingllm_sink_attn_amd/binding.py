"""Thin Python binding over libsinkattn.so (ctypes).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory (outputs and workspace) and streams.  If the
library is not built the calls raise; there is no fallback.

Streams: every call takes ``stream=`` (default: the current stream).  Outputs
and workspace are allocated while that stream is current, so torch's caching
allocator ties them to the stream the kernels run on and cannot hand the
workspace to other work before those kernels finish.

Debug checks: with the environment variable SINK_ATTN_DEBUG=1 every call
first copies its index arrays (cu_seqlens, block_indices, cache lengths,
stream positions) to the host and checks the device-side preconditions the C
ABI documents but does not check (it never reads device memory from the
host), raising SinkAttnError on a violation.  This synchronises, so it is
for debugging only.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsinkattn.so")

BF16, F32 = 0, 1
OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP_ERROR = range(5)
BLOCK_SIZE = 64

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class PrefillDesc(ctypes.Structure):
    _fields_ = [
        ("cu_seqlens", c_vp),
        ("batch", c_i32),
        ("total_tokens", c_i32),
        ("max_seqlen", c_i32),
        ("num_q_heads", c_i32),
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("dtype", c_i32),
        ("softmax_scale", ctypes.c_float),
        ("n_sink", c_i32),
        ("window", c_i32),
        ("block_indices", c_vp),
        ("num_q_blocks", c_i32),
        ("block_size", c_i32),
        ("max_blocks", c_i32),
        ("learnable_sink", c_vp),
    ]


class KvCacheDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32),
        ("n_sink", c_i32),
        ("window", c_i32),
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("quantized", c_i32),
        ("k", c_vp),
        ("v", c_vp),
        ("sink_k", c_vp),
        ("sink_v", c_vp),
        ("win_k", c_vp),
        ("win_v", c_vp),
        ("win_k_scale", c_vp),
        ("win_v_scale", c_vp),
    ]


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("cache_seqlens", c_vp),
        ("batch", c_i32),
        ("slots", c_i32),
        ("num_q_heads", c_i32),
        ("num_kv_heads", c_i32),
        ("head_dim", c_i32),
        ("dtype", c_i32),
        ("softmax_scale", ctypes.c_float),
        ("learnable_sink", c_vp),
        ("num_splits", c_i32),
    ]


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sink_attn status {status}: {msg}")
        self.status = status


_lib = None

_SIGS = {
    "sink_attn_fwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "sink_attn_fwd_gated": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    ctypes.c_size_t, c_vp]),
    "sink_attn_head_importance": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "sink_attn_head_importance_workspace_size": (ctypes.c_size_t, [c_i32, c_i32]),
    "sink_attn_check_fwd_gated": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                          ctypes.c_size_t]),
    "sink_attn_check_head_importance": (c_i32, [c_vp, c_i32, c_i32, c_vp, ctypes.c_size_t]),
    "sink_attn_kvcache_append": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp, c_vp]),
    "sink_attn_kvcache_decode": (c_i32, [c_vp, c_vp, c_i32, c_vp, ctypes.c_float, c_vp, c_i32, c_vp,
                                         c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "sink_attn_kvcache_decode_workspace_size": (ctypes.c_size_t, [c_vp, c_i32, c_i32]),
    "sink_attn_kvcache_prefill": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, ctypes.c_float, c_vp,
                                          c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "sink_attn_kvcache_prefill_workspace_size": (ctypes.c_size_t, [c_vp, c_i32, c_i32]),
    "sink_attn_check_kvcache_prefill": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, ctypes.c_float,
                                                c_vp, c_vp, c_vp, ctypes.c_size_t]),
    "sink_attn_check_kvcache_append": (c_i32, [c_vp, c_vp, c_vp, c_i32, c_vp]),
    "sink_attn_check_kvcache_decode": (c_i32, [c_vp, c_vp, c_i32, c_vp, ctypes.c_float, c_i32, c_vp,
                                               c_vp, c_vp, ctypes.c_size_t]),
    "sink_attn_bwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                              c_vp, ctypes.c_size_t, c_vp]),
    "sink_attn_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t, c_vp]),
    "sink_attn_decode_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "sink_attn_fwd_workspace_size": (ctypes.c_size_t, [c_vp]),
    "sink_attn_bwd_workspace_size": (ctypes.c_size_t, [c_vp]),
    "sink_attn_decode_workspace_size": (ctypes.c_size_t, [c_vp]),
    "sink_attn_check_fwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t]),
    "sink_attn_check_bwd": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    ctypes.c_size_t]),
    "sink_attn_check_decode": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t]),
    "sink_attn_strerror": (ctypes.c_char_p, [c_i32]),
    "sink_attn_last_error": (ctypes.c_char_p, []),
    "sink_attn_prefill_path": (c_i32, [c_vp]),
    "sink_attn_debug_visit_map": (c_i32, [c_vp, c_vp, ctypes.c_size_t, c_vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m streamingllm_sink_attn_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


PEAKS_LIB_PATH = os.path.join(_HERE, "libsinkattn_peaks.so")
_peaks = None

PEAKS_SIGS = {
    "sink_attn_peaks_read": (c_i32, [c_vp, ctypes.c_size_t, c_vp, c_i32, c_vp]),
    "sink_attn_peaks_mfma": (c_i32, [c_i32, c_vp, c_i32, c_vp]),
    "sink_attn_peaks_exp": (c_i32, [c_i32, c_vp, c_i32, c_vp]),
    "sink_attn_peaks_coissue": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_i32, c_vp]),
    "sink_attn_peaks_lds": (c_i32, [c_i32, c_i32, c_vp, c_vp, c_i32, c_vp]),
}


def peaks_lib() -> ctypes.CDLL:
    """The microbenchmark library (include/sink_attn_peaks.h); raises if it
    has not been built."""
    global _peaks
    if _peaks is None:
        if not os.path.exists(PEAKS_LIB_PATH):
            raise RuntimeError(f"{PEAKS_LIB_PATH} is missing: build it with "
                               "`python -m streamingllm_sink_attn_amd.build`")
        h = ctypes.CDLL(PEAKS_LIB_PATH)
        for name, (res, args) in PEAKS_SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _peaks = h
    return _peaks


def _check(status: int):
    if status != OK:
        detail = lib().sink_attn_last_error().decode()
        raise SinkAttnError(status, f"{lib().sink_attn_strerror(status).decode()}: {detail}")


def _p(t: Optional[torch.Tensor]):
    return None if t is None else c_vp(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise SinkAttnError(UNSUPPORTED, f"dtype {t.dtype} not supported")


def _stream(stream) -> c_vp:
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_vp(stream.cuda_stream)


@contextlib.contextmanager
def _on_stream(stream):
    """Makes ``stream`` current for the allocations of one call (a no-op for
    the current stream): outputs and workspace then belong to the stream
    the kernels are enqueued on."""
    if stream is None:
        yield None
    else:
        with torch.cuda.stream(stream):
            yield stream


# ---------------------------------------------------------------------------
# Host-side precondition checks (SINK_ATTN_DEBUG=1)
# ---------------------------------------------------------------------------

def debug_enabled() -> bool:
    return os.environ.get("SINK_ATTN_DEBUG", "") == "1"


def _host_ints(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu").numpy()
    return np.asarray(x).astype(np.int64)


def _bad(msg: str):
    raise SinkAttnError(INVALID_ARGUMENT, f"precondition: {msg}")


def check_prefill_preconditions(cu_seqlens, total_tokens: int, max_seqlen: int,
                                block_indices=None, block_size: int = BLOCK_SIZE) -> None:
    """The device-side preconditions of a packed prefill call: cu_seqlens[0] =
    0, nondecreasing, cu_seqlens[batch] = total_tokens, every length <=
    max_seqlen; with block lists, num_q_blocks >= sum_b ceil(L_b / 64) and
    every entry of sample b's rows in [-1, ceil(L_b / 64))."""
    cu = _host_ints(cu_seqlens).reshape(-1)
    if cu.size == 0:
        _bad("cu_seqlens is empty (it holds batch + 1 entries)")
    if cu[0] != 0:
        _bad(f"cu_seqlens[0] = {cu[0]}, must be 0")
    lengths = np.diff(cu)
    if np.any(lengths < 0):
        b = int(np.nonzero(lengths < 0)[0][0])
        _bad(f"cu_seqlens decreases at sample {b} ({cu[b]} -> {cu[b + 1]})")
    if cu[-1] != int(total_tokens):
        _bad(f"cu_seqlens[batch] = {cu[-1]} != total_tokens = {total_tokens}")
    if lengths.size and int(lengths.max()) > int(max_seqlen):
        b = int(np.argmax(lengths))
        _bad(f"sample {b} has length {int(lengths[b])} > max_seqlen = {max_seqlen}")
    if block_indices is None:
        return
    bi = _host_ints(block_indices)
    if bi.ndim != 3:
        _bad("block_indices must be [num_q_blocks, num_kv_heads, max_blocks]")
    nqb = -(-lengths // block_size)
    if bi.shape[0] < int(nqb.sum()):
        _bad(f"block_indices has {bi.shape[0]} rows < sum_b ceil(L_b / {block_size}) = {int(nqb.sum())}")
    off = 0
    for b, n in enumerate(nqb):
        rows = bi[off:off + int(n)]
        if rows.size and (rows.min() < -1 or rows.max() >= n):
            _bad(f"sample {b}: block ids must be in [-1, {int(n)}), found "
                 f"[{int(rows.min())}, {int(rows.max())}]")
        off += int(n)


def check_decode_preconditions(cache_seqlens, slots: int) -> None:
    """1 <= cache_seqlens[b] <= slots for every sequence."""
    if cache_seqlens is None:
        return
    c = _host_ints(cache_seqlens).reshape(-1)
    if c.size and (c.min() < 1 or c.max() > int(slots)):
        b = int(np.argmin(c)) if c.min() < 1 else int(np.argmax(c))
        _bad(f"cache_seqlens[{b}] = {int(c[b])} outside [1, {slots}]")


def check_stream_positions(counts, name: str, chunk: int = 0) -> None:
    """Stream positions of the rolling cache: counts[b] >= 0 and
    counts[b] + chunk < 2^31."""
    c = _host_ints(counts).reshape(-1)
    if c.size and c.min() < 0:
        b = int(np.argmin(c))
        _bad(f"{name}[{b}] = {int(c[b])} < 0")
    if c.size and int(c.max()) + int(chunk) >= 2 ** 31:
        b = int(np.argmax(c))
        _bad(f"{name}[{b}] + chunk = {int(c[b]) + int(chunk)} >= 2^31")


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise SinkAttnError(INVALID_ARGUMENT, "tensors must be on the GPU")
            if not t.is_contiguous():
                raise SinkAttnError(INVALID_ARGUMENT, "tensors must be contiguous")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def prefill_desc(q: torch.Tensor, k: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                 softmax_scale: float, n_sink: int = 0, window: int = 0,
                 block_indices: Optional[torch.Tensor] = None,
                 learnable_sink: Optional[torch.Tensor] = None) -> PrefillDesc:
    T, hq, d = q.shape
    nqb = int(block_indices.shape[0]) if block_indices is not None else 0
    kb = int(block_indices.shape[2]) if block_indices is not None else 0
    return PrefillDesc(
        cu_seqlens=cu_seqlens.data_ptr() if cu_seqlens is not None else None,
        batch=(cu_seqlens.numel() - 1) if cu_seqlens is not None else 0,
        total_tokens=T, max_seqlen=int(max_seqlen), num_q_heads=hq, num_kv_heads=int(k.shape[1]),
        head_dim=d, dtype=_dtype_code(q), softmax_scale=float(softmax_scale), n_sink=int(n_sink),
        window=int(window),
        block_indices=block_indices.data_ptr() if block_indices is not None else None,
        num_q_blocks=nqb, block_size=BLOCK_SIZE, max_blocks=kb,
        learnable_sink=learnable_sink.data_ptr() if learnable_sink is not None else None)


def _max_seqlen(cu_seqlens: torch.Tensor, max_seqlen: Optional[int]) -> int:
    if max_seqlen is not None:
        return int(max_seqlen)
    c = cu_seqlens.detach().to("cpu")
    return int((c[1:] - c[:-1]).max().item()) if c.numel() > 1 else 0


def fwd(q, k, v, cu_seqlens, max_seqlen=None, softmax_scale=None, n_sink=0, window=0,
        block_indices=None, learnable_sink=None, return_s=True, out=None, stream=None,
        gate0=None):
    """Forward.  Returns (o [T,Hq,D], lse [T,Hq] float32 L_orig, s [T,Hq] or None).

    gate0: None, or a float32 [T,Hq] tensor that receives the first-token gate
    (sink_attn_fwd_gated).
    """
    _need_cuda(q, k, v, cu_seqlens, block_indices, learnable_sink)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    ms = _max_seqlen(cu_seqlens, max_seqlen)
    desc = prefill_desc(q, k, cu_seqlens, ms, scale, n_sink, window, block_indices, learnable_sink)
    if debug_enabled():
        check_prefill_preconditions(cu_seqlens, q.shape[0], ms, block_indices)
    T, hq, _ = q.shape
    with _on_stream(stream):
        o = out if out is not None else torch.empty_like(q)
        lse = torch.empty((T, hq), dtype=torch.float32, device=q.device)
        s = torch.empty((T, hq), dtype=torch.float32, device=q.device) if return_s else None
        L = lib()
        ws_bytes = L.sink_attn_fwd_workspace_size(ctypes.byref(desc))
        ws = _workspace(ws_bytes, q.device)
        if gate0 is None:
            _check(L.sink_attn_fwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(o), _p(lse), _p(s),
                                   _p(ws), ws_bytes, _stream(stream)))
        else:
            _need_cuda(gate0)
            if gate0.dtype != torch.float32 or tuple(gate0.shape) != (T, hq):
                raise SinkAttnError(INVALID_ARGUMENT, "gate0 must be float32 [T, Hq]")
            _check(L.sink_attn_fwd_gated(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(o), _p(lse),
                                         _p(s), _p(gate0), _p(ws), ws_bytes, _stream(stream)))
    return o, lse, s


def fwd_gated(q, k, v, cu_seqlens, max_seqlen=None, softmax_scale=None, n_sink=0, window=0,
              block_indices=None, learnable_sink=None, return_s=True, out=None, stream=None):
    """Forward plus the first-token gate.  Returns (o, lse, s or None, gate0 [T,Hq] float32)."""
    with _on_stream(stream):
        gate0 = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    o, lse, s = fwd(q, k, v, cu_seqlens, max_seqlen, softmax_scale, n_sink, window, block_indices,
                    learnable_sink, return_s, out, stream, gate0=gate0)
    return o, lse, s, gate0


def head_importance(gate, out=None, stream=None):
    """Mean of a per-row gate [rows, H] over the rows: float32 [H] (deterministic)."""
    _need_cuda(gate)
    if gate.dtype != torch.float32 or gate.dim() != 2:
        raise SinkAttnError(INVALID_ARGUMENT, "gate must be float32 [rows, heads]")
    rows, heads = int(gate.shape[0]), int(gate.shape[1])
    with _on_stream(stream):
        imp = out if out is not None else torch.empty(heads, dtype=torch.float32, device=gate.device)
        L = lib()
        ws_bytes = L.sink_attn_head_importance_workspace_size(rows, heads)
        ws = _workspace(ws_bytes, gate.device)
        _check(L.sink_attn_head_importance(_p(gate), rows, heads, _p(imp), _p(ws), ws_bytes,
                                           _stream(stream)))
    return imp


def bwd(q, k, v, o, lse, dout, cu_seqlens, max_seqlen=None, softmax_scale=None, n_sink=0, window=0,
        block_indices=None, learnable_sink=None, stream=None):
    """Backward.  Returns (dq, dk, dv, dsink float32 [Hq] or None).  The
    library runs part of the work on its own second stream, forked from and
    joined back into the call's stream inside the call, so the outputs are
    ordered on the call's stream (SINK_ATTN_SERIAL_BWD=1: one stream)."""
    _need_cuda(q, k, v, o, lse, dout, cu_seqlens, block_indices, learnable_sink)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    ms = _max_seqlen(cu_seqlens, max_seqlen)
    desc = prefill_desc(q, k, cu_seqlens, ms, scale, n_sink, window, block_indices, learnable_sink)
    if debug_enabled():
        check_prefill_preconditions(cu_seqlens, q.shape[0], ms, block_indices)
    with _on_stream(stream):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dsink = (torch.empty(q.shape[1], dtype=torch.float32, device=q.device)
                 if learnable_sink is not None else None)
        L = lib()
        ws_bytes = L.sink_attn_bwd_workspace_size(ctypes.byref(desc))
        ws = _workspace(ws_bytes, q.device)
        _check(L.sink_attn_bwd(ctypes.byref(desc), _p(q), _p(k), _p(v), _p(o), _p(lse), _p(dout),
                               _p(dq), _p(dk), _p(dv), _p(dsink), _p(ws), ws_bytes, _stream(stream)))
    return dq, dk, dv, dsink


def decode_desc(q, k_cache, softmax_scale, cache_seqlens=None, learnable_sink=None,
                num_splits=0) -> DecodeDesc:
    B, hq, d = q.shape
    return DecodeDesc(
        cache_seqlens=cache_seqlens.data_ptr() if cache_seqlens is not None else None,
        batch=B, slots=int(k_cache.shape[1]), num_q_heads=hq, num_kv_heads=int(k_cache.shape[2]),
        head_dim=d, dtype=_dtype_code(q), softmax_scale=float(softmax_scale),
        learnable_sink=learnable_sink.data_ptr() if learnable_sink is not None else None,
        num_splits=int(num_splits))


def decode(q, k_cache, v_cache, cache_seqlens=None, softmax_scale=None, learnable_sink=None,
           num_splits=0, return_s=True, out=None, stream=None):
    """Decode.  Returns (o [B,Hq,D], lse [B,Hq] L_orig, s [B,Hq] or None)."""
    _need_cuda(q, k_cache, v_cache, cache_seqlens, learnable_sink)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    desc = decode_desc(q, k_cache, scale, cache_seqlens, learnable_sink, num_splits)
    if debug_enabled():
        check_decode_preconditions(cache_seqlens, int(k_cache.shape[1]))
    B, hq, _ = q.shape
    with _on_stream(stream):
        o = out if out is not None else torch.empty_like(q)
        lse = torch.empty((B, hq), dtype=torch.float32, device=q.device)
        s = torch.empty((B, hq), dtype=torch.float32, device=q.device) if return_s else None
        L = lib()
        ws_bytes = L.sink_attn_decode_workspace_size(ctypes.byref(desc))
        ws = _workspace(ws_bytes, q.device)
        _check(L.sink_attn_decode(ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(o), _p(lse),
                                  _p(s), _p(ws), ws_bytes, _stream(stream)))
    return o, lse, s


def decode_noalloc(q, k_cache, v_cache, cache_seqlens=None, softmax_scale=None, learnable_sink=None,
                   num_splits=0, o=None, lse=None, s=None, stream=None):
    """Decode through sink_attn_decode_noalloc: the library allocates nothing
    (split partials in its static per-GPU scratch).  The caller passes the
    outputs o [B,Hq,D], lse [B,Hq] float32 and s [B,Hq] float32 or None; when
    omitted they are allocated here, before the call.  Returns (o, lse, s)."""
    _need_cuda(q, k_cache, v_cache, cache_seqlens, learnable_sink, o, lse, s)
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    desc = decode_desc(q, k_cache, scale, cache_seqlens, learnable_sink, num_splits)
    if debug_enabled():
        check_decode_preconditions(cache_seqlens, int(k_cache.shape[1]))
    B, hq, _ = q.shape
    with _on_stream(stream):
        o = o if o is not None else torch.empty_like(q)
        lse = lse if lse is not None else torch.empty((B, hq), dtype=torch.float32, device=q.device)
    _expect(o, tuple(q.shape), q.dtype, "o")
    _expect(lse, (B, hq), torch.float32, "lse")
    _expect(s, (B, hq), torch.float32, "s")
    _check(lib().sink_attn_decode_noalloc(ctypes.byref(desc), _p(q), _p(k_cache), _p(v_cache), _p(o),
                                          _p(lse), _p(s), _stream(stream)))
    return o, lse, s


class KvCache:
    """StreamingLLM rolling KV cache in device memory (the layouts of
    sink_attn_kvcache_desc): bfloat16 [B, n_sink + window, Hkv, D] K and V, or
    with ``quantized`` bfloat16 first tokens plus an e4m3 ring with float32
    scales."""

    def __init__(self, batch, n_sink, window, num_kv_heads, head_dim=128, quantized=False,
                 device="cuda"):
        self.batch, self.n_sink, self.window = int(batch), int(n_sink), int(window)
        self.hkv, self.d, self.quantized = int(num_kv_heads), int(head_dim), bool(quantized)
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        B, hkv, d = self.batch, self.hkv, self.d
        if not self.quantized:
            self.k = z((B, n_sink + window, hkv, d), torch.bfloat16)
            self.v = z((B, n_sink + window, hkv, d), torch.bfloat16)
            self.sink_k = self.sink_v = self.win_k = self.win_v = None
            self.win_k_scale = self.win_v_scale = None
        else:
            self.k = self.v = None
            self.sink_k = z((B, n_sink, hkv, d), torch.bfloat16)
            self.sink_v = z((B, n_sink, hkv, d), torch.bfloat16)
            self.win_k = z((B, window, hkv, d), torch.uint8)
            self.win_v = z((B, window, hkv, d), torch.uint8)
            self.win_k_scale = z((B, hkv, window), torch.float32)
            self.win_v_scale = z((B, hkv, window), torch.float32)

    def desc(self) -> KvCacheDesc:
        ptr = lambda t: t.data_ptr() if t is not None and t.numel() > 0 else None
        return KvCacheDesc(batch=self.batch, n_sink=self.n_sink, window=self.window,
                           num_kv_heads=self.hkv, head_dim=self.d, quantized=int(self.quantized),
                           k=ptr(self.k), v=ptr(self.v), sink_k=ptr(self.sink_k),
                           sink_v=ptr(self.sink_v), win_k=ptr(self.win_k), win_v=ptr(self.win_v),
                           win_k_scale=ptr(self.win_k_scale), win_v_scale=ptr(self.win_v_scale))


def _expect(t, shape, dtype, name):
    """The C ABI sees pointers only: shapes and dtypes are checked here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise SinkAttnError(INVALID_ARGUMENT, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise SinkAttnError(INVALID_ARGUMENT, f"{name} has dtype {t.dtype}, expected {dtype}")


def _heads(q, cache: KvCache, axis):
    hq = int(q.shape[axis]) if q.dim() > axis else 0
    if hq < 1 or hq % cache.hkv != 0:
        raise SinkAttnError(INVALID_ARGUMENT, "query heads must be a positive multiple of the cache's KV heads")
    return hq


def kvcache_append(cache: KvCache, k_new, v_new, n_seen, stream=None):
    """Append k_new, v_new (bf16 [B, C, Hkv, D]) at stream positions n_seen[b] + c."""
    _need_cuda(k_new, v_new, n_seen)
    C = int(k_new.shape[1]) if k_new.dim() == 4 else -1
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _expect(t, (cache.batch, C, cache.hkv, cache.d), torch.bfloat16, name)
    _expect(n_seen, (cache.batch,), torch.int32, "n_seen")
    if debug_enabled():
        check_stream_positions(n_seen, "n_seen", C)
    desc = cache.desc()
    _check(lib().sink_attn_kvcache_append(ctypes.byref(desc), _p(k_new), _p(v_new),
                                          int(k_new.shape[1]), _p(n_seen), _stream(stream)))


def kvcache_decode(cache: KvCache, q, n_tokens, softmax_scale=None, learnable_sink=None,
                   num_splits=0, return_s=True, out=None, stream=None):
    """Decode one query per sequence over the cache (n_tokens[b] tokens appended,
    the current one included).  Returns (o, lse, s or None)."""
    _need_cuda(q, n_tokens, learnable_sink, out)
    hq = _heads(q, cache, 1)
    B = cache.batch
    _expect(q, (B, hq, cache.d), torch.bfloat16, "q")
    _expect(n_tokens, (B,), torch.int32, "n_tokens")
    _expect(learnable_sink, (hq,), torch.float32, "learnable_sink")
    _expect(out, (B, hq, cache.d), torch.bfloat16, "out")
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    if debug_enabled():
        check_stream_positions(n_tokens, "n_tokens")
    desc = cache.desc()
    with _on_stream(stream):
        o = out if out is not None else torch.empty_like(q)
        lse = torch.empty((B, hq), dtype=torch.float32, device=q.device)
        s = torch.empty((B, hq), dtype=torch.float32, device=q.device) if return_s else None
        L = lib()
        ws_bytes = L.sink_attn_kvcache_decode_workspace_size(ctypes.byref(desc), hq, int(num_splits))
        ws = _workspace(ws_bytes, q.device)
        _check(L.sink_attn_kvcache_decode(ctypes.byref(desc), _p(q), hq, _p(n_tokens), float(scale),
                                          _p(learnable_sink), int(num_splits), _p(o), _p(lse), _p(s),
                                          _p(ws), ws_bytes, _stream(stream)))
    return o, lse, s


def kvcache_prefill(cache: KvCache, q, k_new, v_new, n_seen, softmax_scale=None, learnable_sink=None,
                    return_s=True, out=None, stream=None):
    """Chunked prefill against the cache: q [B, C, Hq, D] at stream positions
    n_seen[b] + c attends to the kept first tokens, the window (cache as it is
    before this chunk) and the chunk itself.  The cache is not written: call
    kvcache_append(cache, k_new, v_new, n_seen) afterwards.  Returns (o [B, C,
    Hq, D], lse [B, C, Hq], s or None)."""
    _need_cuda(q, k_new, v_new, n_seen, learnable_sink, out)
    hq = _heads(q, cache, 2)
    B, C = cache.batch, int(q.shape[1])
    _expect(q, (B, C, hq, cache.d), torch.bfloat16, "q")
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        _expect(t, (B, C, cache.hkv, cache.d), torch.bfloat16, name)
    _expect(n_seen, (B,), torch.int32, "n_seen")
    _expect(learnable_sink, (hq,), torch.float32, "learnable_sink")
    _expect(out, (B, C, hq, cache.d), torch.bfloat16, "out")
    scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
    if debug_enabled():
        check_stream_positions(n_seen, "n_seen", C)
    desc = cache.desc()
    with _on_stream(stream):
        o = out if out is not None else torch.empty_like(q)
        lse = torch.empty((B, C, hq), dtype=torch.float32, device=q.device)
        s = torch.empty((B, C, hq), dtype=torch.float32, device=q.device) if return_s else None
        L = lib()
        ws_bytes = L.sink_attn_kvcache_prefill_workspace_size(ctypes.byref(desc), C, hq)
        ws = _workspace(ws_bytes, q.device)
        _check(L.sink_attn_kvcache_prefill(ctypes.byref(desc), _p(q), hq, _p(k_new), _p(v_new), C,
                                           _p(n_seen), float(scale), _p(learnable_sink), _p(o), _p(lse),
                                           _p(s), _p(ws), ws_bytes, _stream(stream)))
    return o, lse, s


def prefill_path(q, k, cu_seqlens, max_seqlen, n_sink=0, window=0, block_indices=None) -> int:
    desc = prefill_desc(q, k, cu_seqlens, max_seqlen, 1.0, n_sink, window, block_indices, None)
    return int(lib().sink_attn_prefill_path(ctypes.byref(desc)))


def debug_visit_map(q, k, cu_seqlens, max_seqlen, n_sink=0, window=0, block_indices=None,
                    stream=None) -> torch.Tensor:
    """uint8 [Hkv * max_seqlen * T] buffer; sample b's masks start at
    Hkv * sum_{b'<b} L_b'^2, each [L_b, L_b] row-major per KV head."""
    desc = prefill_desc(q, k, cu_seqlens, max_seqlen, 1.0, n_sink, window, block_indices, None)
    nbytes = int(k.shape[1]) * int(max_seqlen) * int(q.shape[0])
    with _on_stream(stream):
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
        _check(lib().sink_attn_debug_visit_map(ctypes.byref(desc), _p(out), nbytes, _stream(stream)))
    return out
