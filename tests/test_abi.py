"""The C ABI on the CPU: the library loads, exports every declared symbol, and
its pure-host validation returns the documented status codes.  No call here
launches a kernel; pointers are fake, aligned addresses that are never read."""
import ctypes
import os
import re

import pytest

from streamingllm_sink_attn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sink_attn.h")

FAKE = 0x10000          # aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sink_attn_[a-z_]+)\s*\(", text)))


def test_peaks_library_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "sink_attn_peaks.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(sink_attn_peaks_[a-z_]+)\s*\(", text)))
    assert len(names) == 5
    lib = B.peaks_lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.PEAKS_SIGS)
    # invalid arguments are refused before anything is launched
    assert lib.sink_attn_peaks_read(None, 16, FAKE, 1, None) == 1
    assert lib.sink_attn_peaks_read(FAKE, 15, FAKE, 1, None) == 1
    assert lib.sink_attn_peaks_mfma(0, FAKE, 1, None) == 1
    assert lib.sink_attn_peaks_exp(5, None, 1, None) == 1
    assert lib.sink_attn_peaks_coissue(4, 10, FAKE, FAKE, 1, None) == 1      # no such mode
    assert lib.sink_attn_peaks_coissue(0, 10, FAKE, None, 1, None) == 1
    assert lib.sink_attn_peaks_lds(3, 10, FAKE, FAKE, 1, None) == 1
    assert lib.sink_attn_peaks_lds(0, 0, FAKE, FAKE, 1, None) == 1


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B._SIGS), "binding signatures must cover the header"


def _desc(**kw):
    d = dict(cu_seqlens=FAKE, batch=2, total_tokens=100, max_seqlen=60, num_q_heads=8,
             num_kv_heads=2, head_dim=128, dtype=B.BF16, softmax_scale=0.088, n_sink=4,
             window=32, block_indices=None, num_q_blocks=0, block_size=64, max_blocks=0,
             learnable_sink=FAKE)
    d.update(kw)
    return B.PrefillDesc(**d)


def check_fwd(desc, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, s=FAKE, ws=0):
    return B.lib().sink_attn_check_fwd(ctypes.byref(desc), q, k, v, o, lse, s, ws)


def check_bwd(desc, dsink=FAKE, ws=None, **kw):
    p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
    p.update(kw)
    if ws is None:
        ws = B.lib().sink_attn_bwd_workspace_size(ctypes.byref(desc))
    return B.lib().sink_attn_check_bwd(ctypes.byref(desc), p["q"], p["k"], p["v"], p["o"], p["lse"],
                                       p["dout"], p["dq"], p["dk"], p["dv"], dsink, ws)


def test_check_fwd_ok_and_errors():
    assert check_fwd(_desc()) == B.OK
    assert check_fwd(_desc(), s=None) == B.OK                        # s optional
    assert B.lib().sink_attn_check_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(), q=None) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(), lse=None) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(), q=FAKE + 2) == B.INVALID_ARGUMENT       # misaligned
    assert check_fwd(_desc(num_q_heads=6, num_kv_heads=4)) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(num_kv_heads=0)) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(head_dim=100)) == B.UNSUPPORTED
    assert check_fwd(_desc(head_dim=512)) == B.UNSUPPORTED
    assert check_fwd(_desc(dtype=7)) == B.UNSUPPORTED
    assert check_fwd(_desc(softmax_scale=0.0)) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(softmax_scale=float("nan"))) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(n_sink=-1)) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(batch=-1)) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(cu_seqlens=None)) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(max_seqlen=0)) == B.INVALID_ARGUMENT
    # empty problem: nothing required
    assert check_fwd(_desc(total_tokens=0, batch=0, cu_seqlens=None), q=None, k=None, v=None,
                     o=None, lse=None) == B.OK
    # block lists
    bd = dict(block_indices=FAKE, num_q_blocks=2, max_blocks=3)
    assert check_fwd(_desc(**bd)) == B.OK
    assert check_fwd(_desc(**dict(bd, block_size=32))) == B.UNSUPPORTED
    assert check_fwd(_desc(**dict(bd, max_blocks=0))) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(**dict(bd, num_q_blocks=1))) == B.INVALID_ARGUMENT
    assert check_fwd(_desc(**dict(bd, max_seqlen=10**6, total_tokens=10**6, num_q_blocks=20000))) == B.UNSUPPORTED


def test_last_error_message_and_strerror():
    check_fwd(_desc(head_dim=100))
    assert "head_dim" in B.lib().sink_attn_last_error().decode()
    for st in range(5):
        assert B.lib().sink_attn_strerror(st)
    assert B.lib().sink_attn_strerror(99) == b"unknown status"


def test_check_bwd_dsink_rules_and_workspace():
    d = _desc()
    assert check_bwd(d) == B.OK
    assert check_bwd(d, dsink=None) == B.INVALID_ARGUMENT             # sink set, dsink missing
    assert check_bwd(_desc(learnable_sink=None), dsink=FAKE) == B.INVALID_ARGUMENT
    assert check_bwd(_desc(learnable_sink=None), dsink=None) == B.OK
    need = B.lib().sink_attn_bwd_workspace_size(ctypes.byref(d))
    assert need >= 3 * 100 * 8 * 4
    assert check_bwd(d, ws=need - 1) == B.WORKSPACE_TOO_SMALL
    assert check_bwd(d, dq=None) == B.INVALID_ARGUMENT
    assert check_bwd(d, dout=FAKE + 8) == B.INVALID_ARGUMENT


def _ddesc(**kw):
    d = dict(cache_seqlens=None, batch=4, slots=128, num_q_heads=8, num_kv_heads=2, head_dim=128,
             dtype=B.BF16, softmax_scale=0.088, learnable_sink=FAKE, num_splits=0)
    d.update(kw)
    return B.DecodeDesc(**d)


def test_check_decode():
    L = B.lib()

    def chk(desc, ws=None, **kw):
        p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, s=FAKE)
        p.update(kw)
        if ws is None:
            ws = L.sink_attn_decode_workspace_size(ctypes.byref(desc))
        return L.sink_attn_check_decode(ctypes.byref(desc), p["q"], p["k"], p["v"], p["o"], p["lse"],
                                        p["s"], ws)
    assert chk(_ddesc()) == B.OK
    assert chk(_ddesc(), s=None) == B.OK
    assert chk(_ddesc(slots=0)) == B.INVALID_ARGUMENT
    assert chk(_ddesc(num_splits=-1)) == B.INVALID_ARGUMENT
    assert chk(_ddesc(num_splits=1000)) == B.INVALID_ARGUMENT
    assert chk(_ddesc(head_dim=12)) == B.UNSUPPORTED
    assert chk(_ddesc(), k=None) == B.INVALID_ARGUMENT
    need = L.sink_attn_decode_workspace_size(ctypes.byref(_ddesc()))
    if need:
        assert chk(_ddesc(), ws=need - 1) == B.WORKSPACE_TOO_SMALL
    # one split writes O itself: no partials, no workspace
    assert L.sink_attn_decode_workspace_size(ctypes.byref(_ddesc(num_splits=1))) == 0
    need3 = L.sink_attn_decode_workspace_size(ctypes.byref(_ddesc(num_splits=3)))
    assert need3 >= 4 * 8 * 3 * 130 * 4
    assert chk(_ddesc(num_splits=3), ws=need3 - 1) == B.WORKSPACE_TOO_SMALL


def test_prefill_path_selection():
    L = B.lib()
    assert L.sink_attn_prefill_path(ctypes.byref(_desc())) == 1             # bf16, D=128
    assert L.sink_attn_prefill_path(ctypes.byref(_desc(head_dim=64))) == 0
    assert L.sink_attn_prefill_path(ctypes.byref(_desc(dtype=B.F32))) == 0
    assert L.sink_attn_prefill_path(ctypes.byref(_desc(head_dim=100))) == -1


def test_product_path_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libsinkattn.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_check_fwd_gated_and_head_importance():
    L = B.lib()

    def chk_g(desc, gate0=FAKE, **kw):
        p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, s=FAKE)
        p.update(kw)
        return L.sink_attn_check_fwd_gated(ctypes.byref(desc), p["q"], p["k"], p["v"], p["o"],
                                           p["lse"], p["s"], gate0, 0)
    assert chk_g(_desc()) == B.OK
    assert chk_g(_desc(), gate0=None) == B.OK                       # gate optional
    assert chk_g(_desc(), gate0=FAKE + 2) == B.INVALID_ARGUMENT     # misaligned
    assert chk_g(_desc(head_dim=100)) == B.UNSUPPORTED              # the forward's own checks

    def chk_i(rows, heads, gate=FAKE, imp=FAKE, ws=None):
        if ws is None:
            ws = L.sink_attn_head_importance_workspace_size(rows, heads)
        return L.sink_attn_check_head_importance(gate, rows, heads, imp, ws)
    assert chk_i(1000, 32) == B.OK
    need = L.sink_attn_head_importance_workspace_size(1000, 32)
    assert need >= 32 * 4 * (1000 // 64)
    assert chk_i(1000, 32, ws=need - 1) == B.WORKSPACE_TOO_SMALL
    assert chk_i(0, 32, gate=None) == B.OK                           # no rows: gate not needed
    assert L.sink_attn_head_importance_workspace_size(0, 32) == 0
    assert chk_i(-1, 32) == B.INVALID_ARGUMENT
    assert chk_i(10, 0) == B.INVALID_ARGUMENT
    assert chk_i(10, 4, imp=None) == B.INVALID_ARGUMENT
    assert chk_i(10, 4, gate=FAKE + 1) == B.INVALID_ARGUMENT


def _kdesc(**kw):
    d = dict(batch=4, n_sink=4, window=100, num_kv_heads=2, head_dim=128, quantized=0, k=FAKE,
             v=FAKE, sink_k=None, sink_v=None, win_k=None, win_v=None, win_k_scale=None,
             win_v_scale=None)
    d.update(kw)
    return B.KvCacheDesc(**d)


_Q8 = dict(quantized=1, k=None, v=None, sink_k=FAKE, sink_v=FAKE, win_k=FAKE, win_v=FAKE,
           win_k_scale=FAKE, win_v_scale=FAKE)


def test_check_kvcache_append_and_decode():
    L = B.lib()

    def app(desc, chunk=8, k=FAKE, v=FAKE, n=FAKE):
        return L.sink_attn_check_kvcache_append(ctypes.byref(desc), k, v, chunk, n)

    def dec(desc, hq=8, n=FAKE, scale=0.1, splits=0, q=FAKE, o=FAKE, lse=FAKE, s=None, ws=None):
        if ws is None:
            ws = L.sink_attn_kvcache_decode_workspace_size(ctypes.byref(desc), hq, splits)
        return L.sink_attn_check_kvcache_decode(ctypes.byref(desc), q, hq, n, scale, splits, o, lse, s,
                                                ws)
    assert app(_kdesc()) == B.OK and app(_kdesc(**_Q8)) == B.OK
    assert app(_kdesc(), chunk=0, k=None, v=None, n=None) == B.OK        # nothing to append
    assert app(_kdesc(), chunk=-1) == B.INVALID_ARGUMENT
    assert app(_kdesc(), n=None) == B.INVALID_ARGUMENT
    assert app(_kdesc(window=0)) == B.INVALID_ARGUMENT
    assert app(_kdesc(n_sink=-1)) == B.INVALID_ARGUMENT
    assert app(_kdesc(quantized=2)) == B.INVALID_ARGUMENT
    assert app(_kdesc(head_dim=64)) == B.OK                                 # bf16 layout: any D
    assert app(_kdesc(head_dim=64, **_Q8)) == B.UNSUPPORTED                 # 8-bit ring: D = 128
    assert app(_kdesc(k=None)) == B.INVALID_ARGUMENT                        # bf16 layout needs k, v
    assert app(_kdesc(**dict(_Q8, win_k_scale=None))) == B.INVALID_ARGUMENT
    assert app(_kdesc(**dict(_Q8, n_sink=0, sink_k=None, sink_v=None))) == B.OK
    assert app(_kdesc(**dict(_Q8, win_k=FAKE + 8))) == B.INVALID_ARGUMENT   # misaligned
    assert dec(_kdesc()) == B.OK and dec(_kdesc(**_Q8)) == B.OK
    assert dec(_kdesc(), hq=5) == B.INVALID_ARGUMENT                        # not a multiple of Hkv
    assert dec(_kdesc(), n=None) == B.INVALID_ARGUMENT
    assert dec(_kdesc(), scale=0.0) == B.INVALID_ARGUMENT
    assert dec(_kdesc(), splits=300) == B.INVALID_ARGUMENT
    for q8 in ({}, _Q8):
        need = L.sink_attn_kvcache_decode_workspace_size(ctypes.byref(_kdesc(**q8)), 8, 4)
        assert need >= 4 * 8 * 4 * 130 * 4                                  # B * Hq * splits * (D + 2)
        assert dec(_kdesc(**q8), splits=4, ws=need - 1) == B.WORKSPACE_TOO_SMALL
    # one split on the 8-bit ring: no partials, no workspace
    assert L.sink_attn_kvcache_decode_workspace_size(ctypes.byref(_kdesc(**_Q8)), 8, 1) == 0


def test_check_kvcache_prefill():
    L = B.lib()

    def pre(desc, hq=8, chunk=16, q=FAKE, k=FAKE, v=FAKE, n=FAKE, scale=0.1, o=FAKE, lse=FAKE, s=None,
            ws=None):
        if ws is None:
            ws = L.sink_attn_kvcache_prefill_workspace_size(ctypes.byref(desc), chunk, hq)
        return L.sink_attn_check_kvcache_prefill(ctypes.byref(desc), q, hq, k, v, chunk, n, scale, o, lse,
                                                 s, ws)
    assert pre(_kdesc()) == B.OK and pre(_kdesc(**_Q8)) == B.OK
    assert pre(_kdesc(), chunk=0, q=None, k=None, v=None, n=None, o=None, lse=None) == B.OK
    assert L.sink_attn_kvcache_prefill_workspace_size(ctypes.byref(_kdesc()), 0, 8) == 0
    assert pre(_kdesc(), chunk=-1) == B.INVALID_ARGUMENT
    assert pre(_kdesc(), hq=5) == B.INVALID_ARGUMENT                        # not a multiple of Hkv
    assert pre(_kdesc(), scale=float("nan")) == B.INVALID_ARGUMENT
    for name in ("q", "k", "v", "n", "o", "lse"):
        assert pre(_kdesc(), **{name: None}) == B.INVALID_ARGUMENT, name
    assert pre(_kdesc(), q=FAKE + 4) == B.INVALID_ARGUMENT                  # misaligned
    assert pre(_kdesc(), s=FAKE) == B.OK
    assert pre(_kdesc(head_dim=64, **_Q8)) == B.UNSUPPORTED
    for hd, quant in ((128, False), (64, False), (128, True)):
        d = _kdesc(head_dim=hd, **(_Q8 if quant else {}))
        need = L.sink_attn_kvcache_prefill_workspace_size(ctypes.byref(d), 16, 8)
        rows = d.batch * (d.n_sink + d.window + 16)
        kv = 2 * d.num_kv_heads * hd * 2                 # a K and a V row of Hkv heads, bf16
        qo = 0 if hd == 128 else 2 * 8 * hd * 2 + 2 * 8 * 4
        if hd == 128 and not quant:
            # the bf16 cache with head_dim 128 is read in place: only the
            # three staged 64-row seam tiles of each stream
            staged = d.batch * 3 * 64 * kv
            assert staged <= need <= staged + 16 * 256
        else:
            # packed K, V; for head_dim other than 128 also packed Q, O (bf16)
            # and LSE, s (float32)
            assert rows * (kv + qo) <= need <= rows * (kv + qo) + 16 * 256
        assert pre(d, ws=need - 1) == B.WORKSPACE_TOO_SMALL
    assert pre(_kdesc(batch=60000, window=1 << 20)) == B.UNSUPPORTED         # packed rows past 2^31


def test_binding_cache_shape_checks():
    """The C ABI sees only pointers: the binding checks cache-call shapes."""
    import torch

    class _C:
        batch, hkv, d = 2, 2, 128
    t = torch.zeros((2, 5, 2, 128), dtype=torch.bfloat16)
    B._expect(t, (2, 5, 2, 128), torch.bfloat16, "k_new")
    B._expect(None, (1,), torch.int32, "unused")
    for shape, dtype in (((2, 5, 1, 128), torch.bfloat16), ((2, 5, 2, 128), torch.float32)):
        with pytest.raises(B.SinkAttnError):
            B._expect(t, shape, dtype, "k_new")
    assert B._heads(torch.zeros((2, 5, 8, 128)), _C, 2) == 8
    for hq in (0, 3):
        with pytest.raises(B.SinkAttnError):
            B._heads(torch.zeros((2, 5, hq, 128)), _C, 2)
