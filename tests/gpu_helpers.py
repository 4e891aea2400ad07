"""Shared helpers of the GPU parity tests: device copies of drawn workloads,
calls through the binding, and the tolerance checks."""
import numpy as np
import torch

import oracle
import streamingllm_sink_attn_amd as sa
from streamingllm_sink_attn_amd import workloads as W

DEV = "cuda"

# bf16 inputs, float32 accumulation.  Gradients are stored in bf16: rounding
# a value x to bf16 alone moves it by up to half an ulp, 2^-8 |x| at most, which
# passes 5e-2 once |x| >= 16 (a kept first token's dV sums every row of the
# sample); the absolute bound applies on top of that representation error.
TOL_BF16 = dict(o_max=2e-2, o_mean=2e-3, lse=1e-3, s=1e-3, grad=5e-2, grad_out_rel=2.0 ** -8,
                dsink_rel=1e-2)
# float32 storage
TOL_F32 = dict(o_max=1e-4, o_mean=1e-5, lse=1e-4, s=1e-4, grad=1e-4, grad_out_rel=0.0, dsink_rel=1e-4)


def tol_for(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def dev(t: W.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to(DEV)


def host(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def prefill_args(wl: W.Prefill):
    q, k, v = dev(wl.q, wl.dtype), dev(wl.k, wl.dtype), dev(wl.v, wl.dtype)
    cu = torch.from_numpy(wl.cu_seqlens).to(DEV)
    bi = torch.from_numpy(wl.block_indices).to(DEV) if wl.block_indices is not None else None
    sink = torch.from_numpy(wl.sink).to(DEV) if wl.sink is not None else None
    return q, k, v, cu, bi, sink


def run_fwd(wl: W.Prefill, args=None, max_seqlen=None):
    q, k, v, cu, bi, sink = args if args is not None else prefill_args(wl)
    ms = max_seqlen if max_seqlen is not None else wl.max_seqlen
    o, lse, s = sa.fwd(q, k, v, cu, ms, wl.scale, wl.n_sink, wl.window, bi, sink)
    torch.cuda.synchronize()
    return o, lse, s


def run_bwd(wl: W.Prefill, o, lse, args=None, max_seqlen=None):
    q, k, v, cu, bi, sink = args if args is not None else prefill_args(wl)
    do = dev(wl.do, wl.dtype)
    ms = max_seqlen if max_seqlen is not None else wl.max_seqlen
    g = sa.bwd(q, k, v, o, lse, do, cu, ms, wl.scale, wl.n_sink, wl.window, bi, sink)
    torch.cuda.synchronize()
    return g


def oracle_kwargs(wl: W.Prefill):
    return dict(n_sink=wl.n_sink, window=wl.window, block_indices=wl.block_indices,
                block_size=wl.block_size, sink=wl.sink)


def assert_lse(got, want, tol, what="lse"):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    ninf_w = np.isneginf(want)
    ninf_g = np.isneginf(got)
    assert np.array_equal(ninf_w, ninf_g), f"{what}: -inf pattern differs ({ninf_w.sum()} vs {ninf_g.sum()})"
    fin = ~ninf_w
    if fin.any():
        err = np.max(np.abs(got[fin] - want[fin]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol}"


def assert_out(got, want, tol, what="O"):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    assert mx <= tol["o_max"], f"{what}: max abs err {mx:.3e} > {tol['o_max']}"
    assert mean <= tol["o_mean"], f"{what}: mean abs err {mean:.3e} > {tol['o_mean']}"


def assert_grad(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    # error beyond the output type's own rounding of the exact value
    err = np.abs(got - want) - tol["grad_out_rel"] * np.abs(want)
    worst = float(np.max(err)) if got.size else 0.0
    assert worst <= tol["grad"], (f"{what}: max abs err beyond bf16 rounding {worst:.3e} > {tol['grad']}"
                                  f" (raw max abs err {float(np.max(np.abs(got - want))):.3e})")


def assert_dsink(got, want, tol):
    """Max-normalised check: the worst head's error over the largest |dsink|."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    scale = max(float(np.max(np.abs(want))), 1e-6)
    rel = float(np.max(np.abs(got - want))) / scale
    assert rel <= tol["dsink_rel"], f"dsink: relative err {rel:.3e} > {tol['dsink_rel']}"


def dsink_storage_floor(o_exact, do, lse_exact, sink, out_dtype):
    """Per head: the largest change of -sum_i Delta_i p_sink_i that rounding O
    to the output type can cause.  The backward forms Delta from the O the
    forward stored (it has no other), and rounding each O element to bf16
    moves it by at most half an ulp, 2^-9 |O|, so Delta_i moves by at most
    2^-9 sum_d |O_id dO_id|.  p_sink = sigma(a - L_orig) = exp(a - L_new)."""
    if out_dtype != "bf16":
        return np.zeros(np.asarray(sink).shape, np.float64)
    o = np.asarray(o_exact, np.float64)
    d = np.asarray(do, np.float64)
    lse = np.asarray(lse_exact, np.float64)
    a = np.asarray(sink, np.float64)[None, :]
    with np.errstate(over="ignore"):
        p_sink = 1.0 / (1.0 + np.exp(lse - a))     # -inf rows: 1 (their Delta is 0)
    mag = np.einsum("thd,thd->th", np.abs(o), np.abs(d))
    return 2.0 ** -9 * np.sum(p_sink * mag, axis=0)


def assert_dsink_per_head(got, want, tol, floor):
    """Every head on its own: |got_h - want_h| <= dsink_rel |want_h| + floor_h,
    with floor_h from dsink_storage_floor (the output type's rounding of O)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), "dsink: non-finite values"
    bound = tol["dsink_rel"] * np.abs(want) + np.asarray(floor, np.float64)
    err = np.abs(got - want)
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, ("dsink per head: " + ", ".join(
        f"h{h}: err {err[h]:.3e} > {bound[h]:.3e} (want {want[h]:.3e})" for h in bad[:6]))


def check_fwd_full(wl: W.Prefill, out):
    o, lse, s = out
    tol = tol_for(wl.dtype)
    ro, rl, rs = oracle.fwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, **oracle_kwargs(wl))
    assert_out(host(o), ro, tol)
    assert_lse(host(lse), rl, tol["lse"])
    if s is not None:
        err = float(np.max(np.abs(host(s) - rs))) if rs.size else 0.0
        assert err <= tol["s"], f"s: max abs err {err:.3e}"
    return ro, rl, rs



def check_bwd_full(wl: W.Prefill, max_seqlen=None):
    """Forward, then backward, against the oracle: dQ, dK, dV to the gradient
    bound, dsink max-normalised and head by head (with the floor that the
    output type's rounding of O allows)."""
    args = prefill_args(wl)
    o, lse, s = run_fwd(wl, args, max_seqlen)
    dq, dk, dv, dsink = run_bwd(wl, o, lse, args, max_seqlen)
    kw = oracle_kwargs(wl)
    rdq, rdk, rdv, rds = oracle.bwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale,
                                    wl.do.f32, **kw)
    tol = tol_for(wl.dtype)
    assert_grad(host(dq), rdq, tol, "dQ")
    assert_grad(host(dk), rdk, tol, "dK")
    assert_grad(host(dv), rdv, tol, "dV")
    if wl.sink is not None:
        ro, rl, _ = oracle.fwd(wl.q.f32, wl.k.f32, wl.v.f32, wl.cu_seqlens, wl.scale, **kw)
        assert_dsink(host(dsink), rds, tol)
        floor = dsink_storage_floor(ro, wl.do.f32, rl, wl.sink, wl.dtype)
        assert_dsink_per_head(host(dsink), rds, tol, floor)
    else:
        assert dsink is None
