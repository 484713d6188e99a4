"""Helpers for the GPU parity tests: move storage arrays to and from the
device, run the library through its C ABI binding, and compare against the
fp64 reference with the rules in tolerance.py."""

from __future__ import annotations

import numpy as np
import torch

import oracle
import transformer_normalization_rmsnorm_amd as rn
from rmsnorm_inputs import BF16, F16, bf16_bits_to_f32
from tolerance import (DGAMMA_TOL, FLOOR_BUDGET, FLOOR_FACTOR, LN_FLOOR_BUDGET, SMALL_ROW,
                       budget_for, cancel_scale, check_bf16, check_f16, check_f32,
                       dgamma_error, floor_within_budget, log_report)

# Marker for checks whose rows are built to cancel (degenerate rows): the
# floor's use is reported but not bounded.
UNBOUNDED = None

DEV = "cuda:0"
TORCH_DTYPE = {BF16: torch.bfloat16, F16: torch.float16, "f32": torch.float32}
CODE = {BF16: rn.BF16, F16: rn.F16, "f32": rn.F32}  # the C ABI's dtype codes


def in_f16(rows):
    """The bf16 rows of a case list again with binary16 storage (the kernels
    for the two 16-bit types are the same templates with their own
    conversions, so every 16-bit layout is run in both)."""
    return [tuple(F16 if v == BF16 else v for v in r) for r in rows if BF16 in r]


def to_dev(a: np.ndarray, dtype: str, device=DEV) -> torch.Tensor:
    if dtype == BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == F16:
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()  # float32, or float16 as numpy float16


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    return (bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a)).astype(np.float64)


def check_values(what, got, ref64, dtype, scale=None, budget=FLOOR_BUDGET):
    """got against ref64 by the storage type's rule.  scale: the cancellation
    scale s (None: no floor); the fp32 rule applies F32_FLOOR to it.  budget:
    the largest fraction of elements the floor may decide, per storage type
    (a dict) or one number (UNBOUNDED: report only); rows of at most
    SMALL_ROW elements are not bounded."""
    check = {BF16: check_bf16, F16: check_f16}.get(dtype, check_f32)
    sc = None if scale is None else np.asarray(scale, dtype=np.float64) * FLOOR_FACTOR[dtype]
    ref_arr = np.asarray(ref64)
    N = ref_arr.shape[-1] if ref_arr.ndim >= 1 and ref_arr.size else 0
    b = None if scale is None else budget_for(budget, dtype, N if ref_arr.ndim == 2 else SMALL_ROW + 1)
    r = check(what, got, ref64, scale=sc)
    log_report(r, dtype, b)
    assert r.ok, str(r)
    assert floor_within_budget(r, b), f"floor decides too many elements ({b}): {r}"
    return r


def check_stat(what, got, ref64, scale=None, budget=FLOOR_BUDGET):
    """A float32 statistic (rstd, mean) by the float32 rule; scale as check_values."""
    return check_values(what, got, ref64, "f32", scale=scale, budget=budget)


def check_forward(inp, dtype, eps, offset, y, rstd, h=None, rows=None):
    """Compare GPU forward outputs (numpy, possibly a row sample) with the reference.
    inp["gamma"] None: the non-affine op."""
    x = inp["x"] if rows is None else inp["x"][rows]
    g = inp["gamma"]
    if h is not None:
        r = inp["residual"] if rows is None else inp["residual"][rows]
        h_ref, y64, rstd64 = oracle.fused_add_fwd(x, r, g, dtype, eps, offset)
        assert np.array_equal(h, h_ref), f"h differs at {np.argwhere(h != h_ref)[:5].tolist()}"
    else:
        y64, rstd64 = oracle.fwd(x, g, dtype, eps, offset)
    reports = []
    if y is not None:
        reports.append(check_values("y", y, y64, dtype))
    if rstd is not None:
        reports.append(check_stat("rstd", rstd, rstd64))
    return reports


def reference_h(inp, dtype, eps=1e-6, offset=0.0):
    """h = round(x + residual) from the reference (the backward input of fused-add)."""
    h, _, _ = oracle.fused_add_fwd(inp["x"], inp["residual"], inp["gamma"], dtype, eps, offset, want_y=False)
    return h


def check_backward(inp, dtype, eps, offset, dx, dgamma, *, v_full, dh_full=None, rows=None, budget=FLOOR_BUDGET):
    """Compare GPU backward outputs with the reference.

    v_full: the forward input from the reference side: x, or reference_h() for
    fused-add (never an output of the GPU path), all rows.
    dx: GPU dx for `rows` (all rows if None); dgamma: GPU dgamma (always all rows)."""
    g = inp["gamma"]
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    v = sel(v_full)
    dy = sel(inp["dy"])
    dh = None if dh_full is None else sel(dh_full)
    out = oracle.bwd(dy, v, g, dtype, eps, offset, dh=dh, want_dgamma=rows is None and dgamma is not None)
    rstd64 = 1.0 / np.sqrt(np.mean(widen(v, dtype) ** 2, axis=1) + float(np.float32(eps)))
    g_wide = np.ones(v.shape[1]) if g is None else widen(g, dtype)
    s = cancel_scale(widen(v, dtype), g_wide, widen(dy, dtype), rstd64, out["c64"], out["sabs64"], offset,
                     None if dh is None else widen(dh, dtype))
    reports = [check_values("dx", dx, out["dx64"], dtype, scale=s, budget=budget)]
    if g is None:
        assert dgamma is None
    elif dgamma is not None:
        dg64 = out["dgamma64"] if rows is None else oracle.bwd(inp["dy"], v_full, g, dtype, eps, offset,
                                                               want_dx=False)["dgamma64"]
        err = dgamma_error(dgamma, dg64, dtype)
        assert err <= DGAMMA_TOL[dtype], f"dgamma relative L2 {err:.3g} > {DGAMMA_TOL[dtype]}"
    return reports


def gpu_forward(inp, dtype, eps, offset, fused):
    x = to_dev(inp["x"], dtype)
    g = None if inp["gamma"] is None else to_dev(inp["gamma"], dtype)
    if fused:
        r = to_dev(inp["residual"], dtype)
        y, h, rstd = rn.rmsnorm_fused_add_fwd(x, r, g, eps, offset)
        return {"y": y, "h": h, "rstd": rstd, "x": x, "gamma": g}
    y, rstd = rn.rmsnorm_fwd(x, g, eps, offset)
    return {"y": y, "rstd": rstd, "x": x, "gamma": g}


def gpu_backward(inp, dtype, eps, offset, fwd_out, fused, rstd="gpu"):
    dy = to_dev(inp["dy"], dtype)
    rs = fwd_out["rstd"] if rstd == "gpu" else (None if rstd is None else rstd)
    dx_out, dg_out = None, None
    if fused:
        dh = to_dev(inp["dh"], dtype)
        dx, dg = rn.rmsnorm_fused_add_bwd(dy, dh, fwd_out["h"], fwd_out["gamma"], rs, eps, offset)
    else:
        dx, dg = rn.rmsnorm_bwd(dy, fwd_out["x"], fwd_out["gamma"], rs, eps, offset)
    return dx, dg


def from_dev_opt(t):
    return None if t is None else from_dev(t)


def gpu_ln(inp, dt, eps, offset, fused, stats="gpu", affine=True, bias=True):
    """LayerNorm forward then backward through the binding; numpy results.
    stats=None makes the backward recompute mean and rstd."""
    x = to_dev(inp["x"], dt)
    g = to_dev(inp["gamma"], dt) if affine else None
    b = to_dev(inp["beta"], dt) if bias else None
    out = {}
    if fused:
        r = to_dev(inp["residual"], dt)
        y, h, mean, rstd = rn.layernorm_fused_add_fwd(x, r, g, b, eps, offset)
        out["h"] = h
    else:
        y, mean, rstd = rn.layernorm_fwd(x, g, b, eps, offset)
    out.update(y=y, mean=mean, rstd=rstd)
    dy = to_dev(inp["dy"], dt)
    m_in, r_in = (mean, rstd) if stats == "gpu" else (None, None)
    if fused:
        dx, dg, db = rn.layernorm_fused_add_bwd(dy, to_dev(inp["dh"], dt), out["h"], g, m_in, r_in, eps, offset)
    else:
        dx, dg, db = rn.layernorm_bwd(dy, x, g, m_in, r_in, eps, offset)
    torch.cuda.synchronize()
    out.update(dx=dx, dg=dg, db=db)
    return {k: (None if v is None else from_dev(v)) for k, v in out.items()}


def check_ln(inp, dt, eps, offset, fused, got, affine=True, bias=True, grads=True, budget=LN_FLOOR_BUDGET):
    """Compare LayerNorm results with the reference.

    Rules as for RMSNorm: bf16 within 2 ulp of the rounded reference, float32
    within a relative 1e-5, each at a magnitude floored by the size of the
    terms that cancel:
      y   s = rstd |w| (|v| + mean_j |v|) + |beta|
      dx  s = rstd (|g| + mean_j |g| + |xhat| (|mean_j(g xhat)| + mean_j |g xhat|)) [+ |dh|]
    mean is a float32 result floored at mean_j |v|; dgamma and dbeta (checked
    when grads is true, i.e. when inp holds every row) have the relative-L2
    rule; h (fused add) is bit-exact."""
    g = inp["gamma"] if affine else None
    beta = inp["beta"] if bias else None
    v = inp["x"]
    if fused:
        v, _, _ = oracle.fused_add_fwd(inp["x"], inp["residual"], g, dt, eps, offset, want_y=False)
        assert np.array_equal(got["h"], v), "h differs"
    y64, mean64, rstd64 = oracle.ln_fwd(v, g, beta, dt, eps, offset)
    vw = widen(v, dt)
    w = (widen(g, dt) if g is not None else np.ones(vw.shape[1])) + float(np.float32(offset))
    bw = widen(beta, dt) if beta is not None else np.zeros(vw.shape[1])
    mabs = np.abs(vw).mean(1)
    s_y = rstd64[:, None] * np.abs(w) * (np.abs(vw) + mabs[:, None]) + np.abs(bw)
    check_values("ln y", got["y"], y64, dt, scale=s_y, budget=budget)
    check_stat("ln rstd", got["rstd"], rstd64)
    check_stat("ln mean", got["mean"], mean64, scale=mabs, budget=budget)
    dh = inp["dh"] if fused else None
    out = oracle.ln_bwd(inp["dy"], v, g, dt, eps, offset, dh=dh, want_dgamma=grads, want_dbeta=grads)
    st = out["stats64"]
    gg = widen(inp["dy"], dt) * w
    xhat = (vw - mean64[:, None]) * rstd64[:, None]
    s_dx = rstd64[:, None] * (np.abs(gg) + st[:, 2:3] + np.abs(xhat) * (np.abs(st[:, 1:2]) + st[:, 3:4]))
    if dh is not None:
        s_dx = s_dx + np.abs(widen(dh, dt))
    r_dx = check_values("ln dx", got["dx"], out["dx64"], dt, scale=s_dx, budget=budget)
    if not grads:
        return r_dx
    if affine:
        err = dgamma_error(got["dg"], out["dgamma64"], dt)
        assert err <= DGAMMA_TOL[dt], f"dgamma relative L2 {err:.3g}"
    else:
        assert got["dg"] is None
    err = dgamma_error(got["db"], out["dbeta64"], dt)
    assert err <= DGAMMA_TOL[dt], f"dbeta relative L2 {err:.3g}"
    return r_dx
