"""GPU parity at the size limits.

  * The longest row the library accepts (N = 2^24 elements, and 2^24 - 1 on
    the per-element path), against the fp64 reference on every element.
  * Tensors of more than 2^31 elements (bf16 66560 x 32768, 4.4 GB each), so
    that element offsets, byte offsets of the fp8 output and the partial rows
    all pass 2^31.  The rows are a seeded draw of 1024 rows repeated 65 times
    (built on the device), so each output row equals the reference for its
    source row and dgamma / dbeta equal 65 times the reference over the 1024
    rows.  Rows are compared on a sample that includes the rows on both sides
    of element 2^31 and the last rows.
  * A statistics-only forward over 8.4 million rows: more workgroups than one
    launch can hold, so the capped grid strides over the rows."""

import numpy as np
import pytest
import torch

import oracle
import transformer_normalization_rmsnorm_amd as rn
from gpu_util import (check_backward, check_forward, check_ln, from_dev,
                      gpu_backward, gpu_forward, gpu_ln, reference_h, to_dev)
from rmsnorm_inputs import make_inputs
from tolerance import DGAMMA_TOL, dgamma_error

pytestmark = pytest.mark.gpu

EPS = 1e-6
LN_EPS = 1e-5

LONG_ROW_BUDGET = {"bf16": 1e-3, "f16": 1e-3, "f32": 4e-2}

LONG = [
    (3, rn.MAX_N, "bf16", False),
    (2, rn.MAX_N, "f32", True),
    (2, rn.MAX_N - 1, "f32", False),  # odd: per-element access
]


@pytest.mark.parametrize("M,N,dt,fused", LONG, ids=[f"{d}_{m}x{n}" + ("_fused" if f else "") for m, n, d, f in LONG])
def test_longest_rows(M, N, dt, fused):
    print(f"rmsnorm {dt} {M}x{N} fused={fused}", flush=True)
    inp = make_inputs(M, N, dt, fused=fused)
    out = gpu_forward(inp, dt, EPS, 0.0, fused)
    torch.cuda.synchronize()
    check_forward(inp, dt, EPS, 0.0, from_dev(out["y"]), from_dev(out["rstd"]),
                  from_dev(out["h"]) if fused else None)
    dx, dg = gpu_backward(inp, dt, EPS, 0.0, out, fused)
    torch.cuda.synchronize()
    v = reference_h(inp, dt, EPS, 0.0) if fused else inp["x"]
    # the row dot sums 2^24 float32 terms, so c carries a larger float32 error
    # and more elements need the floor (1.3% measured for fused float32)
    check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg), v_full=v, dh_full=inp["dh"] if fused else None,
                   budget=LONG_ROW_BUDGET)
    del out, dx, dg
    print(f"layernorm {dt} {M}x{N} fused={fused}", flush=True)
    inp = make_inputs(M, N, dt, fused=fused, layernorm=True)
    check_ln(inp, dt, LN_EPS, 0.0, fused, gpu_ln(inp, dt, LN_EPS, 0.0, fused))
    torch.cuda.empty_cache()


BASE_ROWS, REPEATS, WIDE = 1024, 65, 32768
BIG_M = BASE_ROWS * REPEATS  # 66560 rows: 2,181,038,080 elements per tensor


def big_rows():
    edge = (2 ** 31) // WIDE  # the row holding element 2^31
    rows = [0, 1, BASE_ROWS - 1, BASE_ROWS, edge - 2, edge - 1, edge, edge + 1, BIG_M - 2, BIG_M - 1]
    rng = np.random.default_rng(5)
    rows += list(rng.choice(BIG_M, 22, replace=False))
    return np.unique(np.array(rows, dtype=np.int64))


def tiled(a, dt):
    """The [BASE_ROWS, N] storage array repeated to BIG_M rows on the device."""
    return to_dev(a, dt).repeat(REPEATS, 1)


def sampled(t, rows):
    return from_dev(t[torch.from_numpy(rows).to(t.device)])


def base_view(inp, rows):
    """The reference inputs for the sampled rows (each row's source row)."""
    src = rows % BASE_ROWS
    return {k: (v[src] if v.ndim == 2 else v) for k, v in inp.items()}


@pytest.mark.parametrize("fused", [False, True], ids=["plain", "fused"])
def test_rmsnorm_beyond_2_31_elements(fused):
    dt = "bf16"
    print(f"rmsnorm {dt} {BIG_M}x{WIDE} fused={fused}", flush=True)
    inp = make_inputs(BASE_ROWS, WIDE, dt, fused=fused)
    rows = big_rows()
    x, g = tiled(inp["x"], dt), to_dev(inp["gamma"], dt)
    assert x.numel() > 2 ** 31
    if fused:
        r = tiled(inp["residual"], dt)
        y, h, rstd = rn.rmsnorm_fused_add_fwd(x, r, g, EPS, 0.0)
        del r, x
        v = h
    else:
        y, rstd = rn.rmsnorm_fwd(x, g, EPS, 0.0)
        v = x
    torch.cuda.synchronize()
    sub = base_view(inp, rows)
    check_forward(sub, dt, EPS, 0.0, sampled(y, rows), sampled(rstd, rows), sampled(h, rows) if fused else None)
    del y
    dy = tiled(inp["dy"], dt)
    if fused:
        dh = tiled(inp["dh"], dt)
        dx, dg = rn.rmsnorm_fused_add_bwd(dy, dh, v, g, rstd, EPS, 0.0)
    else:
        dx, dg = rn.rmsnorm_bwd(dy, v, g, rstd, EPS, 0.0)
    torch.cuda.synchronize()
    v_base = reference_h(inp, dt, EPS, 0.0) if fused else inp["x"]
    check_backward(sub, dt, EPS, 0.0, sampled(dx, rows), None, v_full=v_base[rows % BASE_ROWS],
                   dh_full=sub["dh"] if fused else None)
    ref = oracle.bwd(inp["dy"], v_base, inp["gamma"], dt, EPS, 0.0, dh=inp["dh"] if fused else None,
                     want_dx=False)
    err = dgamma_error(from_dev(dg), REPEATS * ref["dgamma64"], dt)
    assert err <= DGAMMA_TOL[dt], f"dgamma relative L2 {err:.3g}"
    del dx, dy, v
    torch.cuda.empty_cache()


def test_layernorm_beyond_2_31_elements():
    dt = "bf16"
    print(f"layernorm {dt} {BIG_M}x{WIDE}", flush=True)
    inp = make_inputs(BASE_ROWS, WIDE, dt, layernorm=True)
    rows = big_rows()
    x, g, b = tiled(inp["x"], dt), to_dev(inp["gamma"], dt), to_dev(inp["beta"], dt)
    y, mean, rstd = rn.layernorm_fwd(x, g, b, LN_EPS, 0.0)
    torch.cuda.synchronize()
    got = {"y": sampled(y, rows), "mean": sampled(mean, rows), "rstd": sampled(rstd, rows)}
    del y
    dy = tiled(inp["dy"], dt)
    dx, dg, db = rn.layernorm_bwd(dy, x, g, mean, rstd, LN_EPS, 0.0)
    torch.cuda.synchronize()
    got["dx"] = sampled(dx, rows)
    check_ln(base_view(inp, rows), dt, LN_EPS, 0.0, False, got, grads=False)
    ref = oracle.ln_bwd(inp["dy"], inp["x"], inp["gamma"], dt, LN_EPS, 0.0, want_dx=False)
    for name, t, r in (("dgamma", dg, ref["dgamma64"]), ("dbeta", db, ref["dbeta64"])):
        err = dgamma_error(from_dev(t), REPEATS * r, dt)
        assert err <= DGAMMA_TOL[dt], f"{name} relative L2 {err:.3g}"
    del x, dy, dx
    torch.cuda.empty_cache()


def test_fp8_beyond_2_31_elements():
    dt = "bf16"
    print(f"fp8 forward {dt} {BIG_M}x{WIDE}", flush=True)
    inp = make_inputs(BASE_ROWS, WIDE, dt)
    rows = big_rows()
    x, g = tiled(inp["x"], dt), to_dev(inp["gamma"], dt)
    scale = 16.0
    sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    y8, rstd = rn.rmsnorm_fwd_fp8(x, g, sc, EPS, 0.0, amax=am)
    torch.cuda.synchronize()
    code = y8.view(torch.uint8)[torch.from_numpy(rows).cuda()].cpu().numpy()
    ref = oracle.fwd_fp8(inp["x"][rows % BASE_ROWS], inp["gamma"], dt, EPS, 0.0, scale, tol=1e-5)
    ok = (code == ref["code_lo"]) | (code == ref["code_hi"])
    assert ok.all(), f"{int((~ok).sum())} codes outside the tolerance interval"
    full = oracle.fwd_fp8(inp["x"], inp["gamma"], dt, EPS, 0.0, scale)
    assert abs(float(am.item()) - full["amax64"]) <= 1e-5 * full["amax64"]
    del x, y8
    torch.cuda.empty_cache()


def test_statistics_only_forward_beyond_one_launch():
    """rstd (and LayerNorm's mean) without y for more rows than one launch of
    one 256-thread workgroup per row can address (2^31 work-items): the grid is
    capped and the workgroups stride over the rows."""
    base, reps, N, dt = 4096, 2051, 16, "bf16"
    M = base * reps  # 8,400,896 rows
    assert M * 256 > 2 ** 31
    print(f"statistics-only forward {dt} {M}x{N}", flush=True)
    lib = rn.load_library()
    inp = make_inputs(base, N, dt, layernorm=True)
    x = to_dev(inp["x"], dt).repeat(reps, 1)
    rows = np.unique(np.concatenate([[0, base - 1, M - 2, M - 1, M // 2],
                                     np.random.default_rng(3).choice(M, 27, replace=False)])).astype(np.int64)
    idx = torch.from_numpy(rows).cuda()
    src = inp["x"][rows % base]
    stream = torch.cuda.current_stream().cuda_stream
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    assert lib.rmsnorm_fwd(x.data_ptr(), None, None, rstd.data_ptr(), M, N, EPS, 0.0, rn.BF16, stream) == 0
    mean = torch.empty(M, dtype=torch.float32, device="cuda")
    lrstd = torch.empty(M, dtype=torch.float32, device="cuda")
    assert lib.layernorm_fwd(x.data_ptr(), None, None, None, mean.data_ptr(), lrstd.data_ptr(), M, N, LN_EPS, 0.0,
                             rn.BF16, stream) == 0
    torch.cuda.synchronize()
    from gpu_util import check_stat, widen
    _, rstd64 = oracle.fwd(src, None, dt, EPS, 0.0, want_y=False)
    check_stat("rstd", rstd[idx].cpu().numpy(), rstd64)
    _, mean64, lrstd64 = oracle.ln_fwd(src, None, None, dt, LN_EPS, 0.0, want_y=False)
    check_stat("layernorm rstd", lrstd[idx].cpu().numpy(), lrstd64)
    check_stat("mean", mean[idx].cpu().numpy(), mean64, scale=np.abs(widen(src, dt)).mean(1))
