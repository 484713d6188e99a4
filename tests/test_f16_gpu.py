"""binary16 storage on the GPU beyond the shared case lists (which run every
16-bit layout in both 16-bit types): results outside the binary16 normal
range, the full-size workload shapes, and zero rows.

  * Overflow: gamma large enough that some |y| exceed 65504.  The reference
    rounds those to infinity (nearest even, as the IEEE conversion does), and
    so must the kernel; every other element keeps the usual rule.
  * Subnormal outputs: gamma small enough that y lies mostly below 2^-14,
    where binary16 spacing is fixed at 2^-24; the kernel's conversion must not
    flush them.
  * Full size: the 16384 x 7168 fused residual add in binary16, forward
    outputs and dx on a row sample, dgamma in full (the 4096 x 4096 layer in
    binary16 is one of the benchmark workloads, tested with them)."""

import numpy as np
import pytest
import torch

import oracle
import transformer_normalization_rmsnorm_amd as rn
from gpu_util import (check_backward, check_forward, from_dev, gpu_backward, gpu_forward, reference_h,
                      to_dev)
from rmsnorm_inputs import EPS, F16, make_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _run(inp, fused, offset=0.0, check_dx=True):
    out = gpu_forward(inp, F16, EPS, offset, fused)
    torch.cuda.synchronize()
    y = from_dev(out["y"])
    check_forward(inp, F16, EPS, offset, y, from_dev(out["rstd"]), from_dev(out["h"]) if fused else None)
    if check_dx:
        dx, dg = gpu_backward(inp, F16, EPS, offset, out, fused)
        torch.cuda.synchronize()
        check_backward(inp, F16, EPS, offset, from_dev(dx), from_dev(dg),
                       v_full=reference_h(inp, F16, EPS, offset) if fused else inp["x"],
                       dh_full=inp["dh"] if fused else None)
    return y


@pytest.mark.parametrize("M,N,fused", [(64, 4096, False), (40, 7168, True), (9, 4097, False), (3, 40960, False)])
def test_outputs_beyond_the_largest_finite_value_become_infinite(M, N, fused):
    print(f"f16 overflow {M}x{N} fused={fused}", flush=True)
    inp = make_inputs(M, N, F16, fused=fused)
    inp["gamma"] = (np.abs(inp["gamma"].astype(np.float32)) * np.float32(30000.0)).astype(np.float16)
    y = _run(inp, fused, check_dx=False)
    n_inf = int(np.isinf(y).sum())
    assert n_inf > 0, "no output overflowed: the case does not exercise the overflow"
    assert n_inf < y.size // 2


@pytest.mark.parametrize("M,N,fused", [(64, 4096, False), (40, 7168, True), (1000, 128, False), (9, 4097, True)])
def test_subnormal_outputs_are_kept(M, N, fused):
    print(f"f16 subnormal {M}x{N} fused={fused}", flush=True)
    inp = make_inputs(M, N, F16, fused=fused)
    inp["gamma"] = (inp["gamma"].astype(np.float32) * np.float32(1e-5)).astype(np.float16)
    y = _run(inp, fused)
    a = np.abs(y.astype(np.float64))
    assert np.count_nonzero((a > 0) & (a < 2.0 ** -14)) > y.size // 4


@pytest.mark.parametrize("M,N,fused", [(16384, 7168, True)])  # 4096 x 4096 runs with the workloads
def test_full_size(M, N, fused):
    print(f"f16 full size {M}x{N} fused={fused}", flush=True)
    inp = make_inputs(M, N, F16, fused=fused)
    rows = sample_rows(M, 48)
    out = gpu_forward(inp, F16, EPS, 0.0, fused)
    dx, dg = gpu_backward(inp, F16, EPS, 0.0, out, fused)
    torch.cuda.synchronize()
    sel = torch.from_numpy(rows).cuda()
    h = from_dev(out["h"].index_select(0, sel)) if fused else None
    check_forward(inp, F16, EPS, 0.0, from_dev(out["y"].index_select(0, sel)),
                  from_dev(out["rstd"].index_select(0, sel)), h, rows=rows)
    check_backward(inp, F16, EPS, 0.0, from_dev(dx.index_select(0, sel)), from_dev(dg),
                   v_full=reference_h(inp, F16) if fused else inp["x"], dh_full=inp["dh"] if fused else None,
                   rows=rows)
    assert bool(torch.isfinite(out["y"]).all()) and bool(torch.isfinite(dx).all())


def test_zero_rows_write_zero_gradients():
    x = torch.empty(0, 4096, dtype=torch.float16, device="cuda")
    g = torch.ones(4096, dtype=torch.float16, device="cuda")
    y, rstd = rn.rmsnorm_fwd(x, g)
    dg = torch.full((4096,), float("nan"), dtype=torch.float16, device="cuda")
    _, dg = rn.rmsnorm_bwd(torch.empty_like(x), x, g, rstd, dgamma=dg)
    b = torch.zeros_like(g)
    _, mean, lrstd = rn.layernorm_fwd(x, g, b)
    _, lg, lb = rn.layernorm_bwd(torch.empty_like(x), x, g, mean, lrstd)
    torch.cuda.synchronize()
    assert torch.all(dg == 0) and torch.all(lg == 0) and torch.all(lb == 0)


def test_f16_and_bf16_share_plans_and_differ_in_rounding():
    """The same draw through both 16-bit types: identical plans; binary16 results
    are closer to the fp64 reference than bf16 results (3 more fraction bits)."""
    M, N = 200, 4096
    f = make_inputs(M, N, F16)
    assert rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.F16) == rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.BF16)
    out = gpu_forward(f, F16, EPS, 0.0, False)
    torch.cuda.synchronize()
    y64, _ = oracle.fwd(f["x"], f["gamma"], F16, EPS, 0.0)
    err16 = np.abs(from_dev(out["y"]).astype(np.float64) - y64).max()
    xb = to_dev(f["x"].astype(np.float32), "f32").to(torch.bfloat16)
    gb = to_dev(f["gamma"].astype(np.float32), "f32").to(torch.bfloat16)
    yb, _ = rn.rmsnorm_fwd(xb, gb, EPS)
    errb = (yb.float().cpu().double().numpy() - y64).__abs__().max()
    assert err16 < errb / 4, (err16, errb)
