"""Every compiled workgroup tiling of the fp8-output and LayerNorm forwards
against the fp64 reference.

The forward layouts of these two ops are chosen from measured tables that
can pick any exact tiling (threads = row vectors / chunks per lane, a
multiple of 64 within the launch bound), so each one is forced here on rows
of the widths the tables cover, plain and fused-add."""

import numpy as np
import pytest

import transformer_normalization_rmsnorm_amd as rn
from gpu_util import check_ln, gpu_ln
from rmsnorm_inputs import EPS, make_inputs
from test_fp8_gpu import TOL, check_codes, reference, run_fp8
from tolerance import check_f32

pytestmark = pytest.mark.gpu

CODE = {"bf16": rn.BF16, "f32": rn.F32, "f16": rn.F16}
WIDTHS = [("bf16", 2048), ("bf16", 6144), ("bf16", 12288), ("bf16", 32768), ("f32", 2048), ("f32", 6144),
          ("f16", 4096)]


def tilings(op, N, dt):
    """(threads, chunks) of every exact workgroup tiling the library plans for op at this width."""
    V = 8 if dt != "f32" else 4
    out = []
    for k in (1, 2, 3, 4, 6, 8, 16):
        if (N // V) % k:
            continue
        t = N // V // k
        if t % 64 or not 64 <= t <= 1024:
            continue
        try:
            with rn.plan_override(op, path=rn.PATH_ROWS, vec=V, team=0, threads=t, depth=0):
                p = rn.rmsnorm_query_plan(op, 37, N, CODE[dt], True, 256)  # no device needed
        except rn.RMSNormError:
            continue  # not compiled at this size
        if (p["threads"], p["chunks"]) == (t, k):
            out.append((t, k))
    return out


CASES = [(dt, N, fused, t, k) for dt, N in WIDTHS for fused in (False, True)
         for t, k in tilings(rn.OP_FUSED_ADD_FWD_FP8 if fused else rn.OP_FWD_FP8, N, dt)]
LN_CASES = [(dt, N, fused, t, k) for dt, N in WIDTHS for fused in (False, True)
            for t, k in tilings(rn.OP_LN_FUSED_ADD_FWD if fused else rn.OP_LN_FWD, N, dt)]


def ident(c):
    dt, N, fused, t, k = c
    return f"{dt}_{N}{'_fused' if fused else ''}_{t}x{k}"


def test_every_width_has_several_tilings():
    for dt, N in WIDTHS:
        assert len([c for c in CASES if c[:2] == (dt, N)]) >= 2, (dt, N)
        assert len([c for c in LN_CASES if c[:2] == (dt, N)]) >= 2, (dt, N)


@pytest.mark.parametrize("case", CASES, ids=ident)
def test_fp8_forward_tiling(case):
    dt, N, fused, t, k = case
    M, scale = 37, 32.0
    V = 8 if dt != "f32" else 4
    op = rn.OP_FUSED_ADD_FWD_FP8 if fused else rn.OP_FWD_FP8
    inp = make_inputs(M, N, dt, fused=fused)
    with rn.plan_override(op, path=rn.PATH_ROWS, vec=V, team=0, threads=t, depth=0):
        assert (rn.rmsnorm_query_plan(op, M, N, CODE[dt])["chunks"]) == k
        code, rstd, amax, h = run_fp8(inp, dt, 0.0, fused, scale)
    v, ref = reference(inp, dt, 0.0, fused, scale)
    if fused:
        assert np.array_equal(h, v), "h differs"
    check_codes(code, ref)
    rr = check_f32("rstd", rstd, ref["rstd64"])
    assert rr.ok, str(rr)
    assert abs(amax - ref["amax64"]) <= TOL * ref["amax64"], (amax, ref["amax64"])


@pytest.mark.parametrize("case", LN_CASES, ids=ident)
def test_layernorm_forward_tiling(case):
    dt, N, fused, t, k = case
    M = 37
    V = 8 if dt != "f32" else 4
    op = rn.OP_LN_FUSED_ADD_FWD if fused else rn.OP_LN_FWD
    inp = make_inputs(M, N, dt, fused=fused, layernorm=True)
    with rn.plan_override(op, path=rn.PATH_ROWS, vec=V, team=0, threads=t, depth=0):
        assert (rn.rmsnorm_query_plan(op, M, N, CODE[dt])["chunks"]) == k
        got = gpu_ln(inp, dt, EPS, 0.0, fused)
    r = check_ln(inp, dt, EPS, 0.0, fused, got)
    print(f"{ident(case)}: {r}")
