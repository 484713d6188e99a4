"""GPU parity: the HIP path through the C ABI against the fp64 reference.

Sizes span several workgroup tiles with ragged tails; every selector path
(narrow-row teams, one wavefront per row, workgroup teams, scalar access,
looped rows) is exercised, plus the edge cases (N = 1, odd N, unaligned
storage offsets, M smaller than the grid, M = 0)."""

import numpy as np
import pytest
import torch

import oracle
import transformer_normalization_rmsnorm_amd as rn
from gpu_util import (CODE, check_backward, check_forward, check_ln, from_dev, from_dev_opt,
                      gpu_backward, gpu_forward, in_f16, reference_h, to_dev)
from rmsnorm_inputs import EPS, make_inputs

pytestmark = pytest.mark.gpu

LN_EPS = 1e-5

# (M, N, dtype, fused, gemma)
CASES = [
    (300, 4096, "bf16", False, False),    # wavefront rows fwd, 512-thread bwd, ragged vs the grid
    (257, 8192, "bf16", False, False),    # wide rows
    (130, 6144, "f32", False, True),      # float32, gamma + offset
    (200, 7168, "bf16", True, False),     # fused residual add, 896-thread bwd
    (1000, 128, "bf16", False, False),    # narrow rows: 16-lane teams
    (1000, 128, "bf16", True, False),
    (37, 64, "f32", False, False),        # 16-lane teams of float32
    (64, 2048, "bf16", False, False),
    (33, 5000, "bf16", False, False),     # vector path with a ragged last vector group
    (17, 4097, "bf16", False, False),     # N % 8 != 0: scalar access
    (9, 8200, "bf16", True, False),
    (5, 1, "bf16", False, False),         # N = 1
    (7, 7, "f32", False, True),
    (11, 127, "bf16", True, False),
    (6, 20000, "bf16", False, False),     # wide rows, gamma re-read per row, masked lanes
    (70, 16384, "bf16", False, False),    # wide rows, two chunks per lane, one row ahead
    (45, 16384, "bf16", True, False),
    (9, 32768, "bf16", False, False),     # four chunks per lane x 1024 lanes
    (9, 32768, "bf16", True, True),       # fused: eight chunks x 512 lanes, with offset
    (20, 8192, "f32", False, True),
    (5, 12000, "f32", True, False),
    (7, 16384, "f32", True, False),
    (4, 40000, "f32", True, True),        # beyond the register path: looped rows
    (3, 40960, "bf16", False, False),
    (3, 4096, "bf16", False, False),      # fewer rows than programs
    (1, 3000, "f32", False, False),
]


def case_id(c):
    M, N, dt, fused, gemma = c
    return f"{dt}_{M}x{N}" + ("_fused" if fused else "") + ("_offset1" if gemma else "")


def run_case(M, N, dt, fused, gemma, seed=0):
    inp = make_inputs(M, N, dt, fused=fused, gemma=gemma, seed=seed)
    offset = 1.0 if gemma else 0.0
    out = gpu_forward(inp, dt, EPS, offset, fused)
    torch.cuda.synchronize()
    y, rstd = from_dev(out["y"]), from_dev(out["rstd"])
    h = from_dev(out["h"]) if fused else None
    check_forward(inp, dt, EPS, offset, y, rstd, h)
    v_ref = reference_h(inp, dt, EPS, offset) if fused else inp["x"]
    dx, dg = gpu_backward(inp, dt, EPS, offset, out, fused)
    torch.cuda.synchronize()
    check_backward(inp, dt, EPS, offset, from_dev(dx), from_dev(dg), v_full=v_ref,
                   dh_full=inp["dh"] if fused else None)
    return inp, out, dx, dg


@pytest.mark.parametrize("case", CASES + in_f16(CASES), ids=case_id)
def test_fwd_bwd_parity(case):
    run_case(*case)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3], CASES[4], CASES[9], CASES[14]], ids=case_id)
def test_bwd_recomputes_rstd(case):
    M, N, dt, fused, gemma = case
    inp = make_inputs(M, N, dt, fused=fused, gemma=gemma)
    offset = 1.0 if gemma else 0.0
    out = gpu_forward(inp, dt, EPS, offset, fused)
    dx, dg = gpu_backward(inp, dt, EPS, offset, out, fused, rstd=None)
    torch.cuda.synchronize()
    check_backward(inp, dt, EPS, offset, from_dev(dx), from_dev(dg),
                   v_full=reference_h(inp, dt, EPS, offset) if fused else inp["x"],
                   dh_full=inp["dh"] if fused else None)


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3]], ids=case_id)
def test_bwd_fed_reference_rstd(case):
    """Backward in isolation, fed the reference forward's float32 rstd."""
    M, N, dt, fused, gemma = case
    inp = make_inputs(M, N, dt, fused=fused, gemma=gemma)
    offset = 1.0 if gemma else 0.0
    if fused:
        h_ref, _, rstd64 = oracle.fused_add_fwd(inp["x"], inp["residual"], inp["gamma"], dt, EPS, offset, want_y=False)
        v = h_ref
    else:
        _, rstd64 = oracle.fwd(inp["x"], inp["gamma"], dt, EPS, offset, want_y=False)
        v = inp["x"]
    rs = torch.from_numpy(oracle.round_to(rstd64, "f32")).cuda()
    fwd_out = {"x": to_dev(v, dt), "h": to_dev(v, dt), "gamma": to_dev(inp["gamma"], dt)}
    dx, dg = gpu_backward(inp, dt, EPS, offset, fwd_out, fused, rstd=rs)
    torch.cuda.synchronize()
    check_backward(inp, dt, EPS, offset, from_dev(dx), from_dev(dg), v_full=v, dh_full=inp["dh"] if fused else None)


# Every compiled layout on one shape each: forced through the test override.
FORCED = [
    # (op-kind, M, N, dtype, plan fields)
    ("fwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=512)),
    ("fwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=256)),
    ("fwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=1, team=0, threads=512)),
    ("fwd", 300, 4096, "bf16", dict(path=rn.PATH_LOOP, vec=8, team=0, threads=256)),
    ("fwd", 300, 4096, "bf16", dict(path=rn.PATH_LOOP, vec=1, team=0, threads=1024)),
    ("fwd", 300, 512, "bf16", dict(path=rn.PATH_ROWS, vec=1, team=64, threads=256)),
    ("fwd", 100, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=64, threads=256)),
    ("fwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=256, depth=2, grid=100)),
    ("fwd", 300, 2048, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=128, depth=3, grid=37)),
    ("fwd", 100, 6144, "f32", dict(path=rn.PATH_ROWS, vec=4, team=0, threads=256)),
    ("fwd", 1000, 256, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=32, threads=256)),
    ("bwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=256)),
    ("bwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=1024, grid=7)),
    ("bwd", 300, 2048, "bf16", dict(path=rn.PATH_ROWS, vec=1, team=0, threads=512)),
    ("bwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=3, grid=61)),
    ("bwd", 300, 4096, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=2)),
    ("bwd", 300, 4096, "bf16", dict(path=rn.PATH_LOOP, vec=8, team=0, threads=512)),
    ("bwd", 300, 4096, "bf16", dict(path=rn.PATH_LOOP, vec=1, team=0, threads=1024, grid=300)),
    ("bwd", 300, 1024, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=64, threads=256)),
    ("bwd", 300, 128, "bf16", dict(path=rn.PATH_ROWS, vec=1, team=64, threads=256)),
    ("bwd", 1000, 128, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=16, threads=128)),
    ("bwd", 100, 6144, "f32", dict(path=rn.PATH_ROWS, vec=4, team=0, threads=512)),
    ("bwd", 300, 8192, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=2)),
    ("bwd", 1000, 128, "bf16", dict(path=rn.PATH_ROWS, vec=8, team=16, threads=256, depth=2, grid=5)),
]


@pytest.mark.parametrize("fused", [False, True], ids=["plain", "fused"])
@pytest.mark.parametrize("kind,M,N,dt,fields", FORCED + in_f16(FORCED),
                         ids=[f"{k}_{dt}_{M}x{N}_" + "_".join(f"{a}{b}" for a, b in f.items())
                              for k, M, N, dt, f in FORCED + in_f16(FORCED)])
def test_forced_layouts(kind, M, N, dt, fields, fused):
    if kind == "fwd":
        op = rn.OP_FUSED_ADD_FWD if fused else rn.OP_FWD
    else:
        op = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    with rn.plan_override(op, **fields):
        p = rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)
        for k, v in fields.items():
            assert p[k] == v, (k, p)
        run_case(M, N, dt, fused, dt == "f32")


# Backward layouts that re-read gamma with every row (w_regs = 0), each
# forced on a shape it tiles, with a small grid so that every program walks
# several rows (prefetch ring, clamped tail, dgamma accumulation across rows).
R = rn.PATH_ROWS
WIDE_FORCED = [
    # (fused ops too, M, N, dtype, plan fields)
    (True, 40, 16384, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=0, w_regs=0, grid=7)),
    (True, 40, 16000, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=1, w_regs=0, grid=6)),
    (True, 60, 8192, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=2, w_regs=0, grid=9)),
    # half the lanes with gamma re-read, one row ahead: the fused-add op's choice from 896 lanes and 8 rows
    # per program; and no row ahead at two rows per program
    (True, 60, 8192, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=0, grid=7)),
    (True, 60, 7168, "bf16", dict(path=R, vec=8, team=0, threads=448, depth=1, w_regs=0, grid=7)),
    (True, 60, 4096, "f32", dict(path=R, vec=4, team=0, threads=512, depth=1, w_regs=0, grid=7)),
    (True, 30, 6144, "f32", dict(path=R, vec=4, team=0, threads=768, depth=0, w_regs=0, grid=16)),
    (True, 60, 4096, "f32", dict(path=R, vec=4, team=0, threads=512, depth=2, w_regs=0, grid=13)),
    (True, 30, 24576, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=0, w_regs=0, grid=4)),
    (True, 30, 12000, "f32", dict(path=R, vec=4, team=0, threads=1024, depth=0, w_regs=0, grid=4)),
    (True, 30, 12288, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=0, grid=5)),
    (False, 20, 32768, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=0, w_regs=0, grid=3)),
    (False, 20, 16384, "f32", dict(path=R, vec=4, team=0, threads=1024, depth=0, w_regs=0, grid=3)),
    (True, 30, 16384, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=0, grid=4)),
    (True, 30, 8000, "f32", dict(path=R, vec=4, team=0, threads=512, depth=1, w_regs=0, grid=4)),
    (True, 20, 24576, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    (True, 20, 32768, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    (True, 20, 16384, "f32", dict(path=R, vec=4, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    # w held in registers, several rows per program
    (True, 60, 8192, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=2, w_regs=1, grid=9)),
]


# every layout plain, and fused-add where it is compiled for the fused op at that workgroup size
WIDE_CASES = [(M, N, dt, f, fused) for ok, M, N, dt, f in WIDE_FORCED + in_f16(WIDE_FORCED)
              for fused in ((False, True) if ok else (False,))]


@pytest.mark.parametrize("M,N,dt,fields,fused", WIDE_CASES,
                         ids=[f"{dt}_{M}x{N}_t{f['threads']}_d{f['depth']}_w{f['w_regs']}-" + ("fused" if fu else "plain")
                              for M, N, dt, f, fu in WIDE_CASES])
def test_wide_backward_layouts(M, N, dt, fields, fused):
    op = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    with rn.plan_override(op, **fields):
        p = rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)
        for k, v in fields.items():
            assert p[k] == v, (k, p)
        run_case(M, N, dt, fused, dt == "f32")


# Two rows per reduction (rows_per_step = 2), forced with grids that give odd
# and even row counts per program, one row per program (no second row
# anywhere) and a ragged last vector group.
PAIRS = [
    (300, 4096, "bf16", dict(threads=512, grid=19)),
    (257, 4096, "bf16", dict(threads=512, grid=128)),
    (256, 4096, "bf16", dict(threads=512, grid=256)),
    (100, 2048, "bf16", dict(threads=256, grid=7)),
    (64, 8192, "bf16", dict(threads=1024, grid=5)),
    (45, 5000, "bf16", dict(threads=640, grid=4)),
    (300, 4096, "f32", dict(threads=1024, grid=17)),
    (300, 1024, "f32", dict(threads=256, grid=19)),
]


# the fused-add op's two-row instance is compiled for at most 256 threads
PAIR_CASES = [(M, N, dt, f, False) for M, N, dt, f in PAIRS + in_f16(PAIRS)] + \
    [(M, N, dt, f, True) for M, N, dt, f in PAIRS + in_f16(PAIRS) if f["threads"] <= 256]


@pytest.mark.parametrize("M,N,dt,fields,fused", PAIR_CASES,
                         ids=[f"{dt}_{M}x{N}_t{f['threads']}_g{f['grid']}" + ("_fused" if fu else "")
                              for M, N, dt, f, fu in PAIR_CASES])
def test_two_rows_per_reduction(M, N, dt, fields, fused):
    vec = 4 if dt == "f32" else 8
    op = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    with rn.plan_override(op, path=rn.PATH_ROWS, vec=vec, team=0, depth=1, w_regs=1, rows_per_step=2, **fields):
        p = rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)
        assert (p["rows_per_step"], p["chunks"], p["grid"]) == (2, 1, fields["grid"]), p
        inp, out, dx, _ = run_case(M, N, dt, fused, dt == "f32")
        if fused:
            # dx written over dh (the residual gradient in place) gives the same bytes
            dh = to_dev(inp["dh"], dt)
            dx2, _ = rn.rmsnorm_fused_add_bwd(to_dev(inp["dy"], dt), dh, out["h"], out["gamma"], out["rstd"], EPS,
                                              1.0 if dt == "f32" else 0.0, dx=dh)
            torch.cuda.synchronize()
            assert dx2.data_ptr() == dh.data_ptr()
            assert np.array_equal(from_dev(dx2).view(np.uint8), from_dev(dx).view(np.uint8))
            return
        # non-affine
        inp = make_inputs(M, N, dt, seed=3)
        inp["gamma"] = None
        out = gpu_forward(inp, dt, EPS, 0.0, False)
        dx, dg = gpu_backward(inp, dt, EPS, 0.0, out, False)
        torch.cuda.synchronize()
        assert dg is None
        check_backward(inp, dt, EPS, 0.0, from_dev(dx), None, v_full=inp["x"])


# One-launch backward (PATH_ROWS_COLS): dgamma summed by column workgroups of
# the dx launch, no partial rows.  Forced at every slab width, with one row
# per program and several, a grid that is not a multiple of 8, a ragged row
# (masked lanes), two rows per reduction, plain and fused-add (dx also written
# over dh), rstd given and recomputed, and run to run.
COLS = [
    (512, 2048, "bf16", dict(threads=256, col_chunks=1)),
    (128, 8192, "bf16", dict(threads=1024, col_chunks=8)),
    (256, 4096, "bf16", dict(threads=512, col_chunks=2)),
    (300, 4096, "bf16", dict(threads=512, col_chunks=4, grid=37)),
    (3, 2048, "bf16", dict(threads=256, col_chunks=8)),
    (200, 2000, "bf16", dict(threads=256, col_chunks=2)),
    (100, 4096, "f32", dict(threads=1024, col_chunks=4)),
    (257, 1024, "f32", dict(threads=256, col_chunks=1, grid=100)),
    (64, 2048, "bf16", dict(threads=256, col_chunks=4, rows_per_step=2, grid=16)),
    (1024, 2048, "bf16", dict(threads=256, col_chunks=1, rows_per_step=2)),  # four rows per program
    # two chunks per lane, gamma re-read (rows of more than 512 chunks)
    (256, 8192, "bf16", dict(threads=512, col_chunks=4, w_regs=0)),
    (1000, 8192, "bf16", dict(threads=512, col_chunks=4, w_regs=0)),
    (300, 8000, "bf16", dict(threads=512, col_chunks=2, w_regs=0, grid=37)),
    (600, 4096, "f32", dict(threads=512, col_chunks=4, w_regs=0, depth=0)),
]
COLS_CASES = [(M, N, dt, f, fu) for M, N, dt, f in COLS + in_f16(COLS) for fu in (False, True)]


@pytest.mark.parametrize("M,N,dt,fields,fused", COLS_CASES,
                         ids=[f"{dt}_{M}x{N}_t{f['threads']}_cs{f['col_chunks']}_g{f.get('grid', 0)}"
                              + ("_pairs" if f.get("rows_per_step") == 2 else "") + ("_fused" if fu else "")
                              for M, N, dt, f, fu in COLS_CASES])
def test_one_launch_backward(M, N, dt, fields, fused):
    vec = 4 if dt == "f32" else 8
    gemma = dt == "f32"
    offset = 1.0 if gemma else 0.0
    op = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    over = dict(path=rn.PATH_ROWS_COLS, vec=vec, team=0, depth=1, w_regs=1)
    over.update(fields)
    with rn.plan_override(op, **over):
        p = rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)
        assert (p["path"], p["col_chunks"], p["programs"], p["chunks"]) == (rn.PATH_ROWS_COLS, fields["col_chunks"],
                                                                            0, 2 - over["w_regs"]), p
        inp, out, dx, dg = run_case(M, N, dt, fused, gemma)
        # bit-identical run to run
        dx2, dg2 = gpu_backward(inp, dt, EPS, offset, out, fused)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(dx2).view(np.uint8), from_dev(dx).view(np.uint8))
        assert np.array_equal(from_dev(dg2).view(np.uint8), from_dev(dg).view(np.uint8))
        # rstd recomputed inside the call (a statistics forward, then the one launch)
        dx3, dg3 = gpu_backward(inp, dt, EPS, offset, out, fused, rstd=None)
        torch.cuda.synchronize()
        v_ref = reference_h(inp, dt, EPS, offset) if fused else inp["x"]
        check_backward(inp, dt, EPS, offset, from_dev(dx3), from_dev(dg3), v_full=v_ref,
                       dh_full=inp["dh"] if fused else None)
        if fused:  # dx written over dh gives the same bytes
            dh = to_dev(inp["dh"], dt)
            dx4, _ = rn.rmsnorm_fused_add_bwd(to_dev(inp["dy"], dt), dh, out["h"], out["gamma"], out["rstd"], EPS,
                                              offset, dx=dh)
            torch.cuda.synchronize()
            assert dx4.data_ptr() == dh.data_ptr()
            assert np.array_equal(from_dev(dx4).view(np.uint8), from_dev(dx).view(np.uint8))


@pytest.mark.parametrize("M,N,dt,fused", [(1024, 2048, "bf16", False), (768, 4096, "bf16", True),
                                          (512, 8192, "bf16", False), (768, 2048, "f32", False),
                                          (768, 8192, "bf16", True), (768, 4096, "f32", False),
                                          (512, 6656, "bf16", False)])  # 832 lanes: not halved
def test_one_launch_backward_default_shapes(M, N, dt, fused):
    op = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    assert rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)["path"] == rn.PATH_ROWS_COLS
    run_case(M, N, dt, fused, gemma=dt == "f32")


def test_one_launch_backward_is_the_default_for_few_rows():
    """The selector takes the one-launch path for the 512 x 2048 workload and
    it matches the two-stage backward's dx bit for bit and its dgamma to the
    last rounding; the stage entry point still writes partial rows there."""
    M, N, dt = 512, 2048, "bf16"
    assert rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.BF16)["path"] == rn.PATH_ROWS_COLS
    inp = make_inputs(M, N, dt)
    out = gpu_forward(inp, dt, EPS, 0.0, False)
    dy = to_dev(inp["dy"], dt)
    dx1, dg1 = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=256, depth=1, w_regs=1,
                          rows_per_step=2):
        dx2, dg2 = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
    dx3, ws, programs = rn.rmsnorm_bwd_partials(dy, out["x"], out["gamma"], out["rstd"])
    torch.cuda.synchronize()
    assert programs > 0 and torch.equal(dx1, dx3)
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    a, b = dg1.float(), dg2.float()
    assert ((a - b).abs() <= 2 ** -7 * b.abs()).all()  # at most one bf16 rounding apart
    check_backward(inp, dt, EPS, 0.0, from_dev(dx1), from_dev(dg1), v_full=inp["x"])


# Non-affine op (no gamma): rows and looped paths, plain and fused, with the
# GPU's rstd and with rstd recomputed.
NON_AFFINE = [(300, 4096, "bf16", False), (200, 7168, "bf16", True), (130, 6144, "f32", False),
              (1000, 128, "bf16", True), (17, 4097, "bf16", False), (5, 20000, "f32", True),
              (7, 16384, "bf16", False), (5, 32768, "bf16", True), (6, 12000, "f32", False)]


@pytest.mark.parametrize("M,N,dt,fused", NON_AFFINE + in_f16(NON_AFFINE[:2]),
                         ids=[f"{d}_{m}x{n}{'_fused' if f else ''}" for m, n, d, f in NON_AFFINE + in_f16(NON_AFFINE[:2])])
def test_non_affine(M, N, dt, fused):
    inp = make_inputs(M, N, dt, fused=fused)
    inp["gamma"] = None
    out = gpu_forward(inp, dt, EPS, 0.0, fused)
    torch.cuda.synchronize()
    check_forward(inp, dt, EPS, 0.0, from_dev(out["y"]), from_dev(out["rstd"]), from_dev(out["h"]) if fused else None)
    v_ref = reference_h(inp, dt) if fused else inp["x"]
    for rstd in ("gpu", None):
        dx, dg = gpu_backward(inp, dt, EPS, 0.0, out, fused, rstd=rstd)
        torch.cuda.synchronize()
        assert dg is None
        check_backward(inp, dt, EPS, 0.0, from_dev(dx), None, v_full=v_ref, dh_full=inp["dh"] if fused else None)


def _offset_view(a: torch.Tensor, elems: int) -> torch.Tensor:
    """The same values at a storage offset of `elems` elements (not 16-byte aligned)."""
    flat = torch.empty(a.numel() + elems, dtype=a.dtype, device=a.device)
    v = flat[elems:].view(a.shape)
    v.copy_(a)
    return v


@pytest.mark.parametrize("M,N,dt", [(100, 4096, "bf16"), (50, 6144, "f32"), (300, 128, "bf16"), (100, 4096, "f16")])
def test_unaligned_storage_offsets(M, N, dt):
    for fused in (False, True):
        inp = make_inputs(M, N, dt, fused=fused)
        x = _offset_view(to_dev(inp["x"], dt), 1)
        g = _offset_view(to_dev(inp["gamma"], dt), 3)
        assert x.data_ptr() % 16 != 0
        if fused:
            r = _offset_view(to_dev(inp["residual"], dt), 1)
            y, h, rstd = rn.rmsnorm_fused_add_fwd(x, r, g, EPS, 0.0, y=_offset_view(torch.empty_like(x), 1),
                                                  h_out=_offset_view(torch.empty_like(x), 5))
        else:
            y, rstd = rn.rmsnorm_fwd(x, g, EPS, 0.0, y=_offset_view(torch.empty_like(x), 1))
            h = None
        torch.cuda.synchronize()
        check_forward(inp, dt, EPS, 0.0, from_dev(y), from_dev(rstd), None if h is None else from_dev(h))
        dy = _offset_view(to_dev(inp["dy"], dt), 1)
        dx_out = _offset_view(torch.empty_like(x), 7)
        if fused:
            dh = _offset_view(to_dev(inp["dh"], dt), 1)
            dx, dg = rn.rmsnorm_fused_add_bwd(dy, dh, h, g, rstd, EPS, 0.0, dx=dx_out)
        else:
            dx, dg = rn.rmsnorm_bwd(dy, x, g, rstd, EPS, 0.0, dx=dx_out)
        torch.cuda.synchronize()
        check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg),
                       v_full=reference_h(inp, dt) if fused else inp["x"], dh_full=inp["dh"] if fused else None)


def test_zero_rows_writes_zero_dgamma():
    for dt, td in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        x = torch.empty(0, 4096, dtype=td, device="cuda")
        g = torch.ones(4096, dtype=td, device="cuda")
        y, rstd = rn.rmsnorm_fwd(x, g)
        dg = torch.full((4096,), float("nan"), dtype=td, device="cuda")
        dx, dg = rn.rmsnorm_bwd(torch.empty_like(x), x, g, rstd, dgamma=dg)
        torch.cuda.synchronize()
        assert y.shape == (0, 4096) and torch.all(dg == 0)


def test_in_place_fused_aliases():
    """h_out may overwrite residual; dx may overwrite dh."""
    M, N, dt = 500, 7168, "bf16"
    inp = make_inputs(M, N, dt, fused=True)
    x, g = to_dev(inp["x"], dt), to_dev(inp["gamma"], dt)
    r = to_dev(inp["residual"], dt)
    y, h, rstd = rn.rmsnorm_fused_add_fwd(x, r, g, EPS, 0.0, h_out=r)
    assert h.data_ptr() == r.data_ptr()
    torch.cuda.synchronize()
    check_forward(inp, dt, EPS, 0.0, from_dev(y), from_dev(rstd), from_dev(h))
    dy, dh = to_dev(inp["dy"], dt), to_dev(inp["dh"], dt)
    dx, dg = rn.rmsnorm_fused_add_bwd(dy, dh, h, g, rstd, EPS, 0.0, dx=dh)
    assert dx.data_ptr() == dh.data_ptr()
    torch.cuda.synchronize()
    check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg), v_full=reference_h(inp, dt), dh_full=inp["dh"])


# Fused forwards on the looped path with h_out = residual: later passes must
# read the h each lane stored, not x + residual (residual is h by then).
# bf16 / fp32 N = 10001 at an odd storage offset take the per-element looped
# kernel; bf16 N = 131072, aligned, the 16-byte one with chunks beyond those
# staged in LDS.  Each op's plan is checked to be the looped one.
IN_PLACE_LOOPED = [(24, 10001, "bf16", False), (24, 10001, "f32", False), (6, 131072, "bf16", True)]


def _maybe_offset(t: torch.Tensor, aligned: bool, elems: int) -> torch.Tensor:
    return t if aligned else _offset_view(t, elems)


@pytest.mark.parametrize("M,N,dt,aligned", IN_PLACE_LOOPED,
                         ids=[f"{d}_{m}x{n}" + ("" if a else "_unaligned") for m, n, d, a in IN_PLACE_LOOPED])
def test_in_place_residual_looped(M, N, dt, aligned):
    code = CODE[dt]
    for op in (rn.OP_FUSED_ADD_FWD, rn.OP_FUSED_ADD_FWD_FP8, rn.OP_LN_FUSED_ADD_FWD):
        assert rn.rmsnorm_query_plan(op, M, N, code, vec_ok=aligned)["path"] == rn.PATH_LOOP, op
    inp = make_inputs(M, N, dt, fused=True)
    x = _maybe_offset(to_dev(inp["x"], dt), aligned, 1)
    g = _maybe_offset(to_dev(inp["gamma"], dt), aligned, 3)
    # RMSNorm
    r = _maybe_offset(to_dev(inp["residual"], dt), aligned, 1)
    y, h, rstd = rn.rmsnorm_fused_add_fwd(x, r, g, EPS, 0.0, h_out=r)
    assert h.data_ptr() == r.data_ptr()
    torch.cuda.synchronize()
    check_forward(inp, dt, EPS, 0.0, from_dev(y), from_dev(rstd), from_dev(h))
    # fp8 output
    r = _maybe_offset(to_dev(inp["residual"], dt), aligned, 1)
    sc = torch.tensor([8.0], dtype=torch.float32, device="cuda")
    am = torch.zeros(1, dtype=torch.float32, device="cuda")
    y8, h, rstd = rn.rmsnorm_fused_add_fwd_fp8(x, r, g, sc, EPS, 0.0, amax=am, h_out=r)
    torch.cuda.synchronize()
    h_ref = reference_h(inp, dt)
    assert np.array_equal(from_dev(h), h_ref), "fp8 fused: h differs"
    ref = oracle.fwd_fp8(h_ref, inp["gamma"], dt, EPS, 0.0, 8.0, tol=1e-5)
    codes = y8.view(torch.uint8).cpu().numpy()
    ok = (codes == ref["code_lo"]) | (codes == ref["code_hi"])
    assert ok.all(), f"fp8 fused: {int((~ok).sum())} codes outside the tolerance interval"
    assert abs(float(am.item()) - ref["amax64"]) <= 1e-5 * ref["amax64"]
    # LayerNorm, forward in place then its backward
    lin = make_inputs(M, N, dt, fused=True, layernorm=True)
    xl = _maybe_offset(to_dev(lin["x"], dt), aligned, 1)
    gl = _maybe_offset(to_dev(lin["gamma"], dt), aligned, 3)
    bl = _maybe_offset(to_dev(lin["beta"], dt), aligned, 5)
    rl = _maybe_offset(to_dev(lin["residual"], dt), aligned, 1)
    yl, hl, mean, lrstd = rn.layernorm_fused_add_fwd(xl, rl, gl, bl, LN_EPS, 0.0, h_out=rl)
    assert hl.data_ptr() == rl.data_ptr()
    dxl, dgl, dbl = rn.layernorm_fused_add_bwd(to_dev(lin["dy"], dt), to_dev(lin["dh"], dt), hl, gl, mean, lrstd,
                                               LN_EPS, 0.0)
    torch.cuda.synchronize()
    got = {"y": yl, "h": hl, "mean": mean, "rstd": lrstd, "dx": dxl, "dg": dgl, "db": dbl}
    check_ln(lin, dt, LN_EPS, 0.0, True, {k: from_dev(v) for k, v in got.items()})


def test_workspace_too_small_is_refused_before_launch():
    M, N = 4096, 4096
    x = torch.randn(M, N, device="cuda").to(torch.bfloat16)
    g = torch.ones(N, dtype=torch.bfloat16, device="cuda")
    need = rn.rmsnorm_bwd_workspace_bytes(M, N, rn.BF16)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    dx = torch.full_like(x, 7.0)
    with pytest.raises(rn.RMSNormError) as e:
        rn.rmsnorm_bwd(x, x, g, None, dx=dx, workspace=ws)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(dx == 7.0)  # nothing ran


def test_stage_entry_points_match_one_call():
    M, N, dt = 1000, 4096, "bf16"
    inp = make_inputs(M, N, dt)
    out = gpu_forward(inp, dt, EPS, 0.0, False)
    dy = to_dev(inp["dy"], dt)
    dx1, dg1 = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
    dx2, ws, programs = rn.rmsnorm_bwd_partials(dy, out["x"], out["gamma"], out["rstd"])
    dg2 = torch.empty_like(dg1)
    rn.rmsnorm_dgamma_finalize(ws, programs, N, dg2)
    torch.cuda.synchronize()
    assert programs == rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.BF16)["programs"]
    assert torch.equal(dx1, dx2) and torch.equal(dg1.view(torch.int16), dg2.view(torch.int16))
    # the partials themselves sum (in float64) to the reference dgamma
    part = ws.view(torch.float32)[: programs * rn.partial_ld(N)].view(programs, -1)[:, :N].double().sum(0).cpu().numpy()
    ref = oracle.bwd(inp["dy"], inp["x"], inp["gamma"], dt, EPS, 0.0, want_dx=False)["dgamma64"]
    assert np.linalg.norm(part - ref) / np.linalg.norm(ref) < 1e-5
