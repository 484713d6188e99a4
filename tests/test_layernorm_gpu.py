"""GPU parity of LayerNorm (forward and backward, plain and fused residual add)
against the fp64 reference.

The rules are RMSNorm's, with LayerNorm's cancellation floors (gpu_util.check_ln)."""

import numpy as np
import pytest
import torch

import oracle
import transformer_normalization_rmsnorm_amd as rn
from gpu_util import CODE, check_ln, gpu_ln, in_f16, to_dev
from rmsnorm_inputs import make_inputs
from tolerance import DGAMMA_TOL, dgamma_error

pytestmark = pytest.mark.gpu

EPS = 1e-5


# (M, N, dtype, fused, gemma)
CASES = [
    (300, 4096, "bf16", False, False),    # workgroup teams, w in registers
    (130, 6144, "f32", False, True),      # float32, gamma + offset
    (200, 7168, "bf16", True, False),     # fused residual add
    (1000, 128, "bf16", False, False),    # 16-lane teams
    (1000, 128, "bf16", True, False),
    (37, 64, "f32", False, False),
    (257, 8192, "bf16", False, False),
    (33, 5000, "bf16", False, False),     # ragged vector groups
    (17, 4097, "bf16", False, False),     # scalar access
    (9, 8200, "bf16", True, False),
    (5, 2, "bf16", False, False),         # N = 2
    (70, 16384, "bf16", False, False),    # wide rows: gamma per row
    (45, 16384, "bf16", True, False),
    (20, 24576, "bf16", False, False),
    (7, 12000, "f32", True, True),
    (6, 32768, "bf16", False, False),     # four chunks x 1024 lanes, dbeta in LDS
    (5, 16384, "f32", False, True),
    (6, 32768, "bf16", True, False),      # fused: four chunks x 1024 lanes, exact tiling only
    (5, 30000, "bf16", True, False),      # fused, ragged: eight chunks x 512 lanes, masked
    (5, 16384, "f32", True, False),       # fused float32: four chunks x 1024 lanes
    (4, 40000, "f32", True, True),
    (3, 4096, "bf16", False, False),      # fewer rows than programs
]


def case_id(c):
    M, N, dt, fused, gemma = c
    return f"{dt}_{M}x{N}" + ("_fused" if fused else "") + ("_offset1" if gemma else "")


@pytest.mark.parametrize("case", CASES + in_f16(CASES), ids=case_id)
def test_layernorm_parity(case):
    M, N, dt, fused, gemma = case
    inp = make_inputs(M, N, dt, fused=fused, gemma=gemma, layernorm=True)
    offset = 1.0 if gemma else 0.0
    got = gpu_ln(inp, dt, EPS, offset, fused)
    r = check_ln(inp, dt, EPS, offset, fused, got)
    print(f"{case_id(case)}: {r}")


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3], CASES[8], CASES[11], CASES[15]], ids=case_id)
def test_layernorm_recomputes_statistics(case):
    M, N, dt, fused, gemma = case
    inp = make_inputs(M, N, dt, fused=fused, gemma=gemma, layernorm=True)
    offset = 1.0 if gemma else 0.0
    check_ln(inp, dt, EPS, offset, fused, gpu_ln(inp, dt, EPS, offset, fused, stats=None))


@pytest.mark.parametrize("affine,bias", [(False, False), (True, False), (False, True)])
def test_layernorm_without_gamma_or_beta(affine, bias):
    # rows in registers, and rows beyond them (looped kernels)
    for M, N in ((64, 2048), (3, 40960)):
        for fused in (False, True):
            inp = make_inputs(M, N, "bf16", fused=fused, layernorm=True)
            got = gpu_ln(inp, "bf16", EPS, 0.0, fused, affine=affine, bias=bias)
            check_ln(inp, "bf16", EPS, 0.0, fused, got, affine=affine, bias=bias)


# Every LayerNorm backward layout, forced on a shape it tiles, with a small grid.
R = rn.PATH_ROWS
LN_FORCED = [
    (True, 300, 1024, "bf16", dict(path=R, vec=8, team=64, threads=256)),
    (True, 300, 512, "bf16", dict(path=R, vec=8, team=64, threads=256)),
    (True, 1000, 256, "bf16", dict(path=R, vec=8, team=32, threads=256, grid=7)),
    (True, 300, 4096, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=2, grid=9)),
    (True, 40, 16384, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=0, w_regs=0, grid=7)),
    (True, 40, 8192, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=0, grid=6)),
    (True, 30, 24576, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=0, w_regs=0, grid=4)),
    (True, 30, 16384, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=0, w_regs=0, grid=4)),
    (True, 30, 16384, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=0, grid=4)),
    (True, 20, 24576, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    (True, 20, 32768, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=0, w_regs=0, grid=3)),
    (True, 20, 32768, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    (True, 20, 30000, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    (True, 20, 16384, "f32", dict(path=R, vec=4, team=0, threads=512, depth=0, w_regs=0, grid=3)),
    (True, 20, 15000, "f32", dict(path=R, vec=4, team=0, threads=960, depth=0, w_regs=0, grid=3)),
    (True, 30, 16384, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=1, w_regs=0, grid=4)),
    (True, 30, 8192, "f32", dict(path=R, vec=4, team=0, threads=1024, depth=1, w_regs=0, grid=4)),
    (True, 30, 16000, "bf16", dict(path=R, vec=8, team=0, threads=1024, depth=1, w_regs=0, grid=4)),
    (True, 20, 4000, "f32", dict(path=R, vec=4, team=0, threads=256, depth=0, w_regs=0, grid=3)),
    (True, 100, 2048, "bf16", dict(path=R, vec=1, team=0, threads=512, grid=5)),
    (True, 300, 128, "bf16", dict(path=R, vec=1, team=64, threads=256)),
    # two rows per reduction (plain LayerNorm): odd and even rows per program, one row per program, ragged
    (False, 300, 2048, "bf16", dict(path=R, vec=8, team=0, threads=256, depth=1, w_regs=1, rows_per_step=2, grid=19)),
    (False, 257, 4096, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=1, rows_per_step=2, grid=128)),
    (False, 64, 2048, "bf16", dict(path=R, vec=8, team=0, threads=256, depth=1, w_regs=1, rows_per_step=2, grid=64)),
    (False, 45, 4000, "bf16", dict(path=R, vec=8, team=0, threads=512, depth=1, w_regs=1, rows_per_step=2, grid=4)),
    (False, 300, 1024, "f32", dict(path=R, vec=4, team=0, threads=256, depth=1, w_regs=1, rows_per_step=2, grid=17)),
    (True, 60, 4096, "bf16", dict(path=rn.PATH_LOOP, vec=8, team=0, threads=512, grid=9)),
    (True, 60, 4096, "f32", dict(path=rn.PATH_LOOP, vec=1, team=0, threads=256, grid=9)),
]


# every layout plain, and fused-add where it is compiled for the fused op
LN_CASES = [(M, N, dt, f, fused) for ok, M, N, dt, f in LN_FORCED + in_f16(LN_FORCED)
            for fused in ((False, True) if ok else (False,))]


@pytest.mark.parametrize("M,N,dt,fields,fused", LN_CASES,
                         ids=[f"{dt}_{M}x{N}_" + "_".join(f"{a}{b}" for a, b in f.items()) + "-" +
                              ("fused" if fu else "plain") for M, N, dt, f, fu in LN_CASES])
def test_layernorm_backward_layouts(M, N, dt, fields, fused):
    op = rn.OP_LN_FUSED_ADD_BWD if fused else rn.OP_LN_BWD
    inp = make_inputs(M, N, dt, fused=fused, gemma=(dt == "f32"), layernorm=True)
    offset = 1.0 if dt == "f32" else 0.0
    with rn.plan_override(op, **fields):
        p = rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)
        for k, v in fields.items():
            assert p[k] == v, (k, p)
        check_ln(inp, dt, EPS, offset, fused, gpu_ln(inp, dt, EPS, offset, fused))


# One-launch LayerNorm backward (PATH_ROWS_COLS): dgamma and dbeta summed by
# column workgroups of the dx launch, no partial rows.  Forced at every slab
# width, one row per program and several, a grid that is not a multiple of 8,
# a ragged row, two rows per reduction (plain op); statistics given and
# recomputed, without gamma, and run to run.
LN_COLS = [
    (512, 2048, "bf16", dict(threads=256, col_chunks=1)),
    (128, 8192, "bf16", dict(threads=1024, col_chunks=8)),
    (300, 4096, "bf16", dict(threads=512, col_chunks=4, grid=37)),
    (200, 2000, "bf16", dict(threads=256, col_chunks=2)),
    (100, 4096, "f32", dict(threads=1024, col_chunks=4)),
    (64, 2048, "bf16", dict(threads=256, col_chunks=4, rows_per_step=2, grid=16)),
    (768, 2048, "bf16", dict(threads=256, col_chunks=1, rows_per_step=2)),  # three rows per program
    # two chunks per lane, gamma re-read (rows of more than 512 chunks)
    (1000, 8192, "bf16", dict(threads=512, col_chunks=4, w_regs=0)),
    (300, 4000, "f32", dict(threads=512, col_chunks=2, w_regs=0, grid=37)),
]
LN_COLS_CASES = [(M, N, dt, f, fu) for M, N, dt, f in LN_COLS + in_f16(LN_COLS) for fu in (False, True)
                 if not (fu and f.get("rows_per_step") == 2)]  # fused-add LayerNorm has no two-row instance


@pytest.mark.parametrize("M,N,dt,fields,fused", LN_COLS_CASES,
                         ids=[f"{dt}_{M}x{N}_t{f['threads']}_cs{f['col_chunks']}_g{f.get('grid', 0)}"
                              + ("_pairs" if f.get("rows_per_step") == 2 else "") + ("_fused" if fu else "")
                              for M, N, dt, f, fu in LN_COLS_CASES])
def test_layernorm_one_launch_backward(M, N, dt, fields, fused):
    op = rn.OP_LN_FUSED_ADD_BWD if fused else rn.OP_LN_BWD
    vec = 4 if dt == "f32" else 8
    over = dict(path=rn.PATH_ROWS_COLS, vec=vec, team=0, depth=1, w_regs=1)
    over.update(fields)
    with rn.plan_override(op, **over):
        p = rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)
        assert (p["path"], p["col_chunks"], p["programs"], p["chunks"]) == (rn.PATH_ROWS_COLS, fields["col_chunks"],
                                                                            0, 2 - over["w_regs"]), p
        inp = make_inputs(M, N, dt, fused=fused, layernorm=True)
        got = gpu_ln(inp, dt, EPS, 0.0, fused)
        check_ln(inp, dt, EPS, 0.0, fused, got)
        again = gpu_ln(inp, dt, EPS, 0.0, fused)
        for k in ("dx", "dg", "db"):
            assert np.array_equal(got[k].view(np.uint8), again[k].view(np.uint8)), k
        check_ln(inp, dt, EPS, 0.0, fused, gpu_ln(inp, dt, EPS, 0.0, fused, stats=None))
        check_ln(inp, dt, EPS, 0.0, fused, gpu_ln(inp, dt, EPS, 0.0, fused, affine=False), affine=False)


@pytest.mark.parametrize("M,N,dt,fused", [(768, 4096, "bf16", False), (768, 2048, "bf16", True),
                                          (512, 8192, "bf16", False), (600, 1024, "f32", True),
                                          (1024, 8192, "bf16", False), (1024, 2048, "f32", False),
                                          (600, 4608, "bf16", True),  # 576 lanes: not halved
                                          (1280, 8192, "bf16", True)])  # five rows per program
def test_layernorm_one_launch_backward_is_the_default_for_few_rows(M, N, dt, fused):
    op = rn.OP_LN_FUSED_ADD_BWD if fused else rn.OP_LN_BWD
    assert rn.rmsnorm_query_plan(op, M, N, CODE[dt], True)["path"] == rn.PATH_ROWS_COLS
    inp = make_inputs(M, N, dt, fused=fused, layernorm=True)
    check_ln(inp, dt, EPS, 0.0, fused, gpu_ln(inp, dt, EPS, 0.0, fused))


def test_layernorm_zero_rows_writes_zero_gradients():
    x = torch.empty(0, 4096, dtype=torch.bfloat16, device="cuda")
    g = torch.ones(4096, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(4096, dtype=torch.bfloat16, device="cuda")
    y, mean, rstd = rn.layernorm_fwd(x, g, b)
    dg = torch.full((4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    db = torch.full((4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    rn.layernorm_bwd(torch.empty_like(x), x, g, mean, rstd, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert torch.all(dg == 0) and torch.all(db == 0)


def test_layernorm_gradients_are_bit_identical_run_to_run():
    M, N, dt = 2048, 4096, "bf16"
    inp = make_inputs(M, N, dt, layernorm=True)
    first = gpu_ln(inp, dt, EPS, 0.0, False)
    for _ in range(2):
        again = gpu_ln(inp, dt, EPS, 0.0, False)
        for k in ("y", "mean", "rstd", "dx", "dg", "db"):
            assert np.array_equal(first[k], again[k]), k


def test_layernorm_graph_replay_matches_eager():
    """Fused-add LayerNorm forward + backward captured in a HIP graph; every
    replay, with eager work and synchronisations between them, equals eager."""
    M, N, dt = 2048, 4096, "bf16"
    inp = make_inputs(M, N, dt, fused=True, layernorm=True)
    x, r, g, b = (to_dev(inp[k], dt) for k in ("x", "residual", "gamma", "beta"))
    dy, dh = to_dev(inp["dy"], dt), to_dev(inp["dh"], dt)
    y, h = torch.empty_like(x), torch.empty_like(x)
    mean, rstd = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    dx, dg, db = torch.empty_like(x), torch.empty_like(g), torch.empty_like(g)
    ws = torch.empty(rn.layernorm_bwd_workspace_bytes(M, N, rn.BF16), dtype=torch.uint8, device="cuda")

    def step():
        rn.layernorm_fused_add_fwd(x, r, g, b, EPS, 0.0, y=y, h_out=h, mean=mean, rstd=rstd)
        rn.layernorm_fused_add_bwd(dy, dh, h, g, mean, rstd, EPS, 0.0, dx=dx, dgamma=dg, dbeta=db, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, h, mean, rstd, dx, dg, db)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        for t in (y, h, mean, rstd, dx, dg, db):
            t.fill_(float("nan"))
        _ = (x.float() * 2).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, c in zip(("y", "h", "mean", "rstd", "dx", "dgamma", "dbeta"), (y, h, mean, rstd, dx, dg, db), ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32)), \
                f"replay {i}: {name} differs"


@pytest.mark.parametrize("name", ["bf16_4096x4096", "bf16_16384x7168_fused_add", "f32_16384x6144_offset1",
                                  "bf16_262144x128_per_head"])
def test_layernorm_full_size(name):
    """Benchmark workload shapes with the LayerNorm recipe: y, mean, rstd and dx
    on a sample of rows, dgamma and dbeta over all rows."""
    from rmsnorm_inputs import ALL_WORKLOADS, sample_rows

    w = ALL_WORKLOADS[name]
    print(f"workload {name}", flush=True)
    inp = make_inputs(w.M, w.N, w.dtype, fused=w.fused, gemma=w.gemma, layernorm=True)
    got = gpu_ln(inp, w.dtype, EPS, w.offset, w.fused)
    rows = sample_rows(w.M, 48)
    sub = {k: (v[rows] if v.ndim == 2 else v) for k, v in inp.items()}
    got_s = {k: (v[rows] if (v is not None and k in ("y", "mean", "rstd", "dx", "h")) else v) for k, v in got.items()}
    # dgamma / dbeta need every row: the sampled check skips them, the full reference checks them
    v_full = inp["x"]
    if w.fused:
        v_full, _, _ = oracle.fused_add_fwd(inp["x"], inp["residual"], inp["gamma"], w.dtype, EPS, w.offset,
                                            want_y=False)
    full = oracle.ln_bwd(inp["dy"], v_full, inp["gamma"], w.dtype, EPS, w.offset,
                         dh=inp["dh"] if w.fused else None, want_dx=False)
    for k, ref in (("dg", full["dgamma64"]), ("db", full["dbeta64"])):
        err = dgamma_error(got[k], ref, w.dtype)
        assert err <= DGAMMA_TOL[w.dtype], f"{k} relative L2 {err:.3g}"
    got_s["dg"], got_s["db"] = None, None
    check_ln(sub, w.dtype, EPS, w.offset, w.fused, got_s, grads=False)

