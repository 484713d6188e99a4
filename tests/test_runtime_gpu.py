"""Runtime behaviour on the GPU: run-to-run determinism, HIP graph capture and
replay, caller streams, complete overwrite of poisoned outputs and workspaces,
and reuse across many row counts."""

import numpy as np
import pytest
import torch

import transformer_normalization_rmsnorm_amd as rn
from gpu_util import (CODE, check_backward, check_forward, from_dev, gpu_forward,
                      reference_h, to_dev)
from rmsnorm_inputs import EPS, make_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("M,N,dt,fused", [(4096, 4096, "bf16", False), (777, 7168, "bf16", True),
                                          (300, 6144, "f32", False), (5000, 128, "bf16", False)])
def test_dgamma_bit_identical_run_to_run(M, N, dt, fused):
    inp = make_inputs(M, N, dt, fused=fused)
    out = gpu_forward(inp, dt, EPS, 0.0, fused)
    dy = to_dev(inp["dy"], dt)
    dh = to_dev(inp["dh"], dt) if fused else None
    runs = []
    for _ in range(3):
        if fused:
            dx, dg = rn.rmsnorm_fused_add_bwd(dy, dh, out["h"], out["gamma"], out["rstd"])
        else:
            dx, dg = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
        runs.append((dx.clone(), dg.clone()))
    torch.cuda.synchronize()
    for dx, dg in runs[1:]:
        assert torch.equal(_bits(dg), _bits(runs[0][1]))
        assert torch.equal(_bits(dx), _bits(runs[0][0]))


@pytest.mark.parametrize("M,N,fused", [(2048, 4096, True), (4096, 4096, False), (4096, 2048, True)],
                         ids=["fused_2048x4096", "plain_4096x4096_two_rows", "fused_4096x2048_two_rows"])
def test_graph_replay_matches_eager(M, N, fused):
    """Capture fwd + bwd on the capture stream; replay several times with eager
    work and synchronisations between replays; every replay equals eager bitwise.
    The last two shapes reduce two rows together in the backward."""
    dt = "bf16"
    op = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    assert rn.rmsnorm_query_plan(op, M, N, rn.BF16)["rows_per_step"] == (1 if (M, N) == (2048, 4096) else 2)
    inp = make_inputs(M, N, dt, fused=True)
    x, r, g = to_dev(inp["x"], dt), to_dev(inp["residual"], dt), to_dev(inp["gamma"], dt)
    dy, dh = to_dev(inp["dy"], dt), to_dev(inp["dh"], dt)
    y, h, rstd = torch.empty_like(x), torch.empty_like(x), torch.empty(M, device="cuda")
    dx, dg = torch.empty_like(x), torch.empty_like(g)
    ws, _ = rn.alloc_workspace(M, N, rn.BF16, x.device)

    def step():
        if fused:
            rn.rmsnorm_fused_add_fwd(x, r, g, EPS, 0.0, y=y, h_out=h, rstd=rstd)
            rn.rmsnorm_fused_add_bwd(dy, dh, h, g, rstd, EPS, 0.0, dx=dx, dgamma=dg, workspace=ws)
        else:
            h.copy_(x)
            rn.rmsnorm_fwd(x, g, EPS, 0.0, y=y, rstd=rstd)
            rn.rmsnorm_bwd(dy, x, g, rstd, EPS, 0.0, dx=dx, dgamma=dg, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, h, rstd, dx, dg)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for i in range(4):
        for t in (y, h, rstd, dx, dg):
            t.fill_(float("nan"))
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "h", "rstd", "dx", "dg"), (y, h, rstd, dx, dg), ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {i}: {name} differs"



# Entry points with their own kernels or extra launches: the fp8 forward with
# its amax finalizer, LayerNorm (saved statistics, and statistics recomputed
# into the workspace inside the call), the looped kernels (rows beyond the
# register layouts), the per-element path (N not a multiple of the vector) and
# the one-launch backward for few rows (dgamma by column workgroups).
OTHER_GRAPH_CASES = [("fp8_amax", 2048, 4096), ("fp8_fused_amax", 1024, 7168), ("layernorm_saved_stats", 1024, 4096),
                     ("layernorm_recomputed_stats", 1024, 4096), ("looped", 64, 40000), ("per_element", 300, 1001),
                     ("one_launch", 256, 4096)]


@pytest.mark.parametrize("case,M,N", OTHER_GRAPH_CASES, ids=[c[0] for c in OTHER_GRAPH_CASES])
def test_graph_replay_other_entry_points(case, M, N):
    """As test_graph_replay_matches_eager, for the other entry points: every
    replay writes what the eager calls wrote, bit for bit (amax is reset to 0
    before the eager run and before each replay, as it accumulates)."""
    dt = "bf16"
    ln = case.startswith("layernorm")
    inp = make_inputs(M, N, dt, fused=True, layernorm=ln)
    x, r, g = to_dev(inp["x"], dt), to_dev(inp["residual"], dt), to_dev(inp["gamma"], dt)
    dy = to_dev(inp["dy"], dt)
    if case == "one_launch":
        assert rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.BF16)["path"] == rn.PATH_ROWS_COLS
    if case == "looped":
        assert rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.BF16)["path"] == rn.PATH_LOOP
        assert rn.rmsnorm_query_plan(rn.OP_FWD, M, N, rn.BF16)["path"] == rn.PATH_LOOP
    outs = {}
    if case.startswith("fp8"):
        fused = case == "fp8_fused_amax"
        scale = torch.full((1,), 16.0, dtype=torch.float32, device="cuda")
        outs = {"y8": torch.empty(M, N, dtype=torch.uint8, device="cuda"),
                "rstd": torch.empty(M, device="cuda"), "amax": torch.zeros(1, device="cuda")}
        if fused:
            outs["h"] = torch.empty_like(x)
        ws = torch.empty(max(rn.rmsnorm_fwd_fp8_workspace_bytes(M, N, rn.BF16), 16), dtype=torch.uint8, device="cuda")

        def step():
            if fused:
                rn.rmsnorm_fused_add_fwd_fp8(x, r, g, scale, EPS, 0.0, amax=outs["amax"], y8=outs["y8"],
                                             h_out=outs["h"], rstd=outs["rstd"], workspace=ws)
            else:
                rn.rmsnorm_fwd_fp8(x, g, scale, EPS, 0.0, amax=outs["amax"], y8=outs["y8"], rstd=outs["rstd"],
                                   workspace=ws)
    elif ln:
        beta = to_dev(inp["beta"], dt)
        saved = case == "layernorm_saved_stats"
        outs = {"y": torch.empty_like(x), "mean": torch.empty(M, device="cuda"), "rstd": torch.empty(M, device="cuda"),
                "dx": torch.empty_like(x), "dg": torch.empty_like(g), "db": torch.empty_like(g)}
        ws, _ = rn.alloc_workspace(M, N, rn.BF16, x.device, op=rn.OP_LN_BWD)

        def step():
            rn.layernorm_fwd(x, g, beta, EPS, 0.0, y=outs["y"], mean=outs["mean"], rstd=outs["rstd"])
            rn.layernorm_bwd(dy, x, g, outs["mean"] if saved else None, outs["rstd"] if saved else None, EPS, 0.0,
                             dx=outs["dx"], dgamma=outs["dg"], dbeta=outs["db"], workspace=ws)
    else:
        outs = {"y": torch.empty_like(x), "rstd": torch.empty(M, device="cuda"), "dx": torch.empty_like(x),
                "dg": torch.empty_like(g)}
        ws, _ = rn.alloc_workspace(M, N, rn.BF16, x.device)

        def step():
            rn.rmsnorm_fwd(x, g, EPS, 0.0, y=outs["y"], rstd=outs["rstd"])
            rn.rmsnorm_bwd(dy, x, g, outs["rstd"], EPS, 0.0, dx=outs["dx"], dgamma=outs["dg"], workspace=ws)

    def reset_amax():
        if "amax" in outs:
            outs["amax"].zero_()

    reset_amax()
    step()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outs.items()}
    if "amax" in ref:
        assert ref["amax"].item() > 0.0
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    # the graph holds raw pointers: every tensor it reads (x, r, g, dy, beta,
    # scale, the workspace) stays bound to its own name until the replays end
    for i in range(4):
        for k, t in outs.items():
            if t.dtype == torch.uint8:
                t.fill_(0x7F)
            else:
                t.fill_(float("nan"))
        reset_amax()
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = []
        for k, t in outs.items():
            got, want = (t, ref[k]) if t.dtype == torch.uint8 else (_bits(t), _bits(ref[k]))
            d = got != want
            if bool(d.any()):
                where = d.nonzero()
                bad.append(f"{k}: {int(d.sum())} of {d.numel()} differ, first at {where[:4].tolist()}")
        assert not bad, f"replay {i}: " + "; ".join(bad)


def test_runs_on_the_callers_stream():
    """Two non-default streams, each with its own buffers and workspace."""
    dt = "bf16"
    cases = [make_inputs(1500, 4096, dt, seed=s) for s in (1, 2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = []
    for inp, s in zip(cases, streams):
        x, g, dy = to_dev(inp["x"], dt), to_dev(inp["gamma"], dt), to_dev(inp["dy"], dt)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for _ in range(3):
                y, rstd = rn.rmsnorm_fwd(x, g, EPS, 0.0)
                dx, dg = rn.rmsnorm_bwd(dy, x, g, rstd, EPS, 0.0)
        results.append((y, rstd, dx, dg))
    torch.cuda.synchronize()
    for inp, (y, rstd, dx, dg) in zip(cases, results):
        check_forward(inp, dt, EPS, 0.0, from_dev(y), from_dev(rstd))
        check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg), v_full=inp["x"])


@pytest.mark.parametrize("M,N,dt", [(600, 4096, "bf16"), (100, 6144, "f32"), (700, 128, "bf16"), (5, 20000, "bf16")])
def test_poisoned_outputs_and_workspace_are_overwritten(M, N, dt):
    inp = make_inputs(M, N, dt, fused=True)
    x, r, g = to_dev(inp["x"], dt), to_dev(inp["residual"], dt), to_dev(inp["gamma"], dt)
    dy, dh = to_dev(inp["dy"], dt), to_dev(inp["dh"], dt)
    nan = float("nan")
    y, h = torch.full_like(x, nan), torch.full_like(x, nan)
    rstd = torch.full((M,), nan, device="cuda")
    rn.rmsnorm_fused_add_fwd(x, r, g, EPS, 0.0, y=y, h_out=h, rstd=rstd)
    ws, nbytes = rn.alloc_workspace(M, N, CODE[dt], x.device)
    ws.view(torch.uint8).fill_(0xFF)  # all-ones bytes are NaNs as float32
    dx, dg = torch.full_like(x, nan), torch.full_like(g, nan)
    rn.rmsnorm_fused_add_bwd(dy, dh, h, g, rstd, EPS, 0.0, dx=dx, dgamma=dg, workspace=ws)
    torch.cuda.synchronize()
    check_forward(inp, dt, EPS, 0.0, from_dev(y), from_dev(rstd), from_dev(h))
    check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg), v_full=reference_h(inp, dt), dh_full=inp["dh"])


def test_reuse_across_row_counts():
    """One process, many M at a fixed N; each call is checked."""
    dt, N = "bf16", 4096
    for M in (1, 2, 255, 256, 511, 512, 513, 1023, 2049):
        inp = make_inputs(M, N, dt, seed=M)
        out = gpu_forward(inp, dt, EPS, 0.0, False)
        dx, dg = rn.rmsnorm_bwd(to_dev(inp["dy"], dt), out["x"], out["gamma"], out["rstd"])
        torch.cuda.synchronize()
        check_forward(inp, dt, EPS, 0.0, from_dev(out["y"]), from_dev(out["rstd"]))
        check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg), v_full=inp["x"])


def test_scalar_and_vector_paths_agree():
    """Forced scalar access (looped rows) against the vector path at N = 8192
    (both checked against the reference; dgamma of each is reproducible)."""
    dt, M, N = "bf16", 1024, 8192
    inp = make_inputs(M, N, dt)
    out = gpu_forward(inp, dt, EPS, 0.0, False)
    dy = to_dev(inp["dy"], dt)
    vec = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_LOOP, vec=1, team=0, threads=1024):
        assert rn.rmsnorm_query_plan(rn.OP_BWD, M, N, rn.BF16)["vec"] == 1
        sca = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
        sca2 = rn.rmsnorm_bwd(dy, out["x"], out["gamma"], out["rstd"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(sca[1]), _bits(sca2[1]))
    for dx, dg in (vec, sca):
        check_backward(inp, dt, EPS, 0.0, from_dev(dx), from_dev(dg), v_full=inp["x"])
    diff = (vec[0].float() - sca[0].float()).abs().max().item()
    assert np.isfinite(diff)
