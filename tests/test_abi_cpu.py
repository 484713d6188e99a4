"""C ABI checks that need no GPU: the library loads and exports every symbol the
header declares; argument errors come back as status codes before any HIP
call; the selector is a pure function of (op, M, N, dtype, alignment, CUs).

Calls here use fake device addresses only where an argument check must reject
the call before anything touches a device."""

import ctypes
import glob
import os
import re

import pytest

import transformer_normalization_rmsnorm_amd as rn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rmsnorm.h")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
CUS = 256


@pytest.fixture(scope="module")
def lib():
    return rn.load_library()


def header_functions():
    """Functions declared in every header under include/."""
    names = set()
    for h in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:rmsnorm|layernorm)_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_match_header(lib):
    declared = header_functions()
    assert declared == sorted(rn.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {rn.library_path()}").read()
    exported = set(re.findall(r" T ((?:rmsnorm|layernorm)_\w+)", out))
    assert exported == set(declared)


def test_version_and_status_strings(lib):
    assert lib.rmsnorm_version() >= 1
    assert lib.rmsnorm_status_string(0) == b"ok"
    assert lib.rmsnorm_status_string(3).startswith(b"workspace")
    assert lib.rmsnorm_status_string(99) == b"unknown status"


FAKE = 0x10000  # never dereferenced: every call below fails its checks first
ODD = 0x10001


def fwd(lib, x=FAKE, g=FAKE, y=FAKE, rstd=FAKE, M=4, N=8, eps=1e-6, off=0.0, dt=rn.BF16):
    return lib.rmsnorm_fwd(x, g, y, rstd, M, N, eps, off, dt, None)


def test_fwd_argument_errors(lib):
    assert fwd(lib, dt=7) == EUNSUPPORTED
    assert fwd(lib, M=-1) == EINVAL
    assert fwd(lib, N=0) == EINVAL
    assert fwd(lib, N=2 ** 24 + 1) == EINVAL
    assert fwd(lib, N=2 ** 31) == EINVAL
    assert fwd(lib, eps=-1e-6) == EINVAL
    assert fwd(lib, eps=float("nan")) == EINVAL
    assert fwd(lib, off=float("inf")) == EINVAL
    assert fwd(lib, x=None) == EINVAL
    assert fwd(lib, g=None) == EINVAL
    assert fwd(lib, y=None, rstd=None) == EINVAL
    assert fwd(lib, x=ODD) == EINVAL  # bf16 needs 2-byte alignment
    assert fwd(lib, rstd=FAKE + 2) == EINVAL
    assert fwd(lib, y=FAKE + 64, x=FAKE + 64) == EINVAL  # y aliases x
    assert b"aliases" in lib.rmsnorm_last_error()
    # M = 0 is a successful no-op that needs no pointers at all
    assert fwd(lib, x=None, g=None, y=None, rstd=None, M=0) == OK
    # without gamma (non-affine op) there is no offset
    assert fwd(lib, g=None, off=1.0) == EINVAL
    assert b"offset needs gamma" in lib.rmsnorm_last_error()


def test_fused_fwd_argument_errors(lib):
    f = lib.rmsnorm_fused_add_fwd
    assert f(FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 8, 1e-6, 0.0, rn.BF16, None) == EINVAL  # residual
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 8, 1e-6, 0.0, rn.BF16, None) == EINVAL  # h_out
    assert f(FAKE, FAKE + 256, FAKE + 512, FAKE + 768, FAKE, FAKE + 1024, 4, 8, 1e-6, 0.0, rn.BF16, None) == EINVAL  # h_out == x
    assert f(FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 1e-6, 0.0, rn.F32, None) == EINVAL  # f32 misaligned


def test_fp8_fwd_argument_errors(lib):
    f = lib.rmsnorm_fwd_fp8

    def call(x=FAKE, g=FAKE + 4096, y8=FAKE + 8192, rstd=None, scale=FAKE + 12288, amax=None, ws=None, M=4, N=8,
             off=0.0, dt=rn.BF16):
        return f(x, g, y8, rstd, scale, amax, ws, 0, M, N, 1e-6, off, dt, None)

    assert call(scale=None) == EINVAL
    assert b"y8 and scale" in lib.rmsnorm_last_error()
    assert call(y8=None) == EINVAL
    assert call(scale=FAKE + 12290) == EINVAL     # float32 alignment
    assert call(amax=FAKE + 12294) == EINVAL
    assert call(x=ODD) == EINVAL
    assert call(y8=FAKE) == EINVAL                # y8 aliases x
    assert call(g=None, off=1.0) == EINVAL
    assert call(dt=9) == EUNSUPPORTED
    assert call(M=0, x=None, g=None) == OK        # nothing to do
    ff = lib.rmsnorm_fused_add_fwd_fp8
    assert ff(FAKE, None, FAKE + 4096, FAKE + 8192, FAKE + 16384, None, FAKE + 12288, None, None, 0, 4, 8, 1e-6,
              0.0, rn.BF16, None) == EINVAL      # residual
    size = ctypes.c_size_t(0)
    assert lib.rmsnorm_fwd_fp8_workspace_bytes(4, 0, rn.BF16, ctypes.byref(size)) == EINVAL
    assert lib.rmsnorm_fwd_fp8_workspace_bytes(4, 8, rn.BF16, None) == EINVAL


def test_layernorm_argument_errors(lib):
    f = lib.layernorm_fwd
    # x, gamma, beta, y, mean, rstd
    assert f(FAKE, FAKE + 4096, FAKE + 8193, FAKE + 12288, None, None, 4, 8, 1e-5, 0.0, rn.BF16, None) == EINVAL
    assert f(FAKE, FAKE + 4096, FAKE + 12288, FAKE + 12288, None, None, 4, 8, 1e-5, 0.0, rn.BF16, None) == EINVAL
    assert b"aliases" in lib.rmsnorm_last_error()                       # y == beta
    assert f(FAKE, None, FAKE + 8192, None, None, None, 4, 8, 1e-5, 0.0, rn.BF16, None) == EINVAL  # nothing to do
    assert f(FAKE, None, None, FAKE + 12288, None, None, 4, 8, 1e-5, 1.0, rn.BF16, None) == EINVAL  # offset, no gamma
    assert f(None, None, None, None, None, None, 0, 8, 1e-5, 0.0, rn.BF16, None) == OK
    b = lib.layernorm_bwd
    # dy, x, gamma, mean, rstd, dx, dgamma, dbeta, ws
    args = [FAKE, FAKE + 4096, FAKE + 8192, FAKE + 12288, None, FAKE + 16384, FAKE + 20480, FAKE + 24576,
            FAKE + 32768, 1 << 20, 4, 8, 1e-5, 0.0, rn.BF16, None]
    assert b(*args) == EINVAL                                             # mean without rstd
    assert b"together" in lib.rmsnorm_last_error()
    a2 = list(args); a2[2] = None; a2[3] = None
    assert b(*a2) == EINVAL                                               # dgamma without gamma
    a3 = list(args); a3[3] = None; a3[7] = a3[5]
    assert b(*a3) == EINVAL                                               # dbeta == dx
    a4 = list(args); a4[3] = None; a4[7] = FAKE + 24577
    assert b(*a4) == EINVAL                                               # dbeta misaligned
    size = ctypes.c_size_t(0)
    assert lib.layernorm_bwd_workspace_bytes(4, -1, rn.BF16, ctypes.byref(size)) == EINVAL


def test_bwd_argument_errors(lib):
    b = lib.rmsnorm_bwd
    args = dict(dy=FAKE, x=FAKE + 4096, g=FAKE + 8192, rstd=None, dx=FAKE + 12288, dg=FAKE + 16384, ws=FAKE + 32768)

    def call(**kw):
        a = {**args, **kw}
        return b(a["dy"], a["x"], a["g"], a["rstd"], a["dx"], a["dg"], a["ws"], 1 << 20, kw.get("M", 4),
                 kw.get("N", 8), 1e-6, 0.0, kw.get("dt", rn.BF16), None)

    assert call(dg=None) == EINVAL
    assert call(dy=None) == EINVAL
    assert call(dt=5) == EUNSUPPORTED
    assert call(M=-3) == EINVAL
    assert call(ws=FAKE + 32768 + 8) == EINVAL  # workspace must be 16-byte aligned
    assert call(dx=args["dy"]) == EINVAL  # dx may alias only dh
    assert call(dg=FAKE + 1) == EINVAL
    assert call(g=None) == EINVAL  # dgamma given without gamma
    assert b"dgamma given without gamma" in lib.rmsnorm_last_error()
    fin = lib.rmsnorm_dgamma_finalize
    assert fin(None, 3, 8, FAKE, rn.BF16, None) == EINVAL
    assert fin(FAKE + 8, 3, 8, FAKE, rn.BF16, None) == EINVAL
    assert fin(FAKE, -1, 8, FAKE, rn.BF16, None) == EINVAL
    assert fin(FAKE, 3, 8, None, rn.BF16, None) == EINVAL
    programs = ctypes.c_int64(-1)
    assert lib.rmsnorm_bwd_partials(FAKE, FAKE, FAKE, None, None, FAKE + 4096, FAKE, 0, None, 4, 8, 1e-6, 0.0,
                                    rn.BF16, None) == EINVAL
    assert lib.rmsnorm_bwd_partials(FAKE, FAKE, FAKE, None, None, FAKE + 4096, FAKE, 0, ctypes.byref(programs), 4,
                                    0, 1e-6, 0.0, rn.BF16, None) == EINVAL


def plan(op, M, N, dt=rn.BF16, vec_ok=True, cus=CUS):
    return rn.rmsnorm_query_plan(op, M, N, dt, vec_ok, cus)


def covers(p, N):
    lanes = p["team"] or p["threads"]
    return lanes * p["chunks"] * p["vec"] >= N


@pytest.mark.parametrize("M,N,dt,fused", [
    (512, 2048, rn.BF16, False), (4096, 4096, rn.BF16, False), (1024, 8192, rn.BF16, False),
    (16384, 8192, rn.BF16, False), (16384, 6144, rn.F32, False), (16384, 7168, rn.BF16, True),
    (262144, 128, rn.BF16, False),
])
def test_plans_for_workloads(M, N, dt, fused):
    fop = rn.OP_FUSED_ADD_FWD if fused else rn.OP_FWD
    bop = rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD
    f = plan(fop, M, N, dt)
    b = plan(bop, M, N, dt)
    vec = 8 if dt == rn.BF16 else 4
    # the 512-row backward takes the one-launch path (two rows per program, 2 MiB rows)
    cols = M <= 2 * CUS
    assert f["path"] == rn.PATH_ROWS and b["path"] == (rn.PATH_ROWS_COLS if cols else rn.PATH_ROWS)
    for p in (f, b):
        assert p["vec"] == vec and covers(p, N)
        assert p["threads"] % 64 == 0 and 64 <= p["threads"] <= 1024
    rows_per_block = 1 if b["team"] == 0 else b["threads"] // b["team"]
    per_cu = 1 if b["team"] == 0 else 2
    assert b["grid"] == min(per_cu * CUS, -(-M // rows_per_block))
    # the forward tiles these rows exactly: no masked lanes
    lanes = f["team"] or f["threads"]
    assert lanes * f["chunks"] * f["vec"] == N
    # one row per team, nothing prefetched
    assert f["depth"] == 0 and f["grid"] == -(-M // (1 if f["team"] == 0 else f["threads"] // f["team"]))
    assert b["programs"] == (0 if cols else b["grid"])
    # w = gamma + offset stays in registers when one chunk per lane covers the
    # row, except the fused-add op at 896 or more lanes with 8+ rows per program
    # (half the lanes, two chunks, gamma re-read); the forward has no such field
    half = fused and N // vec >= 896 and N // vec <= 1024 and M >= 8 * CUS
    assert b["w_regs"] == (1 if N // vec <= 1024 and not half else 0) and f["w_regs"] == 0
    if half:
        assert (b["threads"], b["chunks"], b["depth"]) == (N // vec // 2, 2, 1)
    ld = -(-N // 64) * 64
    assert b["workspace_bytes"] == -(-b["programs"] * ld * 4 // 256) * 256 + -(-M * 4 // 256) * 256
    if cols:  # column workgroups in the same launch, in whole rounds of 8
        assert b["col_chunks"] in (1, 2, 4, 8) and b["fin_threads"] == b["threads"]
        assert b["fin_grid"] == -(-(-(-(N // vec) // b["col_chunks"])) // 8) * 8
    else:
        assert b["fin_grid"] == ld // 32 and b["col_chunks"] == 0
    assert f["workspace_bytes"] == 0


# One-launch backward (PATH_ROWS_COLS): rows of one chunk per lane with w in
# registers, or of more than 512 chunks two chunks per lane at half the lanes
# with gamma re-read; RMSNorm up to two rows per program, or four with at most
# 6 MiB of rows, or three at more than 768 chunks; LayerNorm up to four, or
# five at more than 512 chunks; the slab rule: max(threads / M, chunks / CUs)
# as a power of two, at most 8.
COLS, ROWS = rn.PATH_ROWS_COLS, rn.PATH_ROWS
COLS_CASES = [  # (M, N, dtype, fused, RMSNorm path, col_chunks, LayerNorm path, col_chunks)
    (1, 2048, rn.BF16, False, COLS, 8, COLS, 8), (64, 2048, rn.BF16, False, COLS, 4, COLS, 4),
    (256, 4096, rn.BF16, False, COLS, 2, COLS, 2),
    (256, 8192, rn.BF16, False, COLS, 4, COLS, 4), (512, 2048, rn.BF16, False, COLS, 1, COLS, 1),
    (384, 4096, rn.BF16, False, COLS, 2, COLS, 2), (256, 2048, rn.BF16, True, COLS, 1, COLS, 1),
    (128, 2048, rn.F32, False, COLS, 4, COLS, 4), (256, 4096, rn.F16, False, COLS, 2, COLS, 2),
    (512, 4096, rn.BF16, False, COLS, 2, COLS, 2), (512, 2048, rn.F32, False, COLS, 2, COLS, 2),
    (512, 8192, rn.BF16, False, COLS, 4, COLS, 4), (512, 4096, rn.F32, False, COLS, 4, COLS, 4),
    # three and four rows per program: RMSNorm up to 6 MiB of rows
    (768, 2048, rn.BF16, False, COLS, 1, COLS, 1), (768, 4096, rn.BF16, False, COLS, 2, COLS, 2),
    (768, 2048, rn.BF16, True, COLS, 1, COLS, 1), (768, 2048, rn.F32, False, COLS, 2, COLS, 2),
    (1024, 2048, rn.BF16, False, COLS, 1, COLS, 1), (1024, 1536, rn.BF16, False, COLS, 1, COLS, 1),
    (1024, 4096, rn.BF16, False, ROWS, 0, COLS, 2), (1024, 2048, rn.F32, False, ROWS, 0, COLS, 2),
    # rows of more than 512 chunks: two chunks per lane at half the lanes, up to three rows per
    # program for RMSNorm, five for LayerNorm
    (768, 8192, rn.BF16, False, COLS, 4, COLS, 4), (1024, 8192, rn.BF16, False, ROWS, 0, COLS, 4),
    (768, 8192, rn.BF16, True, COLS, 4, COLS, 4), (768, 4096, rn.F32, False, COLS, 4, COLS, 4),
    (1024, 7168, rn.BF16, False, ROWS, 0, COLS, 4), (1280, 8192, rn.BF16, True, ROWS, 0, COLS, 4),
    (1280, 4096, rn.F32, False, ROWS, 0, COLS, 4), (1536, 8192, rn.BF16, False, ROWS, 0, ROWS, 0),
    (1024, 4096, rn.F32, False, ROWS, 0, COLS, 4), (1280, 8192, rn.BF16, False, ROWS, 0, COLS, 4),
    (300, 6144, rn.BF16, False, COLS, 4, COLS, 4), (128, 8192, rn.BF16, False, COLS, 8, COLS, 4),
    # more rows per program: two stages
    (1536, 4096, rn.BF16, False, ROWS, 0, ROWS, 0), (2048, 2048, rn.BF16, False, ROWS, 0, ROWS, 0),
    (4096, 4096, rn.BF16, False, ROWS, 0, ROWS, 0), (0, 2048, rn.BF16, False, ROWS, 0, ROWS, 0),
    (256, 1024, rn.BF16, False, ROWS, 0, ROWS, 0),    # one wavefront per row: not a workgroup team
    (256, 16384, rn.BF16, False, ROWS, 0, ROWS, 0),   # gamma re-read per row
    (200, 2000, rn.BF16, False, COLS, 2, COLS, 2),    # ragged row (masked lanes)
]


@pytest.mark.parametrize("M,N,dt,fused,path,cs,ln_path,ln_cs", COLS_CASES)
def test_one_launch_backward_rule(M, N, dt, fused, path, cs, ln_path, ln_cs):
    for op, stats, want in (((rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD), 1, (path, cs)),
                            ((rn.OP_LN_FUSED_ADD_BWD if fused else rn.OP_LN_BWD), 2, (ln_path, ln_cs))):
        b = plan(op, M, N, dt)
        assert (b["path"], b["col_chunks"]) == want, b
        if want[0] == COLS:
            # two chunks per lane with gamma re-read: LayerNorm rows of more than 512 chunks,
            # RMSNorm rows of more than 768 from one row per program on
            nc = N // (4 if dt == rn.F32 else 8)
            half = nc > 768 and M >= CUS if stats == 1 else nc > 512
            assert b["programs"] == 0 and b["team"] == 0
            assert (b["chunks"], b["w_regs"]) == ((2, 0) if half else (1, 1)), b
            assert b["workspace_bytes"] == stats * (-(-M * 4 // 256) * 256)  # only recomputed statistics
        # never on unaligned data
        assert plan(op, M, N, dt, vec_ok=False)["path"] != COLS


def test_every_backward_width_has_a_plan_around_the_one_launch_rule():
    """Every backward op plans every width from 64 to 8192 bf16 / 4096 fp32
    (whole and ragged chunks) at the row counts where the one-launch rule
    changes, and its one-launch layouts are whole wavefronts."""
    for dt, vec in ((rn.BF16, 8), (rn.F32, 4)):
        for N in list(range(64 * vec, 1024 * vec + 1, 8 * vec)) + [1000 * vec + 8, 777 * vec, 513 * vec]:
            for M in (1, 200, 256, 300, 512, 600, 768, 1024, 1100):
                for op in (rn.OP_BWD, rn.OP_FUSED_ADD_BWD, rn.OP_LN_BWD, rn.OP_LN_FUSED_ADD_BWD):
                    p = plan(op, M, N, dt)
                    assert p["threads"] % 64 == 0 and covers(p, N), (op, M, N, dt, p)
                    if p["path"] == COLS:
                        assert p["col_chunks"] in (1, 2, 4, 8) and p["programs"] == 0


def test_one_launch_backward_workspace_covers_the_two_stage_layout():
    """rmsnorm_bwd_workspace_bytes stays the two-stage size, which the stage
    entry point (rmsnorm_bwd_partials) needs for the same shapes."""
    for M, N in ((512, 2048), (64, 4096), (200, 2000)):
        assert plan(rn.OP_BWD, M, N)["path"] == rn.PATH_ROWS_COLS
        with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=plan(rn.OP_BWD, M, N)["threads"]):
            two = plan(rn.OP_BWD, M, N)
        assert two["path"] == rn.PATH_ROWS and two["programs"] > 0


def test_one_launch_backward_override():
    """The override can force the path and the slab width, and refuses the
    layouts that carry no column workgroups."""
    M, N = 300, 4096
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS_COLS, vec=8, team=0, threads=512, col_chunks=8, grid=37):
        p = plan(rn.OP_BWD, M, N)
    assert (p["path"], p["col_chunks"], p["grid"], p["fin_grid"]) == (rn.PATH_ROWS_COLS, 8, 37, 64)
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS_COLS, vec=8, team=0, threads=512):
        assert plan(rn.OP_BWD, M, N)["col_chunks"] == 2  # the rule: 512 / 300 -> 2
    for bad in (dict(col_chunks=3), dict(team=64, threads=256), dict(vec=1)):
        fields = dict(path=rn.PATH_ROWS_COLS, vec=8, team=0, threads=512)
        fields.update(bad)
        with rn.plan_override(rn.OP_BWD, **fields):
            with pytest.raises(rn.RMSNormError):
                plan(rn.OP_BWD, M, N)
    # LayerNorm too, with at least two wavefronts (one folds dgamma, one dbeta)
    with rn.plan_override(rn.OP_LN_BWD, path=rn.PATH_ROWS_COLS, vec=8, team=0, threads=512):
        assert plan(rn.OP_LN_BWD, M, N)["path"] == rn.PATH_ROWS_COLS
    with rn.plan_override(rn.OP_LN_BWD, path=rn.PATH_ROWS_COLS, vec=8, team=0, threads=64):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_LN_BWD, 8, 512)


def test_plan_shapes_by_width():
    assert plan(rn.OP_FWD, 1000, 128)["team"] == 16      # 16 lanes x 8 bf16
    assert plan(rn.OP_BWD, 1000, 128)["team"] == 16
    assert plan(rn.OP_FWD, 1000, 64, rn.F32)["team"] == 16
    assert plan(rn.OP_FWD, 1000, 8)["team"] == 8
    p = plan(rn.OP_FWD, 1000, 4096)
    assert p["path"] == rn.PATH_ROWS and p["vec"] == 8 and covers(p, 4096)
    p = plan(rn.OP_BWD, 4096, 4096)
    assert (p["team"], p["threads"], p["chunks"]) == (0, 512, 1)
    p = plan(rn.OP_BWD, 1024, 7168)
    assert (p["team"], p["threads"], p["chunks"]) == (0, 896, 1)
    p = plan(rn.OP_BWD, 768, 7168)  # one launch: half the lanes, two chunks each
    assert (p["path"], p["team"], p["threads"], p["chunks"]) == (rn.PATH_ROWS_COLS, 0, 448, 2)
    p = plan(rn.OP_FWD, 1024, 6144, rn.F32)
    assert (p["team"], p["threads"], p["chunks"]) == (0, 192, 8)
    p = plan(rn.OP_FWD, 1024, 7168)
    assert (p["team"], p["threads"], p["chunks"]) == (0, 448, 2)
    p = plan(rn.OP_FWD, 1024, 8192)
    assert (p["team"], p["threads"], p["chunks"]) == (0, 128, 8)
    p = plan(rn.OP_FWD, 4096, 4096)   # 16 rows per compute unit
    assert (p["team"], p["threads"], p["chunks"]) == (0, 256, 2)
    p = plan(rn.OP_BWD, 1024, 6144, rn.F32)
    assert (p["team"], p["threads"], p["chunks"], p["depth"], p["w_regs"]) == (0, 768, 2, 1, 0)


def test_unaligned_and_ragged_take_scalar_access():
    assert plan(rn.OP_FWD, 100, 4096, vec_ok=False)["vec"] == 1
    assert plan(rn.OP_FWD, 100, 4097)["vec"] == 1          # N % 8 != 0
    assert plan(rn.OP_FWD, 100, 5000)["vec"] == 8          # 5000 % 8 == 0
    for N in (1, 7, 127, 4097, 5000, 8200, 12345):
        for op in range(4):
            for vec_ok in (True, False):
                p = plan(op, 77, N, rn.BF16, vec_ok)
                if p["path"] == rn.PATH_ROWS:
                    assert covers(p, N), (op, N, p)


@pytest.mark.parametrize("N,dt,fused,want", [
    # (team, threads, chunks, depth, w_regs)
    (8192, rn.BF16, False, (0, 1024, 1, 1, 1)),     # one chunk per lane: w in registers
    (12288, rn.BF16, False, (0, 768, 2, 1, 0)),
    (16384, rn.BF16, False, (0, 1024, 2, 1, 0)),    # gamma re-read with each row
    (16384, rn.BF16, True, (0, 1024, 2, 1, 0)),
    (20000, rn.BF16, False, (0, 896, 3, 0, 0)),     # masked lanes
    (24576, rn.BF16, True, (0, 1024, 3, 0, 0)),
    (32768, rn.BF16, False, (0, 1024, 4, 0, 0)),
    (32768, rn.BF16, True, (0, 512, 8, 0, 0)),      # the fused op also holds dh: 512-thread bound
    (8192, rn.F32, False, (0, 1024, 2, 1, 0)),
    (12000, rn.F32, True, (0, 1024, 3, 0, 0)),
    (16384, rn.F32, False, (0, 1024, 4, 0, 0)),
    (16384, rn.F32, True, (0, 512, 8, 0, 0)),
])
def test_wide_backward_rows_stay_in_registers(N, dt, fused, want):
    p = plan(rn.OP_FUSED_ADD_BWD if fused else rn.OP_BWD, 4096, N, dt)
    assert p["path"] == rn.PATH_ROWS and covers(p, N)
    assert (p["team"], p["threads"], p["chunks"], p["depth"], p["w_regs"]) == want
    assert p["grid"] == CUS and p["programs"] == CUS


@pytest.mark.parametrize("M,N,dt", [(4096, 4096, rn.BF16), (262144, 128, rn.BF16), (16384, 6144, rn.F32),
                                    (1024, 8192, rn.BF16), (100, 4097, rn.BF16), (64, 100000, rn.BF16)])
def test_fp8_plans_follow_the_forward(M, N, dt):
    for op, op8 in ((rn.OP_FWD, rn.OP_FWD_FP8), (rn.OP_FUSED_ADD_FWD, rn.OP_FUSED_ADD_FWD_FP8)):
        p, q = plan(op, M, N, dt), plan(op8, M, N, dt)
        # the same kind of layout (the workgroup tiling from the fp8 forward's own table)
        for k in ("path", "vec", "depth"):
            assert p[k] == q[k], (k, p, q)
        assert (p["team"] == 0) == (q["team"] == 0)
        if q["path"] == rn.PATH_ROWS:
            assert covers(q, N) and q["depth"] == 0
            if q["team"] == 0 and q["vec"] > 1 and (N // q["vec"]) % 64 == 0:
                # an exact workgroup tiling wherever the row has one
                assert q["threads"] * q["chunks"] == N // q["vec"], q
        assert q["programs"] == q["grid"] and q["fin_grid"] == 1 and q["fin_threads"] == 1024
        assert q["workspace_bytes"] == -(-q["grid"] * 4 // 256) * 256
        assert p["workspace_bytes"] == 0 and p["programs"] == 0
    # the fp8 output exists only for the layouts without prefetch
    with rn.plan_override(rn.OP_FWD_FP8, path=rn.PATH_ROWS, vec=8, team=0, threads=256, depth=1, grid=64):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_FWD_FP8, 4096, 4096)
    with rn.plan_override(rn.OP_FWD_FP8, path=rn.PATH_ROWS, vec=8, team=0, threads=256, depth=0, grid=64):
        q = plan(rn.OP_FWD_FP8, 4096, 4096)
        assert q["grid"] == 64 and q["workspace_bytes"] == 256


@pytest.mark.parametrize("M,N,dt", [(4096, 4096, rn.BF16), (262144, 128, rn.BF16), (16384, 6144, rn.F32),
                                    (1024, 8192, rn.BF16), (100, 4097, rn.BF16), (4096, 16384, rn.BF16),
                                    (2048, 24576, rn.BF16), (64, 100000, rn.BF16)])
def test_layernorm_plans(M, N, dt):
    ld = -(-N // 64) * 64
    for op, rop in ((rn.OP_LN_FWD, rn.OP_FWD), (rn.OP_LN_FUSED_ADD_FWD, rn.OP_FUSED_ADD_FWD)):
        q = plan(op, M, N, dt)
        assert q["workspace_bytes"] == 0 and q["depth"] == 0
        if q["path"] == rn.PATH_ROWS:
            assert covers(q, N) and q["chunks"] <= 8
            p = plan(rop, M, N, dt)
            assert (p["vec"], p["team"]) == (q["vec"], q["team"])  # the same kind of layout as RMSNorm's
            nc = N // q["vec"]
            if q["team"] == 0 and q["vec"] > 1 and nc % 64 == 0:
                # an exact workgroup tiling wherever the row has one
                assert q["threads"] * q["chunks"] == nc, q
    for op in (rn.OP_LN_BWD, rn.OP_LN_FUSED_ADD_BWD):
        q = plan(op, M, N, dt)
        if q["path"] in (rn.PATH_ROWS, rn.PATH_ROWS_COLS):
            assert covers(q, N)
        if q["path"] == rn.PATH_ROWS_COLS:  # one launch: no partial rows, only mean and rstd
            assert q["programs"] == 0 and q["workspace_bytes"] == 2 * (-(-M * 4 // 256) * 256)
            continue
        assert q["programs"] == q["grid"]
        # two sets of partial rows (dgamma, dbeta), then room for mean and rstd
        assert q["workspace_bytes"] == -(-2 * q["programs"] * ld * 4 // 256) * 256 + 2 * (-(-M * 4 // 256) * 256)
        assert q["fin_grid"] == 2 * (ld // 32)
    assert plan(rn.OP_LN_BWD, 64, 100000)["path"] == rn.PATH_LOOP


def test_layernorm_wide_backward_bounds():
    shape = lambda p: (p["path"], p["threads"], p["chunks"], p["depth"], p["w_regs"])
    R = rn.PATH_ROWS
    # LayerNorm holds the mean and a second accumulator set: its own bounds.  Two
    # chunks x 1024 threads with a row ahead fit (the fused op with dbeta in LDS)
    for op in (rn.OP_LN_BWD, rn.OP_LN_FUSED_ADD_BWD):
        assert shape(plan(op, 4096, 16384)) == (R, 1024, 2, 1, 0)
        assert shape(plan(op, 4096, 8192, rn.F32)) == (R, 1024, 2, 1, 0)
    assert shape(plan(rn.OP_LN_BWD, 4096, 4096)) == (R, 512, 1, 1, 1)
    # rows of 32768 bf16 / 16384 fp32 stay in registers for both ops
    for op in (rn.OP_LN_BWD, rn.OP_LN_FUSED_ADD_BWD):
        assert shape(plan(op, 2048, 32768)) == (R, 1024, 4, 0, 0)
        assert shape(plan(op, 2048, 16384, rn.F32)) == (R, 1024, 4, 0, 0)
    assert shape(plan(rn.OP_LN_FUSED_ADD_BWD, 2048, 24576)) == (R, 1024, 3, 0, 0)
    # bf16 fused: four chunks x 1024 threads exist only for exact tilings, so a
    # ragged row takes eight chunks x 512 threads (masked); the plain op and
    # fp32 keep four chunks
    assert shape(plan(rn.OP_LN_FUSED_ADD_BWD, 2048, 30000)) == (R, 512, 8, 0, 0)
    assert shape(plan(rn.OP_LN_BWD, 2048, 30000)) == (R, 960, 4, 0, 0)
    assert shape(plan(rn.OP_LN_FUSED_ADD_BWD, 2048, 15000, rn.F32)) == (R, 960, 4, 0, 0)
    assert shape(plan(rn.OP_LN_FUSED_ADD_BWD, 2048, 28672)) == (R, 896, 4, 0, 0)  # exact
    with rn.plan_override(rn.OP_LN_FUSED_ADD_BWD, path=R, vec=8, team=0, threads=960, depth=0, w_regs=0):
        with pytest.raises(rn.RMSNormError):  # the ragged instance is not compiled
            plan(rn.OP_LN_FUSED_ADD_BWD, 100, 30000)
    with rn.plan_override(rn.OP_LN_FUSED_ADD_BWD, path=R, vec=8, team=0, threads=512, depth=0, w_regs=0):
        assert plan(rn.OP_LN_FUSED_ADD_BWD, 100, 32768)["chunks"] == 8  # exact rows run the masked instance
    with rn.plan_override(rn.OP_LN_BWD, path=R, vec=8, team=0, threads=1024, depth=2, w_regs=0):
        with pytest.raises(rn.RMSNormError):  # two chunks, two rows ahead: not compiled
            plan(rn.OP_LN_BWD, 100, 16384)


def test_loop_path_beyond_registers():
    for N, dt in ((40960, rn.BF16), (65536, rn.BF16), (20000, rn.F32), (32768, rn.F32)):
        for op in (rn.OP_BWD, rn.OP_FUSED_ADD_BWD):
            p = plan(op, 4096, N, dt)
            assert p["path"] == rn.PATH_LOOP and p["w_regs"] == 0, (N, dt, p)
    p = plan(rn.OP_BWD, 64, 100000)
    assert p["path"] == rn.PATH_LOOP and p["grid"] == 64
    p = plan(rn.OP_FWD, 64, 1 << 20, rn.F32)
    assert p["path"] == rn.PATH_LOOP


def test_grid_caps_and_zero_rows():
    assert plan(rn.OP_BWD, 3, 4096)["grid"] == 3
    assert plan(rn.OP_BWD, 10, 128)["grid"] == 1          # 16 rows per workgroup
    z = plan(rn.OP_BWD, 0, 4096)
    assert z["grid"] == 0 and z["programs"] == 0
    assert plan(rn.OP_FWD, 0, 4096)["grid"] == 0
    assert plan(rn.OP_BWD, 10 ** 6, 4096, cus=80)["grid"] == 80


def test_row_limit_is_the_headers():
    """RMSNORM_MAX_N in the header, the binding's MAX_N and the selector agree:
    the longest row is planned (on the looped path), one more element is not."""
    m = re.search(r"#define RMSNORM_MAX_N \(1 << (\d+)\)", open(HEADER).read())
    assert m and (1 << int(m.group(1))) == rn.MAX_N
    for op in (rn.OP_FWD, rn.OP_BWD, rn.OP_FWD_FP8, rn.OP_LN_FWD, rn.OP_LN_FUSED_ADD_BWD):
        p = plan(op, 3, rn.MAX_N)
        assert p["path"] == rn.PATH_LOOP
        assert p["grid"] * p["threads"] < 2 ** 31 and p["fin_grid"] * max(p["fin_threads"], 1) < 2 ** 31
        with pytest.raises(rn.RMSNormError):
            plan(op, 3, rn.MAX_N + 1)


def test_forward_grid_keeps_work_items_below_2_31():
    """A forward over more rows than one launch can address becomes persistent."""
    for op, N in ((rn.OP_FWD, 128), (rn.OP_FWD, 1), (rn.OP_LN_FWD, 64), (rn.OP_FWD_FP8, 8)):
        p = plan(op, 2 ** 40, N)
        assert p["grid"] * p["threads"] < 2 ** 31, p


def test_backward_rows_in_flight_follow_rows_per_program():
    """Two rows in flight from 32 rows per program (w in registers), one below;
    the fused-add ops keep one (RMSNorm's fused-add takes half the lanes with
    two chunks at 896+ lanes from 8 rows per program); layouts that reduce two
    rows together keep depth 1 (their next two rows are in flight)."""
    for op in (rn.OP_BWD, rn.OP_LN_BWD):
        assert plan(op, 16384, 8192)["depth"] == 2
        assert plan(op, 1024, 8192)["depth"] == 1
    p = plan(rn.OP_FUSED_ADD_BWD, 16384, 8192)
    assert (p["threads"], p["chunks"], p["depth"], p["w_regs"]) == (512, 2, 1, 0)
    p = plan(rn.OP_FUSED_ADD_BWD, 256 * 7, 8192)
    assert (p["threads"], p["chunks"], p["depth"], p["w_regs"]) == (1024, 1, 1, 1)
    assert plan(rn.OP_LN_BWD, 256 * 32, 4096)["depth"] == 2  # 512 threads: no two-row reduction
    assert plan(rn.OP_LN_BWD, 256 * 31, 4096)["depth"] == 1
    for M in (256 * 31, 256 * 32, 16384):  # 512 lanes: neither two rows in flight nor half the lanes
        p = plan(rn.OP_FUSED_ADD_BWD, M, 4096)
        assert (p["threads"], p["chunks"], p["depth"], p["w_regs"]) == (512, 1, 1, 1)
    p = plan(rn.OP_BWD, 256 * 32, 4096)
    assert (p["depth"], p["rows_per_step"]) == (1, 2)
    assert plan(rn.OP_LN_FUSED_ADD_BWD, 16384, 8192)["depth"] == 1
    assert plan(rn.OP_BWD, 16384, 8192, cus=80)["depth"] == 2
    assert plan(rn.OP_BWD, 4096, 4096)["depth"] == 1  # 16 rows per program


@pytest.mark.parametrize("M,N,dt,want", [
    (4096, 4096, rn.BF16, 2), (4096, 4096, rn.F16, 2), (4096, 2048, rn.BF16, 2), (16384, 2048, rn.BF16, 2),
    (512, 2048, rn.BF16, 2), (16384, 4096, rn.BF16, 2), (1024, 2048, rn.F32, 2),
    (4096, 4096, rn.F32, 1),     # 1024-thread workgroups: one row per reduction
    (1024, 8192, rn.BF16, 1), (4096, 8192, rn.BF16, 1),
    (16384, 8192, rn.BF16, 1),   # 1024 threads, 64 rows per program: two rows in flight, one at a time
    (256, 4096, rn.BF16, 1),     # one row per program
    (262144, 128, rn.BF16, 1),   # sub-workgroup teams
    (4096, 16384, rn.BF16, 1),   # gamma re-read per row
])
def test_two_rows_per_reduction(M, N, dt, want):
    """rows_per_step = 2 for RMSNorm workgroup teams with w in registers, one
    chunk per lane, at most 512 threads (fused-add and plain LayerNorm: 256)
    and two or more rows per program; never for fused-add LayerNorm, nor for
    the forward."""
    p = plan(rn.OP_BWD, M, N, dt)
    assert p["rows_per_step"] == want, p
    if want == 2:
        assert (p["team"], p["chunks"], p["depth"], p["w_regs"]) == (0, 1, 1, 1)
    f = plan(rn.OP_FUSED_ADD_BWD, M, N, dt)
    assert f["rows_per_step"] == (2 if want == 2 and f["threads"] <= 256 else 1), f
    ln = plan(rn.OP_LN_BWD, M, N, dt)
    assert ln["rows_per_step"] == (2 if want == 2 and ln["threads"] <= 256 else 1), ln
    for op in (rn.OP_LN_FUSED_ADD_BWD, rn.OP_FWD, rn.OP_FUSED_ADD_FWD):
        assert plan(op, M, N, dt)["rows_per_step"] == 1


def test_two_rows_per_reduction_override_checks():
    base = plan(rn.OP_BWD, 4096, 4096)
    fields = {k: base[k] for k in ("path", "vec", "team", "threads", "depth", "w_regs")}
    with rn.plan_override(rn.OP_BWD, **fields):  # rows_per_step not given: one row per reduction
        assert plan(rn.OP_BWD, 4096, 4096)["rows_per_step"] == 1
    with rn.plan_override(rn.OP_BWD, **fields, rows_per_step=2, grid=7):
        p = plan(rn.OP_BWD, 4096, 4096)
        assert p["rows_per_step"] == 2 and p["grid"] == 7
    bad = [
        (rn.OP_BWD, dict(fields, rows_per_step=3)),
        (rn.OP_BWD, dict(fields, rows_per_step=2, depth=2)),
        (rn.OP_BWD, dict(fields, rows_per_step=2, vec=1)),
        (rn.OP_BWD, dict(path=rn.PATH_LOOP, vec=8, team=0, threads=512, rows_per_step=2)),
        (rn.OP_FUSED_ADD_BWD, dict(fields, rows_per_step=2)),  # fused: 256 threads at most
        (rn.OP_LN_BWD, dict(fields, threads=1024, rows_per_step=2)),  # LayerNorm: 512 threads at most
        (rn.OP_LN_FUSED_ADD_BWD, dict(fields, threads=256, rows_per_step=2)),  # not compiled
        (rn.OP_FWD, dict(path=rn.PATH_ROWS, vec=8, team=0, threads=256, rows_per_step=2)),
    ]
    for op, f in bad:
        with rn.plan_override(op, **f):
            with pytest.raises(rn.RMSNormError):
                plan(op, 4096, 4096)


def test_selector_rejects_bad_queries():
    with pytest.raises(rn.RMSNormError):
        plan(10, 4, 4)
    with pytest.raises(rn.RMSNormError):
        plan(rn.OP_FWD, 4, 0)
    with pytest.raises(rn.RMSNormError):
        plan(rn.OP_FWD, 4, 4, dt=3)
    assert plan(rn.OP_FWD, 4, 4, dt=rn.F16)["vec"] == 1


@pytest.mark.parametrize("M,N", [(4096, 4096), (1024, 8192), (16384, 7168), (262144, 128), (33, 5000), (7, 4097),
                                 (4, 40960), (2048, 32768)])
def test_binary16_plans_are_the_bf16_plans(M, N):
    """binary16 has bf16's element size, so every op gets the same plan."""
    ops = [rn.OP_FWD, rn.OP_FUSED_ADD_FWD, rn.OP_BWD, rn.OP_FUSED_ADD_BWD, rn.OP_FWD_FP8, rn.OP_FUSED_ADD_FWD_FP8,
           rn.OP_LN_FWD, rn.OP_LN_FUSED_ADD_FWD, rn.OP_LN_BWD, rn.OP_LN_FUSED_ADD_BWD]
    for op in ops:
        for vec_ok in (True, False):
            assert plan(op, M, N, rn.F16, vec_ok) == plan(op, M, N, rn.BF16, vec_ok), (op, vec_ok)


def test_override_round_trip():
    base = plan(rn.OP_BWD, 4096, 2048)
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=1, team=0, threads=512, grid=100):
        p = plan(rn.OP_BWD, 4096, 2048)
        assert (p["vec"], p["team"], p["threads"], p["chunks"], p["depth"], p["grid"]) == (1, 0, 512, 4, 1, 100)
        assert p["workspace_bytes"] == 100 * 2048 * 4 + 4096 * 4
    assert plan(rn.OP_BWD, 4096, 2048) == base
    # with w in registers, two chunks per lane are compiled for at most 512 threads;
    # with gamma re-read per row, for 1024
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=1024, w_regs=1):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_BWD, 100, 16384)
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=1024, w_regs=0):
        p = plan(rn.OP_BWD, 4096, 16384)
        assert (p["chunks"], p["depth"], p["w_regs"]) == (2, 1, 0)
    # an unset w_regs takes the selector's (1 here), or the other one when only
    # that one is compiled for the layout (two chunks, no prefetch)
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=0):
        p = plan(rn.OP_BWD, 100, 8192)
        assert (p["chunks"], p["depth"], p["w_regs"]) == (2, 0, 0)
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=0, w_regs=1):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_BWD, 100, 8192)
    # the fused op's bound for four chunks without prefetch is 512 threads
    with rn.plan_override(rn.OP_FUSED_ADD_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=1024, depth=0):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_FUSED_ADD_BWD, 100, 32768)
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=1024, depth=0):
        assert plan(rn.OP_BWD, 100, 32768)["chunks"] == 4
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=3):
        assert plan(rn.OP_BWD, 100, 4096)["depth"] == 3
    with rn.plan_override(rn.OP_BWD, path=rn.PATH_ROWS, vec=8, team=0, threads=512, depth=4):
        with pytest.raises(rn.RMSNormError):  # no such depth compiled
            plan(rn.OP_BWD, 100, 4096)
    with rn.plan_override(rn.OP_FWD, path=rn.PATH_LOOP, vec=8, team=0, threads=256):
        p = plan(rn.OP_FWD, 10, 4096)
        assert p["path"] == rn.PATH_LOOP and p["grid"] == 10
    # an override that cannot hold the row is refused for that call
    with rn.plan_override(rn.OP_FWD, path=rn.PATH_ROWS, vec=8, team=16, threads=256):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_FWD, 10, 4096)
    # 16-byte accesses cannot be forced onto unaligned data
    with rn.plan_override(rn.OP_FWD, path=rn.PATH_ROWS, vec=8, team=64, threads=256):
        with pytest.raises(rn.RMSNormError):
            plan(rn.OP_FWD, 10, 4096, vec_ok=False)


def test_fp8_and_layernorm_forwards_keep_their_own_rules():
    """The RMSNorm forward rule applies to neither the fp8 forward nor
    LayerNorm: each has its own sweep table."""
    M, N = 16384, 6144
    assert plan(rn.OP_FWD, M, N, rn.F32)["threads"] == 768
    assert plan(rn.OP_FWD_FP8, M, N, rn.F32)["chunks"] == 6  # 256 threads
    assert plan(rn.OP_LN_FWD, M, N, rn.BF16)["chunks"] == 6  # 128 threads
    assert plan(rn.OP_FWD_FP8, M, N, rn.BF16)["chunks"] == 3  # 256 threads
    assert plan(rn.OP_FWD, M, N, rn.BF16)["chunks"] == 2


_LOG_SNIPPET = r"""
import sys
sys.path.insert(0, {root!r})
import transformer_normalization_rmsnorm_amd as rn
calls = [
    (rn.OP_BWD, 4096, 4096, rn.BF16, 1), (rn.OP_BWD, 4096, 4096, rn.BF16, 1),   # same key twice
    (rn.OP_BWD, 1024, 4096, rn.BF16, 1),                                        # same key, other M
    (rn.OP_FWD, 4096, 4096, rn.BF16, 1), (rn.OP_FWD, 4096, 4097, rn.BF16, 1),   # N % 8 != 0: per-element
    (rn.OP_FWD, 64, 4096, rn.BF16, 0), (rn.OP_FWD, 64, 4096, rn.BF16, 0),       # unaligned: per-element
    (rn.OP_BWD, 8, 131072, rn.BF16, 1), (rn.OP_LN_BWD, 8, 4096, rn.F32, 1),     # looped; LayerNorm
]
for op, M, N, dt, vec_ok in calls:
    rn.rmsnorm_query_plan(op, M, N, dt, vec_ok=bool(vec_ok), num_cus=256)
"""


def _run_logged(env_value):
    import subprocess
    import sys

    env = dict(os.environ)
    env.pop("RMSNORM_LOG", None)
    if env_value is not None:
        env["RMSNORM_LOG"] = env_value
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _LOG_SNIPPET.format(root=root)], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return [ln for ln in r.stderr.splitlines() if ln.startswith("rmsnorm: ")]


def test_plan_log_once_per_key():
    """RMSNORM_LOG=1: one line per (op, path, access width, dtype, N), the
    fallbacks marked with the reason; nothing without the variable or with 0."""
    lines = _run_logged("1")
    assert len(lines) == 6, "\n".join(lines)
    assert sum("rmsnorm: bwd bf16 N=4096 " in ln for ln in lines) == 1
    assert any("fwd bf16 N=4097" in ln and "N not a multiple" in ln for ln in lines)
    assert any("fwd bf16 N=4096" in ln and "not 16-byte aligned" in ln for ln in lines)
    assert any("bwd bf16 N=131072" in ln and "path=loop" in ln and "fallback: looped rows" in ln for ln in lines)
    assert any(ln.startswith("rmsnorm: ln_bwd f32 N=4096") for ln in lines)
    plain = [ln for ln in lines if "fallback" not in ln]
    assert len(plain) == 3 and all("path=rows" in ln for ln in plain)
    assert _run_logged(None) == [] and _run_logged("0") == []


# The forward layout sweep on MI355X (RMSNorm plain and fused-add, bf16 and
# fp32, N = 2048 ... 32768, 2 ... 64 rows per compute unit; every exact
# workgroup tiling; medians of 7 interleaved rounds on cold buffers).  Below
# 16 rows per compute unit the selector takes the tiling measured fastest at
# each swept point: (dtype, fused, M, N) -> threads.
FWD_SWEPT_LATENCY = [
    ("bf16", False, 512, 2048, 128),
    ("bf16", False, 1024, 2048, 256),
    ("bf16", False, 2048, 2048, 256),
    ("bf16", False, 512, 4096, 128),
    ("bf16", False, 1024, 4096, 256),
    ("bf16", False, 2048, 4096, 64),
    ("bf16", False, 512, 6144, 768),
    ("bf16", False, 1024, 6144, 256),
    ("bf16", False, 2048, 6144, 128),
    ("bf16", False, 512, 8192, 512),
    ("bf16", False, 1024, 8192, 128),
    ("bf16", False, 2048, 8192, 512),
    ("bf16", False, 512, 12288, 384),
    ("bf16", False, 1024, 12288, 192),
    ("bf16", False, 2048, 12288, 768),
    ("bf16", False, 512, 16384, 512),
    ("bf16", False, 1024, 16384, 512),
    ("bf16", False, 2048, 16384, 1024),
    ("bf16", False, 512, 24576, 512),
    ("bf16", False, 1024, 24576, 512),
    ("bf16", False, 2048, 24576, 512),
    ("bf16", False, 512, 32768, 512),
    ("bf16", False, 1024, 32768, 512),
    ("bf16", False, 2048, 32768, 512),
    ("f32", False, 512, 2048, 512),
    ("f32", False, 1024, 2048, 128),
    ("f32", False, 2048, 2048, 64),
    ("f32", False, 512, 4096, 256),
    ("f32", False, 1024, 4096, 128),
    ("f32", False, 2048, 4096, 128),
    ("f32", False, 512, 6144, 384),
    ("f32", False, 1024, 6144, 192),
    ("f32", False, 2048, 6144, 768),
    ("f32", False, 512, 8192, 256),
    ("f32", False, 1024, 8192, 256),
    ("f32", False, 2048, 8192, 1024),
    ("f32", False, 512, 12288, 384),
    ("f32", False, 1024, 12288, 512),
    ("f32", False, 2048, 12288, 512),
    ("f32", False, 512, 16384, 512),
    ("f32", False, 1024, 16384, 512),
    ("f32", False, 2048, 16384, 512),
    ("bf16", True, 512, 2048, 64),
    ("bf16", True, 1024, 2048, 128),
    ("bf16", True, 2048, 2048, 64),
    ("bf16", True, 512, 4096, 64),
    ("bf16", True, 1024, 4096, 128),
    ("bf16", True, 2048, 4096, 64),
    ("bf16", True, 512, 8192, 512),
    ("bf16", True, 1024, 8192, 128),
    ("bf16", True, 2048, 8192, 512),
    ("bf16", True, 512, 16384, 256),
    ("bf16", True, 1024, 16384, 256),
    ("bf16", True, 2048, 16384, 1024),
    ("bf16", True, 512, 24576, 512),
    ("bf16", True, 1024, 24576, 512),
    ("bf16", True, 2048, 24576, 384),
]
# From 16 rows per compute unit it takes two chunks per lane where that tiles
# exactly within 1024 threads, else the fewest chunks whose tiling fits.
FWD_SWEPT_THROUGHPUT = [
    ("bf16", False, 4096, 2048),
    ("bf16", False, 8192, 2048),
    ("bf16", False, 16384, 2048),
    ("bf16", False, 4096, 4096),
    ("bf16", False, 8192, 4096),
    ("bf16", False, 16384, 4096),
    ("bf16", False, 4096, 6144),
    ("bf16", False, 8192, 6144),
    ("bf16", False, 16384, 6144),
    ("bf16", False, 4096, 8192),
    ("bf16", False, 8192, 8192),
    ("bf16", False, 16384, 8192),
    ("bf16", False, 4096, 12288),
    ("bf16", False, 8192, 12288),
    ("bf16", False, 16384, 12288),
    ("bf16", False, 4096, 16384),
    ("bf16", False, 8192, 16384),
    ("bf16", False, 16384, 16384),
    ("bf16", False, 4096, 24576),
    ("bf16", False, 8192, 24576),
    ("bf16", False, 4096, 32768),
    ("bf16", False, 8192, 32768),
    ("f32", False, 4096, 2048),
    ("f32", False, 8192, 2048),
    ("f32", False, 16384, 2048),
    ("f32", False, 4096, 4096),
    ("f32", False, 8192, 4096),
    ("f32", False, 16384, 4096),
    ("f32", False, 4096, 6144),
    ("f32", False, 8192, 6144),
    ("f32", False, 16384, 6144),
    ("f32", False, 4096, 8192),
    ("f32", False, 8192, 8192),
    ("f32", False, 16384, 8192),
    ("f32", False, 4096, 12288),
    ("f32", False, 8192, 12288),
    ("f32", False, 4096, 16384),
    ("f32", False, 8192, 16384),
    ("bf16", True, 4096, 2048),
    ("bf16", True, 8192, 2048),
    ("bf16", True, 16384, 2048),
    ("bf16", True, 4096, 4096),
    ("bf16", True, 8192, 4096),
    ("bf16", True, 16384, 4096),
    ("bf16", True, 4096, 8192),
    ("bf16", True, 8192, 8192),
    ("bf16", True, 16384, 8192),
    ("bf16", True, 4096, 16384),
    ("bf16", True, 8192, 16384),
    ("bf16", True, 16384, 16384),
    ("bf16", True, 4096, 24576),
    ("bf16", True, 8192, 24576),
]


def _fewest_chunks_tiling(nchunks):
    for k in (2, 3, 4, 6, 8):
        t = nchunks // k
        if nchunks % k == 0 and t % 64 == 0 and t <= (1024 if k <= 2 else 512):
            return t, k
    raise AssertionError(nchunks)


@pytest.mark.parametrize("dt,fused,M,N,threads", FWD_SWEPT_LATENCY,
                         ids=[f"{d}{'_fused' if f else ''}_{m}x{n}" for d, f, m, n, _ in FWD_SWEPT_LATENCY])
def test_forward_plan_latency_regime(dt, fused, M, N, threads):
    p = plan(rn.OP_FUSED_ADD_FWD if fused else rn.OP_FWD, M, N, rn.BF16 if dt == "bf16" else rn.F32)
    V = 8 if dt == "bf16" else 4
    assert (p["team"], p["threads"], p["chunks"]) == (0, threads, N // V // threads), p


@pytest.mark.parametrize("dt,fused,M,N", FWD_SWEPT_THROUGHPUT,
                         ids=[f"{d}{'_fused' if f else ''}_{m}x{n}" for d, f, m, n in FWD_SWEPT_THROUGHPUT])
def test_forward_plan_throughput_regime(dt, fused, M, N):
    p = plan(rn.OP_FUSED_ADD_FWD if fused else rn.OP_FWD, M, N, rn.BF16 if dt == "bf16" else rn.F32)
    V = 8 if dt == "bf16" else 4
    assert (p["threads"], p["chunks"]) == _fewest_chunks_tiling(N // V), p


def test_forward_plan_24576_takes_six_chunks():
    """bf16 4096 x 24576: 512 threads x 6 chunks (66.7 us measured against 74.1 us for 384 x 8)."""
    p = plan(rn.OP_FWD, 4096, 24576, rn.BF16)
    assert (p["threads"], p["chunks"]) == (512, 6)


# LayerNorm forward sweep on MI355X (every exact workgroup tiling, cold rotating
# buffers, medians of 3 interleaved rounds): per point (storage, fused-add, M,
# N), the chunks per lane whose layout came within 3% of the fastest.  M = 256
# x rows per compute unit.
LN_FWD_SWEPT = [
    ('bf16', False, 512, 2048, (2,)),
    ('bf16', False, 1024, 2048, (2,)),
    ('bf16', False, 2048, 2048, (2, 4)),
    ('bf16', False, 4096, 2048, (2, 4)),
    ('bf16', False, 8192, 2048, (2, 4)),
    ('bf16', False, 16384, 2048, (2, 4)),
    ('bf16', False, 512, 4096, (1, 2)),
    ('bf16', False, 1024, 4096, (2, 4)),
    ('bf16', False, 2048, 4096, (2, 4, 8)),
    ('bf16', False, 4096, 4096, (2, 4)),
    ('bf16', False, 8192, 4096, (2, 4)),
    ('bf16', False, 16384, 4096, (2, 4, 8)),
    ('bf16', False, 512, 6144, (1, 3)),
    ('bf16', False, 1024, 6144, (3, 4, 6)),
    ('bf16', False, 2048, 6144, (2, 3, 4, 6)),
    ('bf16', False, 4096, 6144, (2, 3, 4, 6)),
    ('bf16', False, 8192, 6144, (3, 4, 6)),
    ('bf16', False, 16384, 6144, (4, 6)),
    ('bf16', False, 512, 8192, (2, 4)),
    ('bf16', False, 1024, 8192, (8,)),
    ('bf16', False, 2048, 8192, (2, 4)),
    ('bf16', False, 4096, 8192, (4,)),
    ('bf16', False, 8192, 8192, (2, 4, 8)),
    ('bf16', False, 16384, 8192, (4, 8)),
    ('bf16', False, 512, 12288, (6,)),
    ('bf16', False, 1024, 12288, (8,)),
    ('bf16', False, 2048, 12288, (3, 6)),
    ('bf16', False, 4096, 12288, (3, 6, 8)),
    ('bf16', False, 8192, 12288, (3, 8)),
    ('bf16', False, 16384, 12288, (8,)),
    ('bf16', False, 512, 16384, (4, 8)),
    ('bf16', False, 1024, 16384, (4, 8)),
    ('bf16', False, 2048, 16384, (8,)),
    ('bf16', False, 4096, 16384, (8,)),
    ('bf16', False, 8192, 16384, (4, 8)),
    ('bf16', False, 16384, 16384, (2, 4, 8)),
    ('bf16', False, 512, 24576, (6, 8)),
    ('bf16', False, 1024, 24576, (6,)),
    ('bf16', False, 2048, 24576, (6,)),
    ('bf16', False, 4096, 24576, (6,)),
    ('bf16', False, 8192, 24576, (6,)),
    ('bf16', False, 512, 32768, (8,)),
    ('bf16', False, 1024, 32768, (8,)),
    ('bf16', False, 2048, 32768, (8,)),
    ('bf16', False, 4096, 32768, (8,)),
    ('bf16', False, 8192, 32768, (8,)),
    ('bf16', True, 512, 2048, (1, 2)),
    ('bf16', True, 1024, 2048, (2,)),
    ('bf16', True, 2048, 2048, (4,)),
    ('bf16', True, 4096, 2048, (1, 2, 4)),
    ('bf16', True, 8192, 2048, (1,)),
    ('bf16', True, 16384, 2048, (1, 2, 4)),
    ('bf16', True, 512, 4096, (1, 2, 4)),
    ('bf16', True, 1024, 4096, (2, 4)),
    ('bf16', True, 2048, 4096, (1, 4, 8)),
    ('bf16', True, 4096, 4096, (1, 2, 4)),
    ('bf16', True, 8192, 4096, (1, 2, 4)),
    ('bf16', True, 16384, 4096, (1,)),
    ('bf16', True, 512, 8192, (1, 4)),
    ('bf16', True, 1024, 8192, (4, 8)),
    ('bf16', True, 2048, 8192, (1, 2, 4)),
    ('bf16', True, 4096, 8192, (1, 2, 4)),
    ('bf16', True, 8192, 8192, (1, 4, 8)),
    ('bf16', True, 16384, 8192, (1, 4, 8)),
    ('bf16', True, 512, 16384, (8,)),
    ('bf16', True, 1024, 16384, (8,)),
    ('bf16', True, 2048, 16384, (2, 4, 8)),
    ('bf16', True, 4096, 16384, (2, 4, 8)),
    ('bf16', True, 8192, 16384, (2, 4, 8)),
    ('bf16', True, 16384, 16384, (2, 4, 8)),
    ('bf16', True, 512, 24576, (6, 8)),
    ('bf16', True, 1024, 24576, (6,)),
    ('bf16', True, 2048, 24576, (6, 8)),
    ('bf16', True, 4096, 24576, (6,)),
    ('bf16', True, 8192, 24576, (6,)),
    ('f32', False, 512, 2048, (2,)),
    ('f32', False, 1024, 2048, (8,)),
    ('f32', False, 2048, 2048, (8,)),
    ('f32', False, 4096, 2048, (8,)),
    ('f32', False, 8192, 2048, (2, 4, 8)),
    ('f32', False, 16384, 2048, (2, 4, 8)),
    ('f32', False, 512, 4096, (4,)),
    ('f32', False, 1024, 4096, (8,)),
    ('f32', False, 2048, 4096, (4, 8)),
    ('f32', False, 4096, 4096, (2, 8)),
    ('f32', False, 8192, 4096, (2, 4, 8)),
    ('f32', False, 16384, 4096, (2, 4, 8)),
    ('f32', False, 512, 6144, (8,)),
    ('f32', False, 1024, 6144, (6, 8)),
    ('f32', False, 2048, 6144, (2, 6)),
    ('f32', False, 4096, 6144, (2, 6)),
    ('f32', False, 8192, 6144, (2,)),
    ('f32', False, 16384, 6144, (2,)),
    ('f32', False, 512, 8192, (8,)),
    ('f32', False, 1024, 8192, (8,)),
    ('f32', False, 2048, 8192, (8,)),
    ('f32', False, 4096, 8192, (8,)),
    ('f32', False, 8192, 8192, (2, 4, 8)),
    ('f32', False, 16384, 8192, (2,)),
    ('f32', False, 512, 12288, (8,)),
    ('f32', False, 1024, 12288, (6,)),
    ('f32', False, 2048, 12288, (6,)),
    ('f32', False, 4096, 12288, (6,)),
    ('f32', False, 8192, 12288, (6,)),
    ('f32', False, 512, 16384, (8,)),
    ('f32', False, 1024, 16384, (8,)),
    ('f32', False, 2048, 16384, (8,)),
    ('f32', False, 4096, 16384, (8,)),
    ('f32', False, 8192, 16384, (8,)),
]


@pytest.mark.parametrize("dt,fused,M,N,ok", LN_FWD_SWEPT,
                         ids=[f"{d}{'_fused' if f else ''}_{m}x{n}" for d, f, m, n, _ in LN_FWD_SWEPT])
def test_layernorm_forward_plan_at_swept_points(dt, fused, M, N, ok):
    p = plan(rn.OP_LN_FUSED_ADD_FWD if fused else rn.OP_LN_FWD, M, N, rn.BF16 if dt == "bf16" else rn.F32)
    V = 8 if dt == "bf16" else 4
    assert p["path"] == rn.PATH_ROWS and p["team"] == 0 and p["depth"] == 0
    assert p["threads"] * p["chunks"] * V == N
    assert p["chunks"] in ok, (p["threads"], p["chunks"], ok)


# fp8-output forward sweep on MI355X, as the LayerNorm one above.
F8_FWD_SWEPT = [
    ('bf16', False, 512, 2048, (1, 2, 4)),
    ('bf16', False, 1024, 2048, (2,)),
    ('bf16', False, 2048, 2048, (1, 4)),
    ('bf16', False, 4096, 2048, (2,)),
    ('bf16', False, 8192, 2048, (2, 4)),
    ('bf16', False, 16384, 2048, (2, 4)),
    ('bf16', False, 512, 4096, (2,)),
    ('bf16', False, 1024, 4096, (2, 4, 8)),
    ('bf16', False, 2048, 4096, (2, 4)),
    ('bf16', False, 4096, 4096, (4, 8)),
    ('bf16', False, 8192, 4096, (4, 8)),
    ('bf16', False, 16384, 4096, (4, 8)),
    ('bf16', False, 512, 6144, (1, 4, 6)),
    ('bf16', False, 1024, 6144, (2, 3, 6)),
    ('bf16', False, 2048, 6144, (3, 4)),
    ('bf16', False, 4096, 6144, (3, 4)),
    ('bf16', False, 8192, 6144, (3, 4, 6)),
    ('bf16', False, 16384, 6144, (3, 4)),
    ('bf16', False, 512, 8192, (1, 2, 4)),
    ('bf16', False, 1024, 8192, (2, 4)),
    ('bf16', False, 2048, 8192, (4,)),
    ('bf16', False, 4096, 8192, (4, 8)),
    ('bf16', False, 8192, 8192, (4, 8)),
    ('bf16', False, 16384, 8192, (4, 8)),
    ('bf16', False, 512, 12288, (6,)),
    ('bf16', False, 1024, 12288, (8,)),
    ('bf16', False, 2048, 12288, (6, 8)),
    ('bf16', False, 4096, 12288, (8,)),
    ('bf16', False, 8192, 12288, (8,)),
    ('bf16', False, 16384, 12288, (8,)),
    ('bf16', False, 512, 16384, (4, 8)),
    ('bf16', False, 1024, 16384, (8,)),
    ('bf16', False, 2048, 16384, (8,)),
    ('bf16', False, 4096, 16384, (8,)),
    ('bf16', False, 8192, 16384, (8,)),
    ('bf16', False, 16384, 16384, (8,)),
    ('bf16', False, 512, 24576, (8,)),
    ('bf16', False, 1024, 24576, (6, 8)),
    ('bf16', False, 2048, 24576, (8,)),
    ('bf16', False, 4096, 24576, (8,)),
    ('bf16', False, 8192, 24576, (8,)),
    ('bf16', False, 512, 32768, (8,)),
    ('bf16', False, 1024, 32768, (8,)),
    ('bf16', False, 2048, 32768, (8,)),
    ('bf16', False, 4096, 32768, (8,)),
    ('bf16', False, 8192, 32768, (8,)),
    ('bf16', True, 512, 2048, (1, 4)),
    ('bf16', True, 1024, 2048, (2,)),
    ('bf16', True, 2048, 2048, (4,)),
    ('bf16', True, 4096, 2048, (2, 4)),
    ('bf16', True, 8192, 2048, (1, 2, 4)),
    ('bf16', True, 16384, 2048, (1, 2, 4)),
    ('bf16', True, 512, 4096, (1, 2)),
    ('bf16', True, 1024, 4096, (2, 4, 8)),
    ('bf16', True, 2048, 4096, (2, 4, 8)),
    ('bf16', True, 4096, 4096, (2, 4)),
    ('bf16', True, 8192, 4096, (2, 4)),
    ('bf16', True, 16384, 4096, (2, 4)),
    ('bf16', True, 512, 8192, (2, 4)),
    ('bf16', True, 1024, 8192, (2, 4)),
    ('bf16', True, 2048, 8192, (2, 4)),
    ('bf16', True, 4096, 8192, (2, 4)),
    ('bf16', True, 8192, 8192, (2, 4)),
    ('bf16', True, 16384, 8192, (2, 4)),
    ('bf16', True, 512, 16384, (8,)),
    ('bf16', True, 1024, 16384, (2, 4, 8)),
    ('bf16', True, 2048, 16384, (2, 4, 8)),
    ('bf16', True, 4096, 16384, (2, 4, 8)),
    ('bf16', True, 8192, 16384, (2, 4, 8)),
    ('bf16', True, 16384, 16384, (2, 4, 8)),
    ('bf16', True, 512, 24576, (6,)),
    ('bf16', True, 1024, 24576, (6,)),
    ('bf16', True, 2048, 24576, (6,)),
    ('bf16', True, 4096, 24576, (6,)),
    ('bf16', True, 8192, 24576, (6,)),
    ('f32', False, 512, 2048, (1, 4, 8)),
    ('f32', False, 1024, 2048, (1, 2)),
    ('f32', False, 2048, 2048, (8,)),
    ('f32', False, 4096, 2048, (4, 8)),
    ('f32', False, 8192, 2048, (4, 8)),
    ('f32', False, 16384, 2048, (4, 8)),
    ('f32', False, 512, 4096, (2, 4)),
    ('f32', False, 1024, 4096, (8,)),
    ('f32', False, 2048, 4096, (4, 8)),
    ('f32', False, 4096, 4096, (4, 8)),
    ('f32', False, 8192, 4096, (4, 8)),
    ('f32', False, 16384, 4096, (4, 8)),
    ('f32', False, 512, 6144, (6, 8)),
    ('f32', False, 1024, 6144, (6, 8)),
    ('f32', False, 2048, 6144, (6, 8)),
    ('f32', False, 4096, 6144, (6, 8)),
    ('f32', False, 8192, 6144, (6, 8)),
    ('f32', False, 16384, 6144, (6, 8)),
    ('f32', False, 512, 8192, (8,)),
    ('f32', False, 1024, 8192, (8,)),
    ('f32', False, 2048, 8192, (8,)),
    ('f32', False, 4096, 8192, (8,)),
    ('f32', False, 8192, 8192, (8,)),
    ('f32', False, 16384, 8192, (8,)),
    ('f32', False, 512, 12288, (6, 8)),
    ('f32', False, 1024, 12288, (6,)),
    ('f32', False, 2048, 12288, (6,)),
    ('f32', False, 4096, 12288, (6,)),
    ('f32', False, 8192, 12288, (6,)),
    ('f32', False, 512, 16384, (8,)),
    ('f32', False, 1024, 16384, (8,)),
    ('f32', False, 2048, 16384, (8,)),
    ('f32', False, 4096, 16384, (8,)),
    ('f32', False, 8192, 16384, (8,)),
]


@pytest.mark.parametrize("dt,fused,M,N,ok", F8_FWD_SWEPT,
                         ids=[f"{d}{'_fused' if f else ''}_{m}x{n}" for d, f, m, n, _ in F8_FWD_SWEPT])
def test_fp8_forward_plan_at_swept_points(dt, fused, M, N, ok):
    p = plan(rn.OP_FUSED_ADD_FWD_FP8 if fused else rn.OP_FWD_FP8, M, N, rn.BF16 if dt == "bf16" else rn.F32)
    V = 8 if dt == "bf16" else 4
    assert p["path"] == rn.PATH_ROWS and p["team"] == 0 and p["depth"] == 0
    assert p["threads"] * p["chunks"] * V == N
    assert p["chunks"] in ok, (p["threads"], p["chunks"], ok)


@pytest.mark.parametrize("dt,N", [(rn.BF16, 12288), (rn.BF16, 16384), (rn.F32, 6144), (rn.F32, 8192)])
@pytest.mark.parametrize("op", [rn.OP_BWD, rn.OP_FUSED_ADD_BWD, rn.OP_LN_BWD, rn.OP_LN_FUSED_ADD_BWD])
def test_wide_backward_without_lookahead_at_two_rows_per_program(op, dt, N):
    """Rows with gamma re-read per row take no row ahead when each program has
    at most two rows (measured faster on MI355X), and keep it from three."""
    programs = 256
    for M, depth in ((2 * programs, 0), (2 * programs - 7, 0), (programs, 0), (2 * programs + 1, 1), (4 * programs, 1)):
        p = plan(op, M, N, dt)
        assert p["w_regs"] == 0 and (p["depth"] == 0) == (depth == 0), (M, p)
