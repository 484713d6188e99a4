"""Python binding of the gfx950 RMSNorm library (``librmsnorm_amd.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/rmsnorm.h``.  PyTorch supplies
device memory (``torch.empty``) and the current stream; nothing here computes.
If the library has not been built, importing works but every call raises.
Tensors are bfloat16, float16 or float32 (one dtype per call; rstd, mean,
scale and amax are float32); arithmetic is float32 for every dtype.

Functions mirror the C entry points:
  rmsnorm_fwd(x, gamma, eps, offset)                    -> (y, rstd)
  rmsnorm_fused_add_fwd(x, residual, gamma, eps, offset) -> (y, h, rstd)
  rmsnorm_bwd(dy, x, gamma, rstd, eps, offset)          -> (dx, dgamma)
  rmsnorm_fused_add_bwd(dy, dh, h, gamma, rstd, eps, offset) -> (dx, dgamma)
  rmsnorm_bwd_partials / rmsnorm_dgamma_finalize        (the two backward stages)
  rmsnorm_fwd_fp8(x, gamma, scale, eps, offset, amax=)  -> (y8, rstd)   (E4M3 output)
  rmsnorm_fused_add_fwd_fp8(x, residual, gamma, scale, eps, offset, amax=) -> (y8, h, rstd)
  rmsnorm_bwd_workspace_bytes, rmsnorm_fwd_fp8_workspace_bytes,
  rmsnorm_query_plan, rmsnorm_set_plan_override
  layernorm_fwd(x, gamma, beta, eps, offset)            -> (y, mean, rstd)
  layernorm_fused_add_fwd(x, residual, gamma, beta, ...) -> (y, h, mean, rstd)
  layernorm_bwd(dy, x, gamma, mean, rstd, ...)          -> (dx, dgamma, dbeta)
  layernorm_fused_add_bwd(dy, dh, h, gamma, mean, rstd, ...) -> (dx, dgamma, dbeta)
  layernorm_bwd_workspace_bytes
"""

from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(PKG_DIR, "librmsnorm_amd.so")

F32, BF16, F16 = 0, 1, 2
OP_FWD, OP_FUSED_ADD_FWD, OP_BWD, OP_FUSED_ADD_BWD, OP_FWD_FP8, OP_FUSED_ADD_FWD_FP8 = 0, 1, 2, 3, 4, 5
OP_LN_FWD, OP_LN_FUSED_ADD_FWD, OP_LN_BWD, OP_LN_FUSED_ADD_BWD = 6, 7, 8, 9
PATH_ROWS, PATH_LOOP, PATH_ROWS_COLS = 0, 1, 2
MAX_N = 1 << 24  # longest row any entry point accepts (RMSNORM_MAX_N)
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}

# Exported symbols (kept equal to include/rmsnorm.h; a CPU test checks both).
EXPORTS = (
    "rmsnorm_fwd", "rmsnorm_fused_add_fwd", "rmsnorm_bwd_workspace_bytes", "rmsnorm_bwd",
    "rmsnorm_fused_add_bwd", "rmsnorm_bwd_partials", "rmsnorm_dgamma_finalize", "rmsnorm_query_plan",
    "rmsnorm_set_plan_override", "rmsnorm_status_string", "rmsnorm_last_error", "rmsnorm_version",
    "rmsnorm_fwd_fp8", "rmsnorm_fused_add_fwd_fp8", "rmsnorm_fwd_fp8_workspace_bytes",
    "layernorm_fwd", "layernorm_fused_add_fwd", "layernorm_bwd_workspace_bytes", "layernorm_bwd",
    "layernorm_fused_add_bwd", "rmsnorm_bwd_noalloc",
)


class RMSNormError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} failed: {STATUS.get(status, status)} ({detail})")
        self.status = status


# RMSNORM_ABI_VERSION of include/rmsnorm.h that this binding marshals.
ABI_VERSION = 8


class Plan(ctypes.Structure):
    _fields_ = [
        ("op", ctypes.c_int32), ("path", ctypes.c_int32), ("vec", ctypes.c_int32), ("team", ctypes.c_int32),
        ("threads", ctypes.c_int32), ("chunks", ctypes.c_int32), ("depth", ctypes.c_int32),
        ("w_regs", ctypes.c_int32), ("grid", ctypes.c_int64),
        ("programs", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64), ("fin_threads", ctypes.c_int32),
        ("fin_grid", ctypes.c_int64), ("rows_per_step", ctypes.c_int32), ("col_chunks", ctypes.c_int32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def _bind(lib):
    vp, i64, f, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    sig = {
        "rmsnorm_fwd": [vp, vp, vp, vp, i64, i64, f, f, i32, vp],
        "rmsnorm_fused_add_fwd": [vp, vp, vp, vp, vp, vp, i64, i64, f, f, i32, vp],
        "rmsnorm_bwd_workspace_bytes": [i64, i64, i32, ctypes.POINTER(sz)],
        "rmsnorm_bwd": [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f, f, i32, vp],
        "rmsnorm_bwd_noalloc": [vp, vp, vp, vp, vp, vp, i64, i64, f, f, i32, vp],
        "rmsnorm_fused_add_bwd": [vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f, f, i32, vp],
        "rmsnorm_bwd_partials": [vp, vp, vp, vp, vp, vp, vp, sz, ctypes.POINTER(i64), i64, i64, f, f, i32, vp],
        "rmsnorm_dgamma_finalize": [vp, i64, i64, vp, i32, vp],
        "rmsnorm_query_plan": [i32, i64, i64, i32, i32, i32, ctypes.POINTER(Plan)],
        "rmsnorm_set_plan_override": [i32, ctypes.POINTER(Plan)],
        "rmsnorm_status_string": [i32],
        "rmsnorm_last_error": [],
        "rmsnorm_version": [],
        "rmsnorm_fwd_fp8": [vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f, f, i32, vp],
        "rmsnorm_fused_add_fwd_fp8": [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f, f, i32, vp],
        "rmsnorm_fwd_fp8_workspace_bytes": [i64, i64, i32, ctypes.POINTER(sz)],
        "layernorm_fwd": [vp, vp, vp, vp, vp, vp, i64, i64, f, f, i32, vp],
        "layernorm_fused_add_fwd": [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, f, f, i32, vp],
        "layernorm_bwd_workspace_bytes": [i64, i64, i32, ctypes.POINTER(sz)],
        "layernorm_bwd": [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f, f, i32, vp],
        "layernorm_fused_add_bwd": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i64, i64, f, f, i32, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("rmsnorm_status_string", "rmsnorm_last_error") else ctypes.c_int
    return lib


def library_path() -> str:
    return LIBRARY_PATH


def load_library():
    """Load the built C library; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY_PATH):
            raise RuntimeError(
                f"{LIBRARY_PATH} is not built; run `python -m transformer_normalization_rmsnorm_amd._build` "
                "(or __graft_entry__.build()) first")
        lib = _bind(ctypes.CDLL(LIBRARY_PATH))
        if lib.rmsnorm_version() != ABI_VERSION:
            raise RuntimeError(f"{LIBRARY_PATH} has ABI version {lib.rmsnorm_version()}, this binding "
                               f"expects {ABI_VERSION}; rebuild the library")
        _lib = lib
    return _lib


def _check(rc: int, func: str):
    if rc != 0:
        detail = load_library().rmsnorm_last_error().decode(errors="replace")
        raise RMSNormError(rc, func, detail)


# ---- torch marshalling --------------------------------------------------------

_torch_mod = None
_raw_stream = None


def _torch():
    global _torch_mod, _raw_stream
    if _torch_mod is None:
        import torch

        # the current stream of a device as a raw handle, without building a
        # Stream object per call (falls back to the public API)
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _torch_mod = torch
    return _torch_mod


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _require(t, name, shape=None, dtype=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if device is not None:
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
    elif not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _rows(x):
    if x.dim() < 1:
        raise ValueError("input must have at least one dimension")
    N = x.shape[-1]
    M = x.numel() // N if N else 0
    return M, N


def _stream_handle(index: int) -> int:
    """The caller's current stream on device `index` (what torch launches on)."""
    torch = _torch()
    if _raw_stream is not None:
        return _raw_stream(index)
    return torch.cuda.current_stream(index).cuda_stream


def _launch(dev, name: str, *args):
    """Call entry point `name` with the current stream of the tensors' device
    appended, entering that device only when it is not already current."""
    torch = _torch()
    fn = getattr(load_library(), name)
    idx = dev.index
    if torch.cuda.current_device() == idx:
        rc = fn(*args, _stream_handle(idx))
    else:
        with torch.cuda.device(idx):
            rc = fn(*args, _stream_handle(idx))
    _check(rc, name)


def _on_device_call(dev, f):
    """f() with the tensors' device current (host queries that read it)."""
    torch = _torch()
    if torch.cuda.current_device() == dev.index:
        return f()
    with torch.cuda.device(dev.index):
        return f()


# Backward workspace sizes by (op family, M, N, dtype, device): they depend only
# on those and the device's compute-unit count.  Ops with a forced plan
# (rmsnorm_set_plan_override) are sized from their plans instead.
_ws_cache: dict = {}
_overridden: set = set()


def _bwd_workspace(family: str, M: int, N: int, code: int, dev, ops):
    torch = _torch()
    key = (family, M, N, code, dev.index)
    nbytes = _ws_cache.get(key)
    if nbytes is None:
        query = rmsnorm_bwd_workspace_bytes if family == "rms" else layernorm_bwd_workspace_bytes
        nbytes = _on_device_call(dev, lambda: query(M, N, code))
        if len(_ws_cache) > 4096:
            _ws_cache.clear()
        _ws_cache[key] = nbytes
    if _overridden.intersection(ops):
        def planned():
            nb = nbytes
            for op in ops:
                for vec_ok in (True, False):
                    try:
                        nb = max(nb, rmsnorm_query_plan(op, M, N, code, vec_ok)["workspace_bytes"])
                    except RMSNormError:
                        pass  # a forced vector layout has no unaligned plan
            return nb
        nbytes = _on_device_call(dev, planned)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev), nbytes


def rmsnorm_fwd(x, gamma, eps: float = 1e-6, offset: float = 0.0, *, y=None, rstd=None, save_rstd: bool = True):
    """y = x * rstd * (gamma + offset) over the last dimension; returns (y, rstd).
    gamma None: the non-affine op (offset must be 0)."""
    torch = _torch()
    _require(x, "x")
    M, N = _rows(x)
    dev = x.device
    if gamma is not None:
        _require(gamma, "gamma", (N,), x.dtype, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _require(y, "y", x.shape, x.dtype, dev)
    if rstd is None:
        if save_rstd:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    else:
        _require(rstd, "rstd", x.shape[:-1], torch.float32, dev)
    _launch(dev, "rmsnorm_fwd", _ptr(x), _ptr(gamma), _ptr(y), _ptr(rstd), M, N, eps, offset, _dtype_code(x))
    return y, rstd


def rmsnorm_fused_add_fwd(x, residual, gamma, eps: float = 1e-6, offset: float = 0.0, *, y=None, h_out=None,
                          rstd=None, save_rstd: bool = True):
    """h = x + residual (rounded to the storage dtype), y = rmsnorm(h); returns (y, h, rstd).

    Pass h_out=residual to update the residual stream in place."""
    torch = _torch()
    _require(x, "x")
    M, N = _rows(x)
    dev = x.device
    _require(residual, "residual", x.shape, x.dtype, dev)
    if gamma is not None:
        _require(gamma, "gamma", (N,), x.dtype, dev)
    if y is None:
        y = torch.empty_like(x)
    else:
        _require(y, "y", x.shape, x.dtype, dev)
    if h_out is None:
        h_out = torch.empty_like(x)
    else:
        _require(h_out, "h_out", x.shape, x.dtype, dev)
    if rstd is None:
        if save_rstd:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    else:
        _require(rstd, "rstd", x.shape[:-1], torch.float32, dev)
    _launch(dev, "rmsnorm_fused_add_fwd", _ptr(x), _ptr(residual), _ptr(gamma), _ptr(y), _ptr(h_out), _ptr(rstd),
            M, N, eps, offset, _dtype_code(x))
    return y, h_out, rstd


def rmsnorm_fwd_fp8_workspace_bytes(M: int, N: int, dtype_code: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.rmsnorm_fwd_fp8_workspace_bytes(M, N, dtype_code, ctypes.byref(out)),
           "rmsnorm_fwd_fp8_workspace_bytes")
    return int(out.value)


def _fp8_common(x, residual, gamma, scale, eps, offset, amax, y8, h_out, rstd, save_rstd, workspace):
    torch = _torch()
    _require(x, "x")
    M, N = _rows(x)
    dev = x.device
    fused = residual is not None
    if fused:
        _require(residual, "residual", x.shape, x.dtype, dev)
    if gamma is not None:
        _require(gamma, "gamma", (N,), x.dtype, dev)
    _require(scale, "scale", None, torch.float32, dev)
    if scale.numel() != 1:
        raise ValueError("scale must hold one float32")
    if amax is not None:
        _require(amax, "amax", None, torch.float32, dev)
        if amax.numel() != 1:
            raise ValueError("amax must hold one float32")
    if y8 is None:
        y8 = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev)
    _require(y8, "y8", x.shape, None, dev)
    if y8.element_size() != 1:
        raise ValueError("y8 must be a one-byte tensor (float8_e4m3fn or uint8)")
    if fused and h_out is None:
        h_out = torch.empty_like(x)
    if fused:
        _require(h_out, "h_out", x.shape, x.dtype, dev)
    if rstd is None and save_rstd:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev)
    if rstd is not None:
        _require(rstd, "rstd", x.shape[:-1], torch.float32, dev)
    ws_bytes = 0
    if amax is not None:
        if workspace is None:
            ws_bytes = _on_device_call(dev, lambda: rmsnorm_fwd_fp8_workspace_bytes(M, N, _dtype_code(x)))
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    if fused:
        _launch(dev, "rmsnorm_fused_add_fwd_fp8", _ptr(x), _ptr(residual), _ptr(gamma), _ptr(y8), _ptr(h_out),
                _ptr(rstd), _ptr(scale), _ptr(amax), _ptr(workspace), ws_bytes, M, N, eps, offset, _dtype_code(x))
    else:
        _launch(dev, "rmsnorm_fwd_fp8", _ptr(x), _ptr(gamma), _ptr(y8), _ptr(rstd), _ptr(scale), _ptr(amax),
                _ptr(workspace), ws_bytes, M, N, eps, offset, _dtype_code(x))
    return y8, h_out, rstd


def rmsnorm_fwd_fp8(x, gamma, scale, eps: float = 1e-6, offset: float = 0.0, *, amax=None, y8=None, rstd=None,
                    save_rstd: bool = True, workspace=None):
    """y8 = E4M3(x * rstd * (gamma + offset) * scale) (OCP E4M3, nearest even,
    saturating at +-448); returns (y8, rstd).  scale: one float32 on the GPU;
    amax: one float32 on the GPU, updated in place to max(amax, max |y|)."""
    y8, _, rstd = _fp8_common(x, None, gamma, scale, eps, offset, amax, y8, None, rstd, save_rstd, workspace)
    return y8, rstd


def rmsnorm_fused_add_fwd_fp8(x, residual, gamma, scale, eps: float = 1e-6, offset: float = 0.0, *, amax=None,
                              y8=None, h_out=None, rstd=None, save_rstd: bool = True, workspace=None):
    """h = x + residual (rounded to the storage dtype), y8 = E4M3(rmsnorm(h) * scale);
    returns (y8, h, rstd).  h_out=residual updates the residual stream in place."""
    return _fp8_common(x, residual, gamma, scale, eps, offset, amax, y8, h_out, rstd, save_rstd, workspace)


def rmsnorm_bwd_workspace_bytes(M: int, N: int, dtype_code: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.rmsnorm_bwd_workspace_bytes(M, N, dtype_code, ctypes.byref(out)), "rmsnorm_bwd_workspace_bytes")
    return int(out.value)


def alloc_workspace(M: int, N: int, dtype_code: int, device, op: Optional[int] = None):
    """Workspace for a backward call on `device` (the RMSNorm ops; with `op`
    a LayerNorm op, LayerNorm's), also large enough for a plan forced by
    rmsnorm_set_plan_override.  Returns (tensor, bytes)."""
    torch = _torch()
    device = torch.device(device)
    if op in (OP_LN_BWD, OP_LN_FUSED_ADD_BWD):
        return _bwd_workspace("ln", M, N, dtype_code, device, (OP_LN_BWD, OP_LN_FUSED_ADD_BWD))
    return _bwd_workspace("rms", M, N, dtype_code, device, (OP_BWD, OP_FUSED_ADD_BWD))


def _bwd_common(name, dy, dh, v, gamma, rstd, eps, offset, dx, dgamma, workspace):
    torch = _torch()
    _require(v, "x" if dh is None else "h")
    M, N = _rows(v)
    dev = v.device
    _require(dy, "dy", v.shape, v.dtype, dev)
    if dh is not None:
        _require(dh, "dh", v.shape, v.dtype, dev)
    if gamma is not None:
        _require(gamma, "gamma", (N,), v.dtype, dev)
    if rstd is not None:
        _require(rstd, "rstd", v.shape[:-1], torch.float32, dev)
    if dx is None:
        dx = torch.empty_like(v)
    else:
        _require(dx, "dx", v.shape, v.dtype, dev)
    if gamma is not None:
        if dgamma is None:
            dgamma = torch.empty_like(gamma)
        else:
            _require(dgamma, "dgamma", (N,), v.dtype, dev)
    code = _dtype_code(v)
    if workspace is None:
        workspace, nbytes = _bwd_workspace("rms", M, N, code, dev, (OP_BWD, OP_FUSED_ADD_BWD))
    else:
        _require(workspace, "workspace", device=dev)
        nbytes = workspace.numel() * workspace.element_size()
    if name == "rmsnorm_bwd":
        _launch(dev, name, _ptr(dy), _ptr(v), _ptr(gamma), _ptr(rstd), _ptr(dx), _ptr(dgamma), _ptr(workspace),
                nbytes, M, N, eps, offset, code)
    else:
        _launch(dev, name, _ptr(dy), _ptr(dh), _ptr(v), _ptr(gamma), _ptr(rstd), _ptr(dx), _ptr(dgamma),
                _ptr(workspace), nbytes, M, N, eps, offset, code)
    return dx, dgamma


def rmsnorm_bwd(dy, x, gamma, rstd, eps: float = 1e-6, offset: float = 0.0, *, dx=None, dgamma=None,
                workspace=None):
    """Gradients of rmsnorm_fwd; rstd=None recomputes it.  Returns (dx, dgamma);
    dgamma is None for the non-affine op (gamma None)."""
    return _bwd_common("rmsnorm_bwd", dy, None, x, gamma, rstd, eps, offset, dx, dgamma, workspace)


def rmsnorm_fused_add_bwd(dy, dh, h, gamma, rstd, eps: float = 1e-6, offset: float = 0.0, *, dx=None,
                          dgamma=None, workspace=None):
    """Gradients of rmsnorm_fused_add_fwd: dx (= dresidual) and dgamma.  dh may be None;
    pass dx=dh to accumulate in place."""
    return _bwd_common("rmsnorm_fused_add_bwd", dy, dh, h, gamma, rstd, eps, offset, dx, dgamma, workspace)


def rmsnorm_bwd_partials(dy, v, gamma, rstd, dh=None, eps: float = 1e-6, offset: float = 0.0, *, dx=None,
                         workspace=None):
    """First backward stage: returns (dx, workspace, programs); the float32 partials
    are workspace.view(float32)[: programs * ld] with ld = N rounded up to 64."""
    torch = _torch()
    M, N = _rows(v)
    dev = v.device
    if dx is None:
        dx = torch.empty_like(v)
    if workspace is None:
        workspace, nbytes = _bwd_workspace("rms", M, N, _dtype_code(v), dev, (OP_BWD, OP_FUSED_ADD_BWD))
    else:
        nbytes = workspace.numel() * workspace.element_size()
    programs = ctypes.c_int64(0)
    _launch(dev, "rmsnorm_bwd_partials", _ptr(dy), _ptr(v), _ptr(gamma), _ptr(rstd), _ptr(dh), _ptr(dx),
            _ptr(workspace), nbytes, ctypes.byref(programs), M, N, eps, offset, _dtype_code(v))
    return dx, workspace, int(programs.value)


def rmsnorm_dgamma_finalize(partials, programs: int, N: int, dgamma):
    """Second backward stage: dgamma = fixed-order sum of `programs` partial rows."""
    _launch(dgamma.device, "rmsnorm_dgamma_finalize", _ptr(partials), programs, N, _ptr(dgamma),
            _dtype_code(dgamma))
    return dgamma


def partial_ld(N: int) -> int:
    return (N + 63) // 64 * 64


def rmsnorm_query_plan(op: int, M: int, N: int, dtype_code: int, vec_ok: bool = True, num_cus: int = 0) -> dict:
    lib = load_library()
    p = Plan()
    _check(lib.rmsnorm_query_plan(op, M, N, dtype_code, 1 if vec_ok else 0, num_cus, ctypes.byref(p)),
           "rmsnorm_query_plan")
    return p.as_dict()


def rmsnorm_set_plan_override(op: int, plan: Optional[dict]):
    """Force (path, vec, team, threads[, depth][, w_regs][, grid][, rows_per_step])
    for later calls of `op`; None clears.  A missing depth, w_regs or grid keeps
    the selector's; a missing rows_per_step is 1."""
    lib = load_library()
    if plan is None:
        _check(lib.rmsnorm_set_plan_override(op, None), "rmsnorm_set_plan_override")
        _overridden.discard(op)
        return
    p = Plan()
    p.depth = -1
    p.w_regs = -1
    for k, v in plan.items():
        setattr(p, k, v)
    _check(lib.rmsnorm_set_plan_override(op, ctypes.byref(p)), "rmsnorm_set_plan_override")
    _overridden.add(op)


@contextlib.contextmanager
def plan_override(op: int, **fields):
    """Context manager around rmsnorm_set_plan_override (tests and tuning)."""
    rmsnorm_set_plan_override(op, fields)
    try:
        yield
    finally:
        rmsnorm_set_plan_override(op, None)


# ---- LayerNorm ------------------------------------------------------------------

def layernorm_bwd_workspace_bytes(M: int, N: int, dtype_code: int) -> int:
    lib = load_library()
    out = ctypes.c_size_t(0)
    _check(lib.layernorm_bwd_workspace_bytes(M, N, dtype_code, ctypes.byref(out)), "layernorm_bwd_workspace_bytes")
    return int(out.value)


def _ln_fwd_common(x, residual, gamma, beta, eps, offset, y, h_out, mean, rstd, save_stats):
    torch = _torch()
    _require(x, "x")
    M, N = _rows(x)
    dev = x.device
    fused = residual is not None
    if fused:
        _require(residual, "residual", x.shape, x.dtype, dev)
    for t, name in ((gamma, "gamma"), (beta, "beta")):
        if t is not None:
            _require(t, name, (N,), x.dtype, dev)
    if y is None:
        y = torch.empty_like(x)
    _require(y, "y", x.shape, x.dtype, dev)
    if fused and h_out is None:
        h_out = torch.empty_like(x)
    if fused:
        _require(h_out, "h_out", x.shape, x.dtype, dev)
    if save_stats:
        mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev) if mean is None else mean
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=dev) if rstd is None else rstd
    for t, name in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _require(t, name, x.shape[:-1], torch.float32, dev)
    if fused:
        _launch(dev, "layernorm_fused_add_fwd", _ptr(x), _ptr(residual), _ptr(gamma), _ptr(beta), _ptr(y),
                _ptr(h_out), _ptr(mean), _ptr(rstd), M, N, eps, offset, _dtype_code(x))
    else:
        _launch(dev, "layernorm_fwd", _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), M, N, eps,
                offset, _dtype_code(x))
    return y, h_out, mean, rstd


def layernorm_fwd(x, gamma, beta, eps: float = 1e-5, offset: float = 0.0, *, y=None, mean=None, rstd=None,
                  save_stats: bool = True):
    """y = (x - mean) * rstd * (gamma + offset) + beta over the last dimension;
    returns (y, mean, rstd).  gamma / beta None: no scale / no bias."""
    y, _, mean, rstd = _ln_fwd_common(x, None, gamma, beta, eps, offset, y, None, mean, rstd, save_stats)
    return y, mean, rstd


def layernorm_fused_add_fwd(x, residual, gamma, beta, eps: float = 1e-5, offset: float = 0.0, *, y=None,
                            h_out=None, mean=None, rstd=None, save_stats: bool = True):
    """h = x + residual (rounded to the storage dtype), y = layernorm(h); returns (y, h, mean, rstd)."""
    return _ln_fwd_common(x, residual, gamma, beta, eps, offset, y, h_out, mean, rstd, save_stats)


def _ln_bwd_common(dy, dh, v, gamma, mean, rstd, eps, offset, dx, dgamma, dbeta, want_dbeta, workspace):
    torch = _torch()
    _require(v, "x" if dh is None else "h")
    M, N = _rows(v)
    dev = v.device
    _require(dy, "dy", v.shape, v.dtype, dev)
    if dh is not None:
        _require(dh, "dh", v.shape, v.dtype, dev)
    if gamma is not None:
        _require(gamma, "gamma", (N,), v.dtype, dev)
    for t, name in ((mean, "mean"), (rstd, "rstd")):
        if t is not None:
            _require(t, name, v.shape[:-1], torch.float32, dev)
    if dx is None:
        dx = torch.empty_like(v)
    _require(dx, "dx", v.shape, v.dtype, dev)
    if gamma is not None and dgamma is None:
        dgamma = torch.empty(N, dtype=v.dtype, device=dev)
    if want_dbeta and dbeta is None:
        dbeta = torch.empty(N, dtype=v.dtype, device=dev)
    for t, name in ((dgamma, "dgamma"), (dbeta, "dbeta")):
        if t is not None:
            _require(t, name, (N,), v.dtype, dev)
    code = _dtype_code(v)
    if workspace is None:
        workspace, nbytes = _bwd_workspace("ln", M, N, code, dev, (OP_LN_BWD, OP_LN_FUSED_ADD_BWD))
    else:
        _require(workspace, "workspace", device=dev)
        nbytes = workspace.numel() * workspace.element_size()
    if dh is None:
        _launch(dev, "layernorm_bwd", _ptr(dy), _ptr(v), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dgamma),
                _ptr(dbeta), _ptr(workspace), nbytes, M, N, eps, offset, code)
    else:
        _launch(dev, "layernorm_fused_add_bwd", _ptr(dy), _ptr(dh), _ptr(v), _ptr(gamma), _ptr(mean), _ptr(rstd),
                _ptr(dx), _ptr(dgamma), _ptr(dbeta), _ptr(workspace), nbytes, M, N, eps, offset, code)
    return dx, dgamma, dbeta


def layernorm_bwd(dy, x, gamma, mean, rstd, eps: float = 1e-5, offset: float = 0.0, *, dx=None, dgamma=None,
                  dbeta=None, want_dbeta: bool = True, workspace=None):
    """Gradients of layernorm_fwd; mean = rstd = None recomputes them.
    Returns (dx, dgamma or None, dbeta or None)."""
    return _ln_bwd_common(dy, None, x, gamma, mean, rstd, eps, offset, dx, dgamma, dbeta, want_dbeta, workspace)


def layernorm_fused_add_bwd(dy, dh, h, gamma, mean, rstd, eps: float = 1e-5, offset: float = 0.0, *, dx=None,
                            dgamma=None, dbeta=None, want_dbeta: bool = True, workspace=None):
    """Gradients of layernorm_fused_add_fwd: dx (= dresidual), dgamma, dbeta.
    dh may be None; pass dx=dh to accumulate in place."""
    return _ln_bwd_common(dy, dh, h, gamma, mean, rstd, eps, offset, dx, dgamma, dbeta, want_dbeta, workspace)
