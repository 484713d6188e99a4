"""ctypes wrapper of the fp64 CPU reference (``rmsnorm_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the GPU library or its
Python binding.  Arrays are numpy; storage dtypes are "f32", "bf16" (raw
uint16 bit patterns), "f16" (numpy float16, IEEE binary16) and "f64".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "rmsnorm_oracle.c")
LIBRARY = os.path.join(_HERE, "librmsnorm_oracle.so")

DTYPE_CODE = {"f32": 0, "bf16": 1, "f64": 2, "f16": 3}
NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64, "f16": np.float16}

_lock = threading.Lock()
_lib = None


def compile_command(source: str = SOURCE, output: str = LIBRARY):
    return ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
            "-Wall", "-Wextra", "-shared", "-fPIC", source, "-o", output, "-lm"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the reference with gcc (plain C11 + OpenMP, no fast-math)."""
    tmp = output + ".tmp"
    subprocess.run(compile_command(source, tmp), check=True)
    os.replace(tmp, output)
    return output


def _bind(lib):
    c_i64, c_f, c_vp, c_dp = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_fwd.argtypes = [ctypes.c_int, c_vp, c_vp, c_i64, c_i64, c_f, c_f, c_dp, c_dp]
    lib.oracle_fused_add_fwd.argtypes = [ctypes.c_int, c_vp, c_vp, c_vp, c_i64, c_i64, c_f, c_f,
                                         c_vp, c_dp, c_dp]
    lib.oracle_bwd.argtypes = [ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_f, c_f,
                               c_dp, c_dp, c_dp, c_dp]
    lib.oracle_round.argtypes = [ctypes.c_int, c_dp, c_i64, c_vp]
    lib.oracle_e4m3_encode.argtypes = [c_dp, c_i64, c_vp]
    lib.oracle_e4m3_decode.argtypes = [c_vp, c_i64, c_dp]
    lib.oracle_fwd_fp8.argtypes = [ctypes.c_int, c_vp, c_vp, c_i64, c_i64, c_f, c_f, c_f, ctypes.c_double,
                                   c_vp, c_vp, c_vp, c_dp, c_dp]
    lib.oracle_ln_fwd.argtypes = [ctypes.c_int, c_vp, c_vp, c_vp, c_i64, c_i64, c_f, c_f, c_dp, c_dp, c_dp]
    lib.oracle_ln_bwd.argtypes = [ctypes.c_int, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_f, c_f, c_dp, c_dp, c_dp,
                                  c_dp]
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    for f in (lib.oracle_fwd, lib.oracle_fused_add_fwd, lib.oracle_bwd, lib.oracle_round,
              lib.oracle_num_threads, lib.oracle_e4m3_encode, lib.oracle_e4m3_decode, lib.oracle_fwd_fp8,
              lib.oracle_ln_fwd, lib.oracle_ln_bwd):
        f.restype = ctypes.c_int
    return lib


def load(path: Optional[str] = None):
    """Load the compiled reference, compiling it first when it is missing or stale."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIBRARY
        if path is None and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(SOURCE)):
            build()
        lib = _bind(ctypes.CDLL(p))
        if path is None:
            _lib = lib
        return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _storage(a: np.ndarray, dtype: str) -> np.ndarray:
    want = NP_STORAGE[dtype]
    if a.dtype != want:
        raise TypeError(f"expected {np.dtype(want).name} storage for {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what} failed with status {rc}")


def num_threads(lib=None) -> int:
    return (lib or load()).oracle_num_threads()


def set_num_threads(n: int, lib=None):
    (lib or load()).oracle_set_num_threads(int(n))


def fwd(v, gamma, dtype: str, eps: float, offset: float, *, want_y: bool = True, lib=None):
    """Forward on rows of v [M, N]; returns (y64 or None, rstd64).  gamma None: non-affine."""
    lib = lib or load()
    v = _storage(v, dtype)
    gamma = None if gamma is None else _storage(gamma, dtype)
    M, N = v.shape
    y = np.empty((M, N), np.float64) if want_y else None
    rstd = np.empty(M, np.float64)
    _check(lib.oracle_fwd(DTYPE_CODE[dtype], _ptr(v), _ptr(gamma), M, N, eps, offset,
                          _ptr(y), _ptr(rstd)), "oracle_fwd")
    return y, rstd


def fused_add_fwd(x, r, gamma, dtype: str, eps: float, offset: float, *, want_y: bool = True, lib=None):
    """h = round(x + r), then the forward of h; returns (h storage, y64 or None, rstd64)."""
    lib = lib or load()
    x = _storage(x, dtype)
    r = _storage(r, dtype)
    gamma = None if gamma is None else _storage(gamma, dtype)
    M, N = x.shape
    h = np.empty((M, N), NP_STORAGE[dtype])
    y = np.empty((M, N), np.float64) if want_y else None
    rstd = np.empty(M, np.float64)
    _check(lib.oracle_fused_add_fwd(DTYPE_CODE[dtype], _ptr(x), _ptr(r), _ptr(gamma), M, N, eps,
                                    offset, _ptr(h), _ptr(y), _ptr(rstd)), "oracle_fused_add_fwd")
    return h, y, rstd


def bwd(dy, v, gamma, dtype: str, eps: float, offset: float, *, dh=None, want_dx: bool = True,
        want_dgamma: bool = True, lib=None) -> Dict[str, np.ndarray]:
    """Backward of the forward of v (h for fused-add; dh is then added to dx).

    Returns dx64 [M, N] (or None), dgamma64 [N] (or None), c64 [M] and sabs64 [M].
    """
    lib = lib or load()
    dy = _storage(dy, dtype)
    v = _storage(v, dtype)
    gamma = None if gamma is None else _storage(gamma, dtype)
    want_dgamma = want_dgamma and gamma is not None
    if dh is not None:
        dh = _storage(dh, dtype)
    M, N = v.shape
    dx = np.empty((M, N), np.float64) if want_dx else None
    dg = np.empty(N, np.float64) if want_dgamma else None
    c = np.empty(M, np.float64)
    s = np.empty(M, np.float64)
    _check(lib.oracle_bwd(DTYPE_CODE[dtype], _ptr(dy), _ptr(v), _ptr(gamma), _ptr(dh), M, N, eps,
                          offset, _ptr(dx), _ptr(dg), _ptr(c), _ptr(s)), "oracle_bwd")
    return {"dx64": dx, "dgamma64": dg, "c64": c, "sabs64": s}


def round_to(a64, dtype: str, lib=None) -> np.ndarray:
    """Round float64 values to a storage dtype (nearest, ties to even)."""
    lib = lib or load()
    a64 = np.ascontiguousarray(a64, dtype=np.float64)
    out = np.empty(a64.shape, NP_STORAGE[dtype])
    _check(lib.oracle_round(DTYPE_CODE[dtype], _ptr(a64), a64.size, _ptr(out)), "oracle_round")
    return out


def e4m3_encode(t64, lib=None) -> np.ndarray:
    """Nearest OCP E4M3 (FN) codes to float64 values, ties to even, saturating at +-448."""
    lib = lib or load()
    t64 = np.ascontiguousarray(t64, dtype=np.float64)
    out = np.empty(t64.shape, np.uint8)
    _check(lib.oracle_e4m3_encode(_ptr(t64), t64.size, _ptr(out)), "oracle_e4m3_encode")
    return out


def e4m3_decode(codes, lib=None) -> np.ndarray:
    """Values of E4M3 (FN) codes as float64 (NaN for 0x7F / 0xFF)."""
    lib = lib or load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, np.float64)
    _check(lib.oracle_e4m3_decode(_ptr(codes), codes.size, _ptr(out)), "oracle_e4m3_decode")
    return out


def fwd_fp8(v, gamma, dtype: str, eps: float, offset: float, scale: float, *, tol: float = 0.0,
            lib=None) -> Dict[str, np.ndarray]:
    """fp8-output forward of v: code = E4M3(y64 * scale), amax = max |y64|.

    With tol > 0 also code_lo / code_hi, the codes of t * (1 -+ tol) in value
    order.  Returns code, code_lo, code_hi (or None), rstd64 [M], amax64 (float).
    """
    lib = lib or load()
    v = _storage(v, dtype)
    gamma = None if gamma is None else _storage(gamma, dtype)
    M, N = v.shape
    code = np.empty((M, N), np.uint8)
    lo = np.empty((M, N), np.uint8) if tol > 0 else None
    hi = np.empty((M, N), np.uint8) if tol > 0 else None
    rstd = np.empty(M, np.float64)
    amax = np.zeros(1, np.float64)
    _check(lib.oracle_fwd_fp8(DTYPE_CODE[dtype], _ptr(v), _ptr(gamma), M, N, eps, offset, scale, tol,
                              _ptr(code), _ptr(lo), _ptr(hi), _ptr(rstd), _ptr(amax)), "oracle_fwd_fp8")
    return {"code": code, "code_lo": lo, "code_hi": hi, "rstd64": rstd, "amax64": float(amax[0])}


def ln_fwd(v, gamma, beta, dtype: str, eps: float, offset: float, *, want_y: bool = True, lib=None):
    """LayerNorm forward of rows of v; returns (y64 or None, mean64, rstd64).
    gamma None: w = 1 (offset 0); beta None: no bias."""
    lib = lib or load()
    v = _storage(v, dtype)
    gamma = None if gamma is None else _storage(gamma, dtype)
    beta = None if beta is None else _storage(beta, dtype)
    M, N = v.shape
    y = np.empty((M, N), np.float64) if want_y else None
    mean = np.empty(M, np.float64)
    rstd = np.empty(M, np.float64)
    _check(lib.oracle_ln_fwd(DTYPE_CODE[dtype], _ptr(v), _ptr(gamma), _ptr(beta), M, N, eps, offset, _ptr(y),
                             _ptr(mean), _ptr(rstd)), "oracle_ln_fwd")
    return y, mean, rstd


def ln_bwd(dy, v, gamma, dtype: str, eps: float, offset: float, *, dh=None, want_dx: bool = True,
           want_dgamma: bool = True, want_dbeta: bool = True, lib=None) -> Dict[str, np.ndarray]:
    """LayerNorm backward of the forward of v (h for fused-add; dh is added to dx).

    Returns dx64 [M, N], dgamma64 [N] (None without gamma), dbeta64 [N], and
    stats64 [M, 4] = (mean g, mean g*xhat, mean |g|, mean |g*xhat|) per row.
    """
    lib = lib or load()
    dy = _storage(dy, dtype)
    v = _storage(v, dtype)
    gamma = None if gamma is None else _storage(gamma, dtype)
    want_dgamma = want_dgamma and gamma is not None
    if dh is not None:
        dh = _storage(dh, dtype)
    M, N = v.shape
    dx = np.empty((M, N), np.float64) if want_dx else None
    dg = np.empty(N, np.float64) if want_dgamma else None
    db = np.empty(N, np.float64) if want_dbeta else None
    st = np.empty((M, 4), np.float64)
    _check(lib.oracle_ln_bwd(DTYPE_CODE[dtype], _ptr(dy), _ptr(v), _ptr(gamma), _ptr(dh), M, N, eps, offset,
                             _ptr(dx), _ptr(dg), _ptr(db), _ptr(st)), "oracle_ln_bwd")
    return {"dx64": dx, "dgamma64": dg, "dbeta64": db, "stats64": st}
