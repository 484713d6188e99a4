#!/usr/bin/env python3
"""RMSNorm forward + backward on one MI355X: throughput and roofline.

One step = one pass of the whole path over a batch: the forward (rstd, y) of
one buffer set and the backward (dx, dgamma partials, dgamma finalizer) of
another, so that no step re-reads data an earlier kernel just left in the
256 MB last-level cache.  Buffers rotate over enough sets to exceed 1 GiB
("cold" data); a "hot" variant that reuses one set is reported beside it.

Default workload: bf16 rows of M=4096 x N=4096, eps 1e-6, offset 0.

Prints ONE JSON line (driver contract) with, among others:
  value       achieved GB/s of the whole step (algorithmic bytes / time)
  roofline    the dominant kernel (backward main) against the 8 TB/s HBM peak,
              and against the practical peak a plain three-stream kernel reaches
  practical_ceilings  nontemporal copy / three-stream probe rates at this size
  cpu_baseline the fp64 reference timed on the host cores on the same workload

Other modes:
  --report PATH      write a detailed JSON report (every op, cold/hot, direct/graph)
  --all-workloads    add every workload to the report
  --counters-run     a short fixed sequence of launches for rocprofv3 --pmc runs (--workload NAME)
  --timeline-run     warmup, then a few timed steps only, for a rocprofv3 --kernel-trace timeline
  --summarize-counters FETCH_DIR WRITE_DIR   per-kernel HBM bytes from two rocprofv3 --pmc runs of
                     --counters-run (FETCH_SIZE, then WRITE_SIZE), calibrated on the copies in the
                     same runs, against the algorithmic bytes (--workload NAME)
  --summarize-pmc DIR  per-kernel medians of any rocprofv3 --pmc counters
  --summarize-trace DIR  per-step kernel timeline of a rocprofv3 --kernel-trace run of --timeline-run
  --summarize-stats DIR  the kernel table of a rocprofv3 --kernel-trace --stats run
  --summarize-report REPORT_JSON  per-workload table of a --report run
"""

from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "RMSNorm fwd+bwd µs/call and achieved HBM GB/s (% of peak), bf16 4096x4096"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_{workload}.txt")


def source_hash(plan=None) -> str:
    """Identity of the backward main kernel as measured: the sources that define
    it and (when given) its launch plan.  Counters taken on a different identity
    are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_normalization_rmsnorm_amd", "csrc")
    for name in ("device_common.h", "bwd_kernels.h", "bwd_bf16.hip", "rmsnorm_internal.h"):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    if plan is not None:
        h.update(json.dumps(plan, sort_keys=True).encode())
    return h.hexdigest()[:16]


def bwd_plan(rn, w, num_cus: int = 0):
    """The backward plan of workload w (num_cus 0: the current device's count)."""
    op = rn.OP_FUSED_ADD_BWD if w.fused else rn.OP_BWD
    return rn.rmsnorm_query_plan(op, w.M, w.N, dtype_code(rn, w.dtype), True, num_cus)


def dtype_code(rn, dtype: str) -> int:
    return {"bf16": rn.BF16, "f16": rn.F16, "f32": rn.F32}[dtype]


class Sets:
    """K rotating device buffer sets for one workload, plus raw C-ABI call closures."""

    def __init__(self, w, lib, rn, torch, n_sets: int):
        from rmsnorm_inputs import make_workload_inputs

        self.w, self.lib, self.rn, self.torch = w, lib, rn, torch
        dev = torch.device("cuda:0")
        inp = make_workload_inputs(w)
        td = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
        import numpy as np

        def up(a):
            if w.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        base = {k: up(v) for k, v in inp.items()}
        del inp
        M, N = w.M, w.N
        self.dt = dtype_code(rn, w.dtype)
        self.ws_bytes = rn.rmsnorm_bwd_workspace_bytes(M, N, self.dt)
        self.ws8_bytes = rn.rmsnorm_fwd_fp8_workspace_bytes(M, N, self.dt)
        self.ws_ln_bytes = rn.layernorm_bwd_workspace_bytes(M, N, self.dt)
        self.sets = []
        for _ in range(n_sets):
            s = {
                "x": base["x"].clone(), "dy": base["dy"].clone(), "gamma": base["gamma"].clone(),
                "y": torch.empty(M, N, dtype=td, device=dev), "rstd": torch.empty(M, dtype=torch.float32, device=dev),
                "dx": torch.empty(M, N, dtype=td, device=dev), "dg": torch.empty(N, dtype=td, device=dev),
                "ws": torch.empty(max(self.ws_bytes, self.ws_ln_bytes, 16), dtype=torch.uint8, device=dev),
                # LayerNorm: bias (any values: timing only), saved statistics, dbeta
                "beta": base["gamma"].clone(), "mean": torch.empty(M, dtype=torch.float32, device=dev),
                "lrstd": torch.empty(M, dtype=torch.float32, device=dev),
                "db": torch.empty(N, dtype=td, device=dev),
                # fp8-output forward: E4M3 codes, scale, amax and its partials
                "y8": torch.empty(M, N, dtype=torch.uint8, device=dev),
                "scale": torch.full((1,), 16.0, dtype=torch.float32, device=dev),
                "amax": torch.zeros(1, dtype=torch.float32, device=dev),
                "ws8": torch.empty(max(self.ws8_bytes, 16), dtype=torch.uint8, device=dev),
            }
            if w.fused:
                s["residual"] = base["residual"].clone()
                s["h"] = torch.empty(M, N, dtype=td, device=dev)
                s["dh"] = base["dh"].clone()
            self.sets.append(s)
        del base
        torch.cuda.synchronize()
        bp = rn.rmsnorm_query_plan(rn.OP_FUSED_ADD_BWD if w.fused else rn.OP_BWD, M, N, self.dt)
        # partial rows of the stage entry point (bwd_main): the two-stage layout's, whose grid the
        # one-launch backward of few rows shares
        self.programs = bp["grid"] if bp["path"] == rn.PATH_ROWS_COLS else bp["programs"]

    def stream(self):
        return ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: status {rc}: {self.lib.rmsnorm_last_error().decode()}")

    def fwd(self, i, st):
        s, w, L = self.sets[i % len(self.sets)], self.w, self.lib
        if w.fused:
            rc = L.rmsnorm_fused_add_fwd(s["x"].data_ptr(), s["residual"].data_ptr(), s["gamma"].data_ptr(),
                                         s["y"].data_ptr(), s["h"].data_ptr(), s["rstd"].data_ptr(), w.M, w.N,
                                         w.eps, w.offset, self.dt, st)
        else:
            rc = L.rmsnorm_fwd(s["x"].data_ptr(), s["gamma"].data_ptr(), s["y"].data_ptr(), s["rstd"].data_ptr(),
                               w.M, w.N, w.eps, w.offset, self.dt, st)
        self._check(rc, "fwd")

    def fwd_fp8(self, i, st):
        s, w, L = self.sets[i % len(self.sets)], self.w, self.lib
        if w.fused:
            rc = L.rmsnorm_fused_add_fwd_fp8(s["x"].data_ptr(), s["residual"].data_ptr(), s["gamma"].data_ptr(),
                                             s["y8"].data_ptr(), s["h"].data_ptr(), s["rstd"].data_ptr(),
                                             s["scale"].data_ptr(), s["amax"].data_ptr(), s["ws8"].data_ptr(),
                                             self.ws8_bytes, w.M, w.N, w.eps, w.offset, self.dt, st)
        else:
            rc = L.rmsnorm_fwd_fp8(s["x"].data_ptr(), s["gamma"].data_ptr(), s["y8"].data_ptr(), s["rstd"].data_ptr(),
                                   s["scale"].data_ptr(), s["amax"].data_ptr(), s["ws8"].data_ptr(), self.ws8_bytes,
                                   w.M, w.N, w.eps, w.offset, self.dt, st)
        self._check(rc, "fwd_fp8")

    def ln_fwd(self, i, st):
        s, w, L = self.sets[i % len(self.sets)], self.w, self.lib
        if w.fused:
            rc = L.layernorm_fused_add_fwd(s["x"].data_ptr(), s["residual"].data_ptr(), s["gamma"].data_ptr(),
                                           s["beta"].data_ptr(), s["y"].data_ptr(), s["h"].data_ptr(),
                                           s["mean"].data_ptr(), s["lrstd"].data_ptr(), w.M, w.N, w.eps, w.offset,
                                           self.dt, st)
        else:
            rc = L.layernorm_fwd(s["x"].data_ptr(), s["gamma"].data_ptr(), s["beta"].data_ptr(), s["y"].data_ptr(),
                                 s["mean"].data_ptr(), s["lrstd"].data_ptr(), w.M, w.N, w.eps, w.offset, self.dt, st)
        self._check(rc, "ln_fwd")

    def ln_bwd(self, i, st):
        s, w, L = self.sets[i % len(self.sets)], self.w, self.lib
        nb = s["ws"].numel()
        if w.fused:
            rc = L.layernorm_fused_add_bwd(s["dy"].data_ptr(), s["dh"].data_ptr(), s["h"].data_ptr(),
                                           s["gamma"].data_ptr(), s["mean"].data_ptr(), s["lrstd"].data_ptr(),
                                           s["dh"].data_ptr(), s["dg"].data_ptr(), s["db"].data_ptr(),
                                           s["ws"].data_ptr(), nb, w.M, w.N, w.eps, w.offset, self.dt, st)
        else:
            rc = L.layernorm_bwd(s["dy"].data_ptr(), s["x"].data_ptr(), s["gamma"].data_ptr(), s["mean"].data_ptr(),
                                 s["lrstd"].data_ptr(), s["dx"].data_ptr(), s["dg"].data_ptr(), s["db"].data_ptr(),
                                 s["ws"].data_ptr(), nb, w.M, w.N, w.eps, w.offset, self.dt, st)
        self._check(rc, "ln_bwd")

    def bwd(self, i, st):
        s, w, L = self.sets[i % len(self.sets)], self.w, self.lib
        if w.fused:  # dx written over dh: dx is the residual gradient
            rc = L.rmsnorm_fused_add_bwd(s["dy"].data_ptr(), s["dh"].data_ptr(), s["h"].data_ptr(),
                                         s["gamma"].data_ptr(), s["rstd"].data_ptr(), s["dh"].data_ptr(),
                                         s["dg"].data_ptr(), s["ws"].data_ptr(), self.ws_bytes, w.M, w.N, w.eps,
                                         w.offset, self.dt, st)
        else:
            rc = L.rmsnorm_bwd(s["dy"].data_ptr(), s["x"].data_ptr(), s["gamma"].data_ptr(), s["rstd"].data_ptr(),
                               s["dx"].data_ptr(), s["dg"].data_ptr(), s["ws"].data_ptr(), self.ws_bytes, w.M, w.N,
                               w.eps, w.offset, self.dt, st)
        self._check(rc, "bwd")

    def bwd_main(self, i, st):
        s, w, L = self.sets[i % len(self.sets)], self.w, self.lib
        p = ctypes.c_int64(0)
        v = s["h"] if w.fused else s["x"]
        dh = s["dh"].data_ptr() if w.fused else None
        dx = s["dh"].data_ptr() if w.fused else s["dx"].data_ptr()
        rc = L.rmsnorm_bwd_partials(s["dy"].data_ptr(), v.data_ptr(), s["gamma"].data_ptr(), s["rstd"].data_ptr(),
                                    dh, dx, s["ws"].data_ptr(), self.ws_bytes, ctypes.byref(p), w.M, w.N, w.eps,
                                    w.offset, self.dt, st)
        self._check(rc, "bwd_main")

    def finalize(self, i, st):
        s = self.sets[i % len(self.sets)]
        rc = self.lib.rmsnorm_dgamma_finalize(s["ws"].data_ptr(), self.programs, self.w.N, s["dg"].data_ptr(),
                                              self.dt, st)
        self._check(rc, "finalize")


def time_direct(torch, fn, iters, warmup, repeats=5, rotate=True):
    """Median over `repeats` of (event time of `iters` back-to-back calls) / iters, in us."""
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(warmup):
        fn(i, st)
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            fn(i if rotate else 0, st)
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1000.0 / iters)
    return statistics.median(out)


def time_graph(torch, fn, iters, repeats=5, rotate=True):
    """Median per-call time of a HIP graph holding `iters` calls, in us."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        fn(0, st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(iters):
            fn(i if rotate else 0, st)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) * 1000.0 / iters)
    del g
    return statistics.median(out)


def n_sets_for(w, cold: bool) -> int:
    if not cold:
        return 1
    per_set = (6 if w.fused else 4) * w.M * w.N * w.elem_bytes
    return max(2, min(16, math.ceil((1 << 30) / per_set) + 1))


def measure_workload(w, lib, rn, torch, iters, warmup, detailed=True):
    """Per-op timings of one workload.  Always: cold buffers, direct launches
    (fwd, bwd, bwd main) and the finalizer from a graph.  detailed: also hot
    buffers and graph replays of fwd and bwd."""
    from rmsnorm_inputs import algorithmic_bytes

    res = {"workload": w.name, "M": w.M, "N": w.N, "dtype": w.dtype, "fused": w.fused, "offset": w.offset}
    dt = dtype_code(rn, w.dtype)
    fop_code, bop_code = (rn.OP_FUSED_ADD_FWD, rn.OP_FUSED_ADD_BWD) if w.fused else (rn.OP_FWD, rn.OP_BWD)
    res["plans"] = {"fwd": rn.rmsnorm_query_plan(fop_code, w.M, w.N, dt), "bwd": rn.rmsnorm_query_plan(bop_code, w.M, w.N, dt)}
    fop, bop = ("fused_fwd", "fused_bwd") if w.fused else ("fwd", "bwd")
    bytes_f = algorithmic_bytes(fop, w.M, w.N, w.elem_bytes)
    bytes_b = algorithmic_bytes(bop, w.M, w.N, w.elem_bytes)
    bytes_main = algorithmic_bytes(bop + "_main", w.M, w.N, w.elem_bytes)
    bytes_f8 = algorithmic_bytes(("fused_" if w.fused else "") + "fwd_fp8", w.M, w.N, w.elem_bytes)
    bytes_lf = algorithmic_bytes("ln_fused_fwd" if w.fused else "ln_fwd", w.M, w.N, w.elem_bytes)
    bytes_lb = algorithmic_bytes("ln_fused_bwd" if w.fused else "ln_bwd", w.M, w.N, w.elem_bytes)
    res["bytes"] = {"fwd": bytes_f, "bwd": bytes_b, "bwd_main": bytes_main, "fwd_fp8": bytes_f8,
                    "ln_fwd": bytes_lf, "ln_bwd": bytes_lb}
    # traffic of the backward's dgamma reduction beyond the compulsory bytes:
    # its P partial rows of N floats (two sets for LayerNorm: dgamma and
    # dbeta), written once and read once; or, for the one-launch backward of
    # few rows, the column workgroups' second read of dy and x
    ln_bop = rn.OP_LN_FUSED_ADD_BWD if w.fused else rn.OP_LN_BWD
    bplan = res["plans"]["bwd"]
    ln_plan = rn.rmsnorm_query_plan(ln_bop, w.M, w.N, dt)
    res["plans"]["ln_bwd"] = ln_plan
    second_read = 2 * w.M * w.N * w.elem_bytes
    extra_rms = second_read if bplan["path"] == rn.PATH_ROWS_COLS else 2 * bplan["programs"] * w.N * 4
    extra_ln = second_read if ln_plan["path"] == rn.PATH_ROWS_COLS else 2 * 2 * ln_plan["programs"] * w.N * 4
    res["workspace_bytes"] = {"bwd": extra_rms, "ln_bwd": extra_ln}
    for mode in (("cold", "hot") if detailed else ("cold",)):
        S = Sets(w, lib, rn, torch, n_sets_for(w, mode == "cold"))
        K = len(S.sets)
        r = {"sets": K}
        # every set's rstd must exist before a backward reads it
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i in range(K):
            S.fwd(i, st)
        r["fwd_us"] = time_direct(torch, S.fwd, iters, warmup)
        r["bwd_us"] = time_direct(torch, lambda i, s: S.bwd(i + K // 2, s), iters, warmup)
        r["bwd_main_us"] = time_direct(torch, S.bwd_main, iters, warmup)
        r["finalize_us"] = time_graph(torch, S.finalize, iters)
        # fp8-output forward with amax (main kernel + amax fold)
        r["fwd_fp8_us"] = time_direct(torch, S.fwd_fp8, iters, warmup)
        # LayerNorm on the same buffers (its statistics first, for the backward)
        for i in range(K):
            S.ln_fwd(i, st)
        r["ln_fwd_us"] = time_direct(torch, S.ln_fwd, iters, warmup)
        r["ln_bwd_us"] = time_direct(torch, lambda i, s: S.ln_bwd(i + K // 2, s), iters, warmup)
        if mode == "cold":
            sh = shim_times(S, rn, torch, iters, warmup)
            r["shim_fwd_us"], r["shim_bwd_us"] = sh["fwd_us"], sh["bwd_us"]
        if detailed:
            r["fwd_graph_us"] = time_graph(torch, S.fwd, iters)
            r["bwd_graph_us"] = time_graph(torch, lambda i, s: S.bwd(i + K // 2, s), iters)
        for op, b in (("fwd", bytes_f), ("bwd", bytes_b), ("bwd_main", bytes_main), ("fwd_fp8", bytes_f8),
                      ("ln_fwd", bytes_lf), ("ln_bwd", bytes_lb)):
            r[op + "_GBs"] = b / (r[op + "_us"] * 1e3)
            r[op + "_pct_peak"] = 100.0 * r[op + "_GBs"] / HBM_PEAK_GBS
        # the backward's bandwidth with its workspace traffic counted too
        for op, b in (("bwd", bytes_b + res["workspace_bytes"]["bwd"]),
                      ("ln_bwd", bytes_lb + res["workspace_bytes"]["ln_bwd"])):
            r[op + "_incl_ws_GBs"] = b / (r[op + "_us"] * 1e3)
        res[mode] = r
        del S
        torch.cuda.empty_cache()
    return res


def practical_ceilings(torch, tensor_bytes: int, iters: int = 50):
    """Best measured GB/s of a plain nontemporal copy (1 read + 1 write stream)
    and a three-stream kernel (2 reads + 1 write) over tensors of the
    workload's size, on rotating cold buffers: what a streaming kernel with
    the same traffic reaches on this GPU."""
    from transformer_normalization_rmsnorm_amd import _build

    lib = ctypes.CDLL(_build.PROBE_LIBRARY)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.stream_probe_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    lib.stream_probe_three.argtypes = [vp, vp, vp, i64, i32, i32, vp]
    n16 = tensor_bytes // 16
    K = max(2, math.ceil((1 << 30) / (3 * tensor_bytes)) + 1)
    bufs = [[torch.empty(n16 * 16, dtype=torch.uint8, device="cuda") for _ in range(3)] for _ in range(K)]
    for b in bufs:
        for t in b:
            t.fill_(1)
    best = {"copy": 0.0, "three": 0.0}
    full = max(1, n16 // 256)
    for kind, moved in (("copy", 2 * n16 * 16), ("three", 3 * n16 * 16)):
        for unroll in (1, 2, 4):
            for blocks in sorted({1024, 2048, 4096, max(1, full // unroll)}):
                def fn(i, st, kind=kind, unroll=unroll, blocks=blocks):
                    a, b, c = bufs[i % K]
                    if kind == "copy":
                        rc = lib.stream_probe_copy(a.data_ptr(), c.data_ptr(), n16, blocks, unroll, st)
                    else:
                        rc = lib.stream_probe_three(a.data_ptr(), b.data_ptr(), c.data_ptr(), n16, blocks, unroll, st)
                    if rc != 0:
                        raise RuntimeError(f"stream probe failed: {rc}")
                us = time_direct(torch, fn, iters, 5, repeats=3)
                best[kind] = max(best[kind], moved / (us * 1e3))
    del bufs
    torch.cuda.empty_cache()
    return {"tensor_bytes": n16 * 16, "copy_GBs": round(best["copy"], 1), "three_stream_GBs": round(best["three"], 1)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_fwd_bwd_timers(w, lib):
    """(fwd, bwd) closures running the fp64 reference on the workload's host arrays."""
    import oracle
    from rmsnorm_inputs import make_workload_inputs

    inp = make_workload_inputs(w)
    if w.fused:
        h, _, _ = oracle.fused_add_fwd(inp["x"], inp["residual"], inp["gamma"], w.dtype, w.eps, w.offset, lib=lib,
                                       want_y=False)

        def fwd():
            oracle.fused_add_fwd(inp["x"], inp["residual"], inp["gamma"], w.dtype, w.eps, w.offset, lib=lib)

        def bwd():
            oracle.bwd(inp["dy"], h, inp["gamma"], w.dtype, w.eps, w.offset, dh=inp["dh"], lib=lib)
    else:
        def fwd():
            oracle.fwd(inp["x"], inp["gamma"], w.dtype, w.eps, w.offset, lib=lib)

        def bwd():
            oracle.bwd(inp["dy"], inp["x"], inp["gamma"], w.dtype, w.eps, w.offset, lib=lib)
    return fwd, bwd


def _median_time(fn, seconds: float, min_runs: int = 3):
    times = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end or len(times) < min_runs:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times), len(times)


def cpu_baseline(w, seconds: float, single_thread_workloads=("bf16_512x2048", "bf16_4096x4096", "bf16_1024x8192")):
    """The fp64 reference, as it stands, on the host cores (bounded run):
    forward and backward timed separately on the workload with every thread
    the reference's OpenMP runtime uses, then with one thread on the smaller
    workloads (median of at least 3 runs each)."""
    import oracle
    from rmsnorm_inputs import ALL_WORKLOADS, algorithmic_bytes

    lib = oracle.load()
    fop, bop = ("fused_fwd", "fused_bwd") if w.fused else ("fwd", "bwd")
    fbytes = algorithmic_bytes(fop, w.M, w.N, w.elem_bytes)
    bbytes = algorithmic_bytes(bop, w.M, w.N, w.elem_bytes)
    threads = oracle.num_threads(lib)
    fwd, bwd = _oracle_fwd_bwd_timers(w, lib)
    tf, nf = _median_time(fwd, seconds / 2)
    tb, nb = _median_time(bwd, seconds / 2)
    single = {}
    try:
        oracle.set_num_threads(1, lib)
        for name in single_thread_workloads:
            ww = ALL_WORKLOADS[name]
            f1, b1 = _oracle_fwd_bwd_timers(ww, lib)
            t1f, _ = _median_time(f1, 0.0)
            t1b, _ = _median_time(b1, 0.0)
            fo, bo = ("fused_fwd", "fused_bwd") if ww.fused else ("fwd", "bwd")
            single[name] = {"fwd_us": round(t1f * 1e6, 1), "bwd_us": round(t1b * 1e6, 1),
                            "fwd_GBs": round(algorithmic_bytes(fo, ww.M, ww.N, ww.elem_bytes) / t1f / 1e9, 3),
                            "bwd_GBs": round(algorithmic_bytes(bo, ww.M, ww.N, ww.elem_bytes) / t1b / 1e9, 3)}
    finally:
        oracle.set_num_threads(threads, lib)
    t = tf + tb
    return {
        "value": (fbytes + bbytes) / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
        "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
        "sample": f"whole {w.name} workload, fp64 C reference (OpenMP, {threads} threads): forward median of "
                  f"{nf} runs, backward median of {nb} runs, ~{seconds:.0f} s; value = compulsory bytes of fwd + "
                  f"bwd / (fwd + bwd time); single_thread: the same reference on one thread, median of 3",
        "us_per_call": t * 1e6, "fwd_us": round(tf * 1e6, 1), "bwd_us": round(tb * 1e6, 1),
        "fwd_GBs": round(fbytes / tf / 1e9, 3), "bwd_GBs": round(bbytes / tb / 1e9, 3),
        "single_thread": single,
    }


def shim_times(S, rn, torch, iters: int, warmup: int):
    """Forward and backward through the Python binding, which allocates the
    outputs (and the backward's workspace) with torch.empty on every call:
    the cost a framework caller sees, beside the raw C-ABI launches."""
    w, K = S.w, len(S.sets)
    fwd = rn.rmsnorm_fused_add_fwd if w.fused else rn.rmsnorm_fwd
    bwd = rn.rmsnorm_fused_add_bwd if w.fused else rn.rmsnorm_bwd

    def f(i, st):
        s = S.sets[i % K]
        if w.fused:
            fwd(s["x"], s["residual"], s["gamma"], w.eps, w.offset)
        else:
            fwd(s["x"], s["gamma"], w.eps, w.offset)

    def b(i, st):
        s = S.sets[(i + K // 2) % K]
        if w.fused:
            bwd(s["dy"], s["dh"], s["h"], s["gamma"], s["rstd"], w.eps, w.offset)
        else:
            bwd(s["dy"], s["x"], s["gamma"], s["rstd"], w.eps, w.offset)

    return {"fwd_us": round(time_direct(torch, f, iters, warmup), 3), "bwd_us": round(time_direct(torch, b, iters, warmup), 3)}


def small_shape_launch_paths(lib, rn, torch, name: str = "bf16_512x2048", iters: int = 200):
    """Forward and backward of a small, host-bound workload by direct launches
    and by replay of a captured HIP graph of the same calls (cold buffers)."""
    from rmsnorm_inputs import ALL_WORKLOADS, algorithmic_bytes

    w = ALL_WORKLOADS[name]
    S = Sets(w, lib, rn, torch, n_sets_for(w, True))
    K = len(S.sets)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(K):
        S.fwd(i, st)
    out = {"workload": name}
    for op, fn in (("fwd", S.fwd), ("bwd", lambda i, s: S.bwd(i + K // 2, s))):
        nbytes = algorithmic_bytes(op, w.M, w.N, w.elem_bytes)
        d = time_direct(torch, fn, iters, 20)
        g = time_graph(torch, fn, iters)
        out[op] = {"direct_us": round(d, 3), "graph_us": round(g, 3),
                   "direct_GBs": round(nbytes / (d * 1e3), 1), "graph_GBs": round(nbytes / (g * 1e3), 1)}
    out["python_binding"] = shim_times(S, rn, torch, iters, 20)
    del S
    torch.cuda.empty_cache()
    return out


def counters_traffic(ident: str, workload: str):
    """HBM bytes per backward-main dispatch from committed rocprofv3 counters,
    or None when missing or taken on a different kernel (sources or plan)."""
    path = COUNTERS_FILE.format(workload=workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != ident:
        return None
    try:
        return float(vals["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def counters_run(rn, torch, workload: str = "bf16_4096x4096"):
    """Fixed launch sequence for rocprofv3 --pmc: a plain copy of known size,
    then forward, backward main and finalizer on one workload (the default
    one unless --workload names another); where the workload's backward is
    the one-launch kernel (few rows), five of those too."""
    from rmsnorm_inputs import ALL_WORKLOADS

    w = ALL_WORKLOADS[workload]
    lib = rn.load_library()
    S = Sets(w, lib, rn, torch, 4)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(5):
        dst.copy_(src)  # 256 MiB read + 256 MiB written
    for i in range(5):
        S.fwd(i, st)
    for i in range(5):
        S.bwd_main(i + 1, st)
    for i in range(5):
        S.finalize(i, st)
    if bwd_plan(rn, w)["path"] == rn.PATH_ROWS_COLS:
        for i in range(5):
            S.bwd(i + 1, st)
    torch.cuda.synchronize()
    print("counters run done", flush=True)


def _rocprof_rows(d: str, suffix: str):
    import csv

    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _short(name: str) -> str:
    for a, b in (("(rmsnorm::BwdArgs)", ""), ("(rmsnorm::FwdArgs)", ""), ("rmsnorm::", ""), ("unsigned short", "bf16"),
                 ("void ", "")):
        name = name.replace(a, b)
    return name


def summarize_counters(fetch_dir: str, write_dir: str, workload: str):
    """HBM bytes per dispatch of each library kernel in a --counters-run, from
    a FETCH_SIZE run and a WRITE_SIZE run.  FETCH_SIZE is calibrated on the
    plain copies of the same runs (a copy reads what it writes, and WRITE_SIZE
    counts written bytes exactly): factor = sum WRITE / sum FETCH over them."""
    from rmsnorm_inputs import ALL_WORKLOADS, algorithmic_bytes

    w = ALL_WORKLOADS[workload]
    per = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        for r in _rocprof_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], int(r["Grid_Size"]))  # one kernel may run at two launch sizes
            per.setdefault(counter, {}).setdefault(key, []).append(float(r["Counter_Value"]))
    copies = [k for k in per["FETCH_SIZE"] if "copyBuffer" in k[0]]
    f_sum = sum(sum(per["FETCH_SIZE"][k]) for k in copies)
    w_sum = sum(sum(per["WRITE_SIZE"].get(k, [])) for k in copies)
    factor = w_sum / f_sum
    fop, bop = ("fused_fwd", "fused_bwd") if w.fused else ("fwd", "bwd")
    B = w.elem_bytes
    programs = None
    out = [f"# HBM traffic per dispatch, {workload} (rocprofv3 PMC counters)",
           "#",
           "# Commands (run from /tmp with TMPDIR=/tmp, repository root R, output directory O):",
           f"#   timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d $O/pmc_fetch_{workload} "
           f"-o fetch -- python3 $R/bench.py --counters-run --workload {workload}",
           f"#   timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d $O/pmc_write_{workload} "
           f"-o write -- python3 $R/bench.py --counters-run --workload {workload}",
           f"#   python3 $R/bench.py --summarize-counters $O/pmc_fetch_{workload} "
           f"$O/pmc_write_{workload} --workload {workload}",
           "# bench.py --counters-run launches five 256 MiB device copies, then five forward, five backward-main",
           "# and five finalizer dispatches of the workload (four rotating buffer sets); where the backward takes",
           "# one launch (few rows), also five of those: dx rows plus dgamma column workgroups.",
           "#",
           f"# Calibration: the copies' WRITE_SIZE / FETCH_SIZE = {w_sum:.1f} / {f_sum:.1f} KiB -> fetch factor "
           f"{factor:.4f} (WRITE_SIZE counts written bytes exactly).",
           "# Medians over the dispatches; bytes = KiB x 1024 (FETCH x factor).",
           "#",
           f"{'kernel':72s} {'read MB':>9s} {'write MB':>9s} {'total MB':>9s} {'algorithmic MB':>15s} {'ratio':>6s}"]
    rows = {}
    import transformer_normalization_rmsnorm_amd as rn

    bplan = bwd_plan_for(w)
    one_launch_threads = ((bplan["grid"] + bplan["fin_grid"]) * bplan["threads"]
                          if bplan["path"] == rn.PATH_ROWS_COLS else None)
    for key, vals in per["FETCH_SIZE"].items():
        k, grid_threads = key
        if "rmsnorm::" not in k:
            continue
        rd = statistics.median(vals) * 1024 * factor
        wr = statistics.median(per["WRITE_SIZE"].get(key, [0.0])) * 1024
        if "bwd_" in k and grid_threads == one_launch_threads:
            alg = algorithmic_bytes(bop, w.M, w.N, B)
            kind = "backward, one launch"
        elif "finalize_kernel" in k:
            plan = None
            try:
                import transformer_normalization_rmsnorm_amd as rn

                op = rn.OP_FUSED_ADD_BWD if w.fused else rn.OP_BWD
                plan = rn.rmsnorm_query_plan(op, w.M, w.N, dtype_code(rn, w.dtype), True, 256)
            except Exception:
                plan = None
            # the stage finalizer sums the two-stage layout's partial rows
            programs = (plan["grid"] if plan["path"] == rn.PATH_ROWS_COLS else plan["programs"]) if plan else 256
            alg = programs * w.N * 4 + w.N * B
            kind = "finalizer"
        elif "bwd_" in k:
            alg = algorithmic_bytes(bop + "_main", w.M, w.N, B)
            kind = "backward main"
        else:
            alg = algorithmic_bytes(fop, w.M, w.N, B)
            kind = "forward"
        rows[kind] = (k, rd, wr, alg)
        label = _short(k) if kind != "backward, one launch" else "(one launch) " + _short(k)
        out.append(f"{label[:72]:72s} {rd / 1e6:9.3f} {wr / 1e6:9.3f} {(rd + wr) / 1e6:9.3f} {alg / 1e6:15.3f} "
                   f"{(rd + wr) / alg:6.3f}")
    out.append("#")
    out.append("# Algorithmic bytes: forward 2MNB + NB + 4M (fused 4MNB + NB + 4M); backward main 3MNB + NB + 4M")
    out.append("# (fused 4MNB + NB + 4M), its P x N x 4 partial-row writes not counted; finalizer P x N x 4 + NB;")
    out.append("# the one-launch backward 3MNB + 2NB + 4M (fused 4MNB + 2NB + 4M), its column workgroups' second")
    out.append("# read of dy and x not counted.")
    if "backward main" in rows:
        k, rd, wr, alg = rows["backward main"]
        out.append("")
        out.append(f"workload: {workload}")
        out.append(f"source_hash: {source_hash(bwd_plan_for(w))}")
        out.append(f"fetch_factor: {factor:.6f}")
        out.append(f"traffic_bytes_per_dispatch: {rd + wr:.0f}")
        out.append(f"read_bytes_per_dispatch: {rd:.0f}")
        out.append(f"write_bytes_per_dispatch: {wr:.0f}")
        out.append(f"algorithmic_bytes_per_dispatch: {alg}")
    print("\n".join(out))


def bwd_plan_for(w, num_cus: int = 256):
    """The plan on a device of num_cus compute units (MI355X: 256), so that a
    summary made without a GPU hashes the plan the benchmark will see."""
    import transformer_normalization_rmsnorm_amd as rn

    return bwd_plan(rn, w, num_cus)


def summarize_pmc(d: str):
    """Per library kernel, the median of each counter over its dispatches."""
    per = {}
    for r in _rocprof_rows(d, "counter_collection.csv"):
        if "rmsnorm::" in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    for k, cs in per.items():
        print(_short(k))
        for c, vals in sorted(cs.items()):
            print(f"    {c:22s} {statistics.median(vals):16.1f}   ({len(vals)} dispatches)")


def summarize_stats(d: str):
    """The kernel table of a rocprofv3 --kernel-trace --stats run, per kernel
    and launch geometry (workgroup size x workgroups: one kernel instance may
    serve several workloads), from the per-dispatch trace: calls and average /
    min / max duration, most total time first."""
    rows = _rocprof_rows(d, "kernel_trace.csv")
    groups = {}
    for r in rows:
        wg = int(r["Workgroup_Size_X"])
        key = (r["Kernel_Name"], wg, int(r["Grid_Size_X"]) // max(wg, 1))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"# {'kernel':66s} {'wg x grid':>12s} {'calls':>6s} {'avg us':>8s} {'min us':>8s} {'max us':>8s}")
    for (name, wg, grid), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"  {_short(name)[:66]:66s} {f'{wg}x{grid}':>12s} {len(ds):6d} {statistics.fmean(ds):8.2f} "
              f"{min(ds):8.2f} {max(ds):8.2f}")


def summarize_report(path: str):
    """Per workload of a --report run: cold-buffer times of every op (direct
    launches; the finalizer from a graph; shim_*: through the Python binding,
    outputs allocated per call), GB/s and % of the 8 TB/s peak, hot and
    graph-replay times, the streaming ceilings and the plans."""
    with open(path) as f:
        rep = json.load(f)

    def fmt(v, spec, width):
        return format(v, spec) if v is not None else "-".rjust(width)

    print(f"# {'workload':28s} {'op':9s} {'cold us':>8s} {'GB/s':>7s} {'%peak':>6s} {'hot us':>7s} {'graph us':>9s} "
          f"{'incl. ws GB/s':>13s}")
    for wl in rep["workloads"]:
        c, h = wl["cold"], wl.get("hot", {})
        for op in ("fwd", "bwd", "bwd_main", "finalize", "fwd_fp8", "ln_fwd", "ln_bwd", "shim_fwd", "shim_bwd"):
            if op + "_us" not in c:
                continue
            cells = [fmt(c[op + "_us"], "8.2f", 8), fmt(c.get(op + "_GBs"), "7.1f", 7),
                     fmt(c.get(op + "_pct_peak"), "6.1f", 6), fmt(h.get(op + "_us"), "7.2f", 7),
                     fmt(c.get(op + "_graph_us"), "9.2f", 9), fmt(c.get(op + "_incl_ws_GBs"), "13.1f", 13)]
            print(f"  {wl['workload']:28s} {op:9s} " + " ".join(cells))
        ce = wl.get("ceilings", {})
        if ce:
            print(f"  {wl['workload']:28s} ceilings: copy {ce['copy_GBs']:.0f} GB/s, three-stream "
                  f"{ce['three_stream_GBs']:.0f} GB/s")
        for k in ("fwd", "bwd", "ln_bwd"):
            p = wl.get("plans", {}).get(k)
            if p:
                print(f"  {wl['workload']:28s} {k} plan: path {p['path']} vec {p['vec']} team {p['team']} threads "
                      f"{p['threads']} chunks {p['chunks']} depth {p['depth']} w_regs {p['w_regs']} rows/step "
                      f"{p['rows_per_step']} grid {p['grid']}")


def summarize_trace(d: str):
    """Per-step timeline of a --timeline-run: each step is the forward of one
    buffer set then the backward (main, finalizer) of another, back to back on
    one stream.  Times relative to the step's first kernel start, in us,
    median over the traced steps (the warmup steps excluded)."""
    rows = _rocprof_rows(d, "kernel_trace.csv")
    ks = sorted(((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in rows
                 if "rmsnorm::" in r["Kernel_Name"]), key=lambda t: t[0])
    steps = []
    i = 0
    while i + 2 < len(ks):
        a, b, c = ks[i], ks[i + 1], ks[i + 2]
        if "fwd_" in a[2] and "bwd_" in b[2] and "finalize" in c[2]:
            steps.append((a, b, c))
            i += 3
        else:
            i += 1
    steps = steps[-10:]
    if not steps:
        raise SystemExit("no fwd / bwd / finalize triples in the trace")
    def med(f):
        return statistics.median(f(s) for s in steps)
    t0 = lambda s: s[0][0]
    fields = [
        ("forward kernel", lambda s: (s[0][1] - s[0][0]) / 1e3),
        ("gap forward end -> backward main start", lambda s: (s[1][0] - s[0][1]) / 1e3),
        ("backward main kernel", lambda s: (s[1][1] - s[1][0]) / 1e3),
        ("gap backward main end -> finalizer start", lambda s: (s[2][0] - s[1][1]) / 1e3),
        ("finalizer kernel", lambda s: (s[2][1] - s[2][0]) / 1e3),
        ("step: forward start -> finalizer end", lambda s: (s[2][1] - t0(s)) / 1e3),
    ]
    nxt = [(steps[j + 1][0][0] - steps[j][2][1]) / 1e3 for j in range(len(steps) - 1)]
    print(f"# kernels: {_short(steps[0][0][2])}; {_short(steps[0][1][2])}; {_short(steps[0][2][2])}")
    print(f"# {len(steps)} steps traced (medians, us)")
    for name, f in fields:
        print(f"{name:45s} {med(f):8.2f}")
    if nxt:
        print(f"{'gap finalizer end -> next step forward start':45s} {statistics.median(nxt):8.2f}")


def timeline_run(rn, torch, workload: str, steps: int = 10, warmup: int = 5):
    """Only the bench step (forward of one set, backward of another), for a
    kernel-trace timeline."""
    from rmsnorm_inputs import ALL_WORKLOADS

    w = ALL_WORKLOADS[workload]
    lib = rn.load_library()
    S = Sets(w, lib, rn, torch, n_sets_for(w, True))
    K = len(S.sets)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(K):
        S.fwd(i, st)
    torch.cuda.synchronize()
    for i in range(warmup + steps):
        S.fwd(i, st)
        S.bwd(i + K // 2, st)
    torch.cuda.synchronize()
    print("timeline run done", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="bf16_4096x4096")
    ap.add_argument("--report", default=None)
    ap.add_argument("--all-workloads", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--counters-run", action="store_true")
    ap.add_argument("--timeline-run", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-report", metavar="REPORT_JSON")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_report:
        summarize_report(args.summarize_report)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.workload)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} (WORLD_SIZE={world}) is not supported; "
              "this benchmark runs on a single GPU.  Across GPUs the rows would shard with no exchange except "
              "dgamma: each GPU's partial rows, finalized locally and then gathered and summed in rank order",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_normalization_rmsnorm_amd as rn
    from rmsnorm_inputs import ALL_WORKLOADS as WORKLOADS, algorithmic_bytes

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.counters_run:
        counters_run(rn, torch, args.workload)
        return
    if args.timeline_run:
        timeline_run(rn, torch, args.workload)
        return
    lib = rn.load_library()
    w = WORKLOADS[args.workload]
    fop, bop = ("fused_fwd", "fused_bwd") if w.fused else ("fwd", "bwd")
    step_bytes = algorithmic_bytes(fop, w.M, w.N, w.elem_bytes) + algorithmic_bytes(bop, w.M, w.N, w.elem_bytes)

    # ---- the timed steps (contract): W warmup steps, then exactly K steps ----
    S = Sets(w, lib, rn, torch, n_sets_for(w, True))
    K = len(S.sets)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(K):
        S.fwd(i, st)

    def step(i):
        S.fwd(i, st)
        S.bwd(i + K // 2, st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    del S
    torch.cuda.empty_cache()

    # ---- per-op and per-kernel timings (cold, direct launches) ----
    detail = measure_workload(w, lib, rn, torch, iters=200, warmup=30, detailed=bool(args.report))
    cold = detail["cold"]
    main_us = cold["bwd_main_us"]
    roofline = {
        "kernel": f"backward main ({'fused-add ' if w.fused else ''}rows, dx + dgamma partials)",
        "bound": "hbm", "achieved": detail["bytes"]["bwd_main"] / (main_us * 1e3), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": None, "traffic": counters_traffic(source_hash(bwd_plan(rn, w)), w.name),
        "bytes_per_launch": detail["bytes"]["bwd_main"], "avg_launch_us": main_us,
    }
    roofline["frac"] = roofline["achieved"] / roofline["peak"]
    ceil = practical_ceilings(torch, w.M * w.N * w.elem_bytes)
    # the backward main kernel streams two tensors in and one out
    roofline["practical_peak"] = ceil["three_stream_GBs"]
    roofline["frac_of_practical"] = roofline["achieved"] / ceil["three_stream_GBs"]

    small = small_shape_launch_paths(lib, rn, torch)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    value = step_bytes / (ms_per_step * 1e6)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"RMSNorm fwd+bwd {w.dtype} M={w.M} N={w.N} eps={w.eps} offset={w.offset}"
                               f"{' fused residual add' if w.fused else ''}, rotating cold buffers",
                   "M": w.M, "N": w.N, "storage": w.dtype, "fused_add": w.fused, "parallelism": "none (1 GPU)"},
        "us_per_step": round(ms_per_step * 1e3, 3),
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "fwd_us": round(cold["fwd_us"], 3), "bwd_us": round(cold["bwd_us"], 3),
        "fwd_fp8_us": round(cold["fwd_fp8_us"], 3), "fwd_fp8_GBs": round(cold["fwd_fp8_GBs"], 1),
        "ln_fwd_us": round(cold["ln_fwd_us"], 3), "ln_bwd_us": round(cold["ln_bwd_us"], 3),
        "fwd_GBs": round(cold["fwd_GBs"], 1), "bwd_GBs": round(cold["bwd_GBs"], 1),
        "bwd_incl_ws_GBs": round(cold["bwd_incl_ws_GBs"], 1),
        "fwd_pct_peak": round(cold["fwd_pct_peak"], 2), "bwd_pct_peak": round(cold["bwd_pct_peak"], 2),
        "bwd_main_us": round(main_us, 3), "finalize_us": round(cold["finalize_us"], 3),
        "python_binding_us": {"fwd": cold["shim_fwd_us"], "bwd": cold["shim_bwd_us"]},
        "roofline": roofline, "cpu_baseline": cpu, "practical_ceilings": ceil, "small_shape_graph": small,
        "source_hash": source_hash(bwd_plan(rn, w)), "wall_s_timed_region": round(wall, 4),
    }
    if args.report:
        line["hot_fwd_us"] = round(detail["hot"]["fwd_us"], 3)
        line["hot_bwd_us"] = round(detail["hot"]["bwd_us"], 3)
        line["fwd_graph_us"] = round(cold["fwd_graph_us"], 3)
        line["bwd_graph_us"] = round(cold["bwd_graph_us"], 3)
        report = {"bench_line": line, "workloads": [detail]}
        detail["ceilings"] = ceil
        if args.all_workloads:
            for name, ww in WORKLOADS.items():
                if name != w.name:
                    print(f"measuring {name}", file=sys.stderr, flush=True)
                    dd = measure_workload(ww, lib, rn, torch, iters=100, warmup=20)
                    dd["ceilings"] = practical_ceilings(torch, ww.M * ww.N * ww.elem_bytes, iters=20)
                    report["workloads"].append(dd)
        os.makedirs(os.path.dirname(os.path.abspath(args.report)), exist_ok=True)
        with open(args.report, "w") as f:
            json.dump(report, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
