"""Seeded synthetic inputs for RMSNorm forward/backward workloads.

This module is shared by the CPU reference checks, the GPU parity tests and the
benchmark.  It draws random numbers and packs them into storage formats; it holds
none of the normalisation arithmetic.

Recipe (the same for every workload):
  * ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal`` in float32;
  * draw order: x, residual (fused-add only), dy, dh (fused-add only), gamma;
  * gamma = 1 + 0.1 z with offset 0, or gamma = 0.1 z with offset 1 (the
    Gemma-style "gamma + offset" scaling);
  * eps = 1e-6 (the float32 nearest to it);
  * bf16 storage is the float32 draw rounded to nearest, ties to even, kept as
    raw uint16 bit patterns; f16 (IEEE binary16) storage is numpy's float16
    cast of the float32 draw (also nearest, ties to even).

The workloads are the pages' shapes: a 512x2048 and a 4096x4096 bf16 layer, wide
rows (8192) in bf16, a Gemma-style float32 layer (6144 wide), a DeepSeek-like
hidden size (7168) with a fused residual add, and a per-head norm (128 wide).
WIDE_WORKLOADS are rows beyond the pages' 8192-wide scope (16384 and 32768
wide, plain and fused, bf16 and float32) at 64-128 MiB per tensor;
F16_WORKLOADS repeats the 4096 x 4096 layer with binary16 storage.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

EPS = 1e-6

# storage dtype codes (match the C ABI: 0 = float32, 1 = bfloat16, 2 = binary16)
F32 = "f32"
BF16 = "bf16"
F16 = "f16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    dtype: str  # "bf16", "f16" or "f32"
    fused: bool = False
    gemma: bool = False  # gamma = 0.1 z with offset 1.0 instead of 1 + 0.1 z
    eps: float = EPS

    @property
    def offset(self) -> float:
        return 1.0 if self.gemma else 0.0

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_512x2048", 512, 2048, BF16),
        Workload("bf16_4096x4096", 4096, 4096, BF16),
        Workload("bf16_1024x8192", 1024, 8192, BF16),
        Workload("bf16_16384x8192", 16384, 8192, BF16),
        Workload("f32_16384x6144_offset1", 16384, 6144, F32, gemma=True),
        Workload("bf16_16384x7168_fused_add", 16384, 7168, BF16, fused=True),
        Workload("bf16_262144x128_per_head", 262144, 128, BF16),
    ]
}

WIDE_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_4096x16384", 4096, 16384, BF16),
        Workload("bf16_2048x32768", 2048, 32768, BF16),
        Workload("bf16_4096x16384_fused_add", 4096, 16384, BF16, fused=True),
        Workload("f32_4096x8192", 4096, 8192, F32),
        Workload("f32_2048x16384_offset1", 2048, 16384, F32, gemma=True),
    ]
}

# The 4096 x 4096 layer again with binary16 storage (same bytes as bf16).
F16_WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [Workload("f16_4096x4096", 4096, 4096, F16)]
}

ALL_WORKLOADS: Dict[str, Workload] = {**WORKLOADS, **WIDE_WORKLOADS, **F16_WORKLOADS}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Pack float32 values into bf16 bit patterns (nearest, ties to even).

    Storage conversion for generated inputs only; inputs are finite by
    construction.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Unpack bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(a)
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(a) if dtype == BF16 else np.asarray(a).astype(np.float32)


def make_inputs(
    M: int,
    N: int,
    dtype: str,
    *,
    fused: bool = False,
    gemma: bool = False,
    seed: int = 0,
    rows: Optional[np.ndarray] = None,
    layernorm: bool = False,
) -> Dict[str, np.ndarray]:
    """Generate storage-dtype arrays x, [residual], dy, [dh], gamma [, beta].

    ``rows`` (optional) keeps only those rows of the [M, N] tensors after the
    full draw, so a sampled check sees exactly the values of the full workload.
    ``layernorm``: after gamma also draw beta = 0.1 z, then a per-row shift
    2 z_i added to x before the storage rounding, so that rows have the
    nonzero means LayerNorm removes (the RMSNorm draws are unchanged).
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, np.ndarray] = {}

    def draw(shape):
        return rng.standard_normal(size=shape, dtype=np.float32)

    order = ["x"] + (["residual"] if fused else []) + ["dy"] + (["dh"] if fused else [])
    x32 = None
    for name in order:
        a = draw((M, N))
        if rows is not None:
            a = a[rows]
        if name == "x" and layernorm:
            x32 = a  # stored after the row shift is drawn
        else:
            out[name] = to_storage(a, dtype)
    z = draw((N,))
    g = (0.1 * z) if gemma else (1.0 + 0.1 * z)
    out["gamma"] = to_storage(g.astype(np.float32), dtype)
    if layernorm:
        out["beta"] = to_storage((0.1 * draw((N,))).astype(np.float32), dtype)
        shift = 2.0 * draw((M,))
        if rows is not None:
            shift = shift[rows]
        out["x"] = to_storage((x32 + shift[:, None]).astype(np.float32), dtype)
    return {k: out[k] for k in (["x"] + [n for n in out if n != "x"])}


def make_workload_inputs(w: Workload, seed: int = 0, rows: Optional[np.ndarray] = None):
    return make_inputs(w.M, w.N, w.dtype, fused=w.fused, gemma=w.gemma, seed=seed, rows=rows)


def sample_rows(M: int, count: int, seed: int = 1234) -> np.ndarray:
    """Sorted sample of row indices that always includes the first and last row."""
    if count >= M:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, M - 1), size=max(count - 2, 0), replace=False)
    return np.unique(np.concatenate([[0, M - 1], pick])).astype(np.int64)


def algorithmic_bytes(op: str, M: int, N: int, elem_bytes: int) -> int:
    """Compulsory HBM bytes of one call (workspace excluded).

    plain fwd : read x, gamma; write y, rstd        = 2MNB + NB + 4M
    plain bwd : read dy, x, gamma, rstd; write dx, dgamma = 3MNB + 2NB + 4M
    fused fwd : read x, residual, gamma; write y, h, rstd = 4MNB + NB + 4M
    fused bwd : read dy, dh, h, gamma, rstd; write dx, dgamma = 4MNB + 2NB + 4M
    bwd main  : the backward without the dgamma write (3MNB + NB + 4M plain)
    fp8 fwd   : read x, gamma; write y8 (1 byte), rstd  = MNB + MN + NB + 4M
    fused fp8 : read x, residual, gamma; write y8, h, rstd = 3MNB + MN + NB + 4M
    ln fwd    : read x, gamma, beta; write y, mean, rstd = 2MNB + 2NB + 8M
    ln bwd    : read dy, x, gamma, mean, rstd; write dx, dgamma, dbeta = 3MNB + 3NB + 8M
    (fused LayerNorm: + 2MNB forward (residual read, h write), + MNB backward (dh read))
    """
    B = elem_bytes
    table = {
        "ln_fwd": 2 * M * N * B + 2 * N * B + 8 * M,
        "ln_bwd": 3 * M * N * B + 3 * N * B + 8 * M,
        "ln_fused_fwd": 4 * M * N * B + 2 * N * B + 8 * M,
        "ln_fused_bwd": 4 * M * N * B + 3 * N * B + 8 * M,
        "fwd_fp8": M * N * B + M * N + N * B + 4 * M,
        "fused_fwd_fp8": 3 * M * N * B + M * N + N * B + 4 * M,
        "fwd": 2 * M * N * B + N * B + 4 * M,
        "bwd": 3 * M * N * B + 2 * N * B + 4 * M,
        "fused_fwd": 4 * M * N * B + N * B + 4 * M,
        "fused_bwd": 4 * M * N * B + 2 * N * B + 4 * M,
        "bwd_main": 3 * M * N * B + N * B + 4 * M,
        "fused_bwd_main": 4 * M * N * B + N * B + 4 * M,
    }
    return table[op]
