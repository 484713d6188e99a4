"""Parity rules for GPU results against the fp64 reference.

Tolerances (stated for this op: fp32 elementwise relative error <= 1e-5 and
dgamma relative L2 <= 1e-5; bf16 outputs within 2 bf16 ulp of the fp64 result
rounded to bf16 and bf16 dgamma relative L2 <= 1e-3), with these readings:

  * ulp_bf16(a) = 2^(floor(log2|a|) - 7), with the fixed subnormal spacing
    2^-133 below 2^-126.
  * dx is a difference of terms that can cancel (dy*w against xhat*c).  Any
    float32 computation carries an absolute error proportional to the size of
    those terms, s_ij = rstd_i (|g_ij| + |xhat_ij| (|c_i| + S_i)) [+ |dh_ij|],
    so the bf16 rule is taken at magnitude max(|dx|, 2^-14 s) and the fp32
    relative rule at max(|dx|, F32_FLOOR s).  Both floors allow the same
    absolute error at cancellation, 2 ulp_bf16(2^-14 s) = 1e-5 F32_FLOOR s =
    2^-20 s: the float32 error of the difference does not depend on the
    storage type.  (s >= |dx| by the triangle inequality, so a floor of s
    itself would be the larger bound on every element.)
  * Floor use is bounded and reported.  Every report counts the elements
    where the floor is the larger bound (floor_active) and those that pass
    only because of it (floor_used: they fail the rule without the floor).
    A check fails when floor_used exceeds its budget, a fraction of the
    elements (plus FLOOR_SLACK) per storage type: FLOOR_BUDGET for RMSNorm's
    dx, LN_FLOOR_BUDGET for LayerNorm (whose forward subtracts the row mean
    and so needs the floor on shifted rows too).  The budgets are about 3x the
    largest fraction measured on MI355X over the parity suite: 16-bit rules
    at most 4e-5 of the elements; float32 dx 1.5e-3 (fused add, whose dh
    term cancels too) and 3.6e-3 on a 1110-element case; float32 LayerNorm
    9e-3.  Rows built to cancel (the degenerate rows) and rows of at most
    SMALL_ROW elements, where the result is all cancellation (RMSNorm dx at
    N = 1 and LayerNorm dx at N = 2 are eps-sized remainders), are reported,
    not bounded; rows of 2^24 elements carry a row sum of 2^24 float32 terms
    and take a budget of their own.  With RMSNORM_PARITY_LOG set to a path,
    each report is appended there as one JSON line.
  * bf16 dgamma is compared with the fp64 dgamma rounded once to bf16; fp32
    dgamma with the fp64 dgamma itself.
  * Fused-add h = round(x + r) must be bit-exact.

binary16 (f16) storage, for which no tolerance is stated, takes the bf16 rule
with its own spacing: within 2 f16 ulp of the fp64 result rounded to f16, with
ulp_f16(a) = 2^(floor(log2|a|) - 10) and the fixed subnormal spacing 2^-24
below 2^-14.  The cancellation floor is 2^-11 s, which gives the same absolute
allowance as bf16's (2 ulp_f16(2^-11 s) = 2 ulp_bf16(2^-14 s) = 2^-20 s): the
float32 error of the difference does not depend on the storage type.  dgamma
keeps the 16-bit bound, relative L2 <= 1e-3 against the fp64 dgamma rounded to
f16; one element one f16 ulp off (relative 2^-10 at most) stays within it
even for a one-column dgamma.
"""

from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from rmsnorm_inputs import bf16_bits_to_f32

BF16_FLOOR = 2.0 ** -14
F16_FLOOR = 2.0 ** -11
F32_REL = 1e-5
F32_FLOOR = 2.0 ** -20 / F32_REL
# largest fraction of the elements whose verdict the floor may decide, per
# storage type, plus a few elements of slack for small cases
FLOOR_BUDGET = {"bf16": 1e-3, "f16": 1e-3, "f32": 5e-3}
LN_FLOOR_BUDGET = {"bf16": 1e-3, "f16": 1e-3, "f32": 2e-2}
FLOOR_SLACK = 2
SMALL_ROW = 4


def ulp_bf16(a) -> np.ndarray:
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(a)  # a = m 2^e, m in [0.5, 1)
    q = np.maximum(e - 1, -126)
    u = np.ldexp(1.0, q - 7)
    return np.where(a == 0, 2.0 ** -133, u)


def ulp_f16(a) -> np.ndarray:
    a = np.abs(np.asarray(a, dtype=np.float64))
    _, e = np.frexp(a)
    q = np.maximum(e - 1, -14)
    u = np.ldexp(1.0, q - 10)
    return np.where(a == 0, 2.0 ** -24, u)


@dataclasses.dataclass
class Report:
    what: str
    n: int
    fails: int
    pure_fails: int  # failures under the rule without the cancellation floor
    floor_active: int
    worst: float  # worst error in units of the allowed tolerance
    worst_index: int

    @property
    def ok(self) -> bool:
        return self.fails == 0

    @property
    def floor_used(self) -> int:
        """Elements that pass only because of the floor (they fail without it)."""
        return max(self.pure_fails - self.fails, 0)

    def __str__(self):
        return (f"{self.what}: n={self.n} fails={self.fails} pure_rule_fails={self.pure_fails} "
                f"floor_active={self.floor_active} floor_used={self.floor_used} "
                f"worst={self.worst:.3g} of tolerance at flat index {self.worst_index}")

    def as_dict(self):
        return {"what": self.what, "n": self.n, "fails": self.fails, "pure_rule_fails": self.pure_fails,
                "floor_active": self.floor_active, "floor_used": self.floor_used, "worst": self.worst}


def budget_for(budget, dtype: str, N: int):
    """The fraction that bounds floor use: a per-type table or a number; None
    (not bounded) for rows of at most SMALL_ROW elements."""
    if budget is None or N <= SMALL_ROW:
        return None
    return budget[dtype] if isinstance(budget, dict) else budget


def floor_within_budget(r: Report, budget) -> bool:
    """floor_used <= budget * n + FLOOR_SLACK; budget None: not bounded."""
    return budget is None or r.floor_used <= budget * r.n + FLOOR_SLACK


def log_report(r: Report, dtype: str, budget, note: str = ""):
    """One summary line per check on stdout, and one JSON line in the file
    named by RMSNORM_PARITY_LOG (when set), tagged with the running test."""
    import json
    import os

    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    print(f"parity {test} [{dtype}] {r} budget={budget}", flush=True)
    path = os.environ.get("RMSNORM_PARITY_LOG")
    if path:
        rec = {"test": test, "dtype": dtype, "budget": budget, "note": note, **r.as_dict()}
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def _report(what, err, tol, tol_pure, floor_mask):
    bad = ~(err <= tol)  # NaN counts as a failure
    ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err > 0, np.inf, 0.0))
    ratio = np.where(np.isnan(ratio), np.inf, ratio)
    wi = int(np.argmax(ratio)) if ratio.size else -1
    return Report(what, int(err.size), int(bad.sum()), int((~(err <= tol_pure)).sum()),
                  int(floor_mask.sum()), float(ratio.flat[wi]) if ratio.size else 0.0, wi)


def check_bf16(what, got_bits, ref64, *, scale=None, ulps=2.0) -> Report:
    """got_bits (uint16 bf16) within `ulps` bf16 ulp of round_bf16(ref64)."""
    ref64 = np.asarray(ref64, dtype=np.float64).ravel()
    got = bf16_bits_to_f32(np.asarray(got_bits).ravel()).astype(np.float64)
    ref_r = bf16_bits_to_f32(oracle.round_to(ref64, "bf16")).astype(np.float64)
    mag = np.abs(ref64)
    if scale is not None:
        floor = BF16_FLOOR * np.asarray(scale, dtype=np.float64).ravel()
        floor_mask = floor > mag
        mag = np.maximum(mag, floor)
    else:
        floor_mask = np.zeros(mag.shape, bool)
    err = np.abs(got - ref_r)
    return _report(what, err, ulps * ulp_bf16(mag), ulps * ulp_bf16(np.abs(ref64)), floor_mask)


def check_f16(what, got, ref64, *, scale=None, ulps=2.0) -> Report:
    """got (numpy float16) within `ulps` f16 ulp of round_f16(ref64)."""
    ref64 = np.asarray(ref64, dtype=np.float64).ravel()
    got = np.asarray(got).ravel()
    assert got.dtype == np.float16, got.dtype
    got = got.astype(np.float64)
    ref_r = oracle.round_to(ref64, "f16").astype(np.float64)
    mag = np.abs(ref64)
    if scale is not None:
        floor = F16_FLOOR * np.asarray(scale, dtype=np.float64).ravel()
        floor_mask = floor > mag
        mag = np.maximum(mag, floor)
    else:
        floor_mask = np.zeros(mag.shape, bool)
    with np.errstate(invalid="ignore"):  # an infinity equal to the rounded reference is exact
        err = np.where(got == ref_r, 0.0, np.abs(got - ref_r))
    return _report(what, err, ulps * ulp_f16(mag), ulps * ulp_f16(np.abs(ref64)), floor_mask)


def check_f32(what, got, ref64, *, scale=None, rel=F32_REL) -> Report:
    """|got - ref64| <= rel * max(|ref64|, scale); callers pass F32_FLOOR * s
    for a cancellation floor (scale_for())."""
    ref64 = np.asarray(ref64, dtype=np.float64).ravel()
    got = np.asarray(got, dtype=np.float64).ravel()
    mag = np.abs(ref64)
    if scale is not None:
        s = np.asarray(scale, dtype=np.float64).ravel()
        floor_mask = s > mag
        mag = np.maximum(mag, s)
    else:
        floor_mask = np.zeros(mag.shape, bool)
    err = np.abs(got - ref64)
    return _report(what, err, rel * mag, rel * np.abs(ref64), floor_mask)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def dgamma_error(got_storage, ref64, dtype: str) -> float:
    """Relative L2 of dgamma: bf16 / f16 against ref64 rounded to that type, fp32 against ref64."""
    if dtype == "f16":
        got = np.asarray(got_storage)
        assert got.dtype == np.float16, got.dtype
        return rel_l2(got.astype(np.float64), oracle.round_to(ref64, "f16").astype(np.float64))
    if dtype == "bf16":
        got = bf16_bits_to_f32(np.asarray(got_storage)).astype(np.float64)
        ref = bf16_bits_to_f32(oracle.round_to(ref64, "bf16")).astype(np.float64)
        return rel_l2(got, ref)
    return rel_l2(np.asarray(got_storage, dtype=np.float64), ref64)


DGAMMA_TOL = {"bf16": 1e-3, "f16": 1e-3, "f32": 1e-5}

# The floor factor each checker applies to the cancellation scale s
# (check_bf16 and check_f16 apply theirs inside; check_f32 takes the floored
# magnitude itself).
FLOOR_FACTOR = {"bf16": 1.0, "f16": 1.0, "f32": F32_FLOOR}


def cancel_scale(v_wide, gamma_wide, dy_wide, rstd64, c64, sabs64, offset, dh_wide=None):
    """s_ij = rstd_i (|dy w| + |v rstd| (|c_i| + S_i)) [+ |dh|]; all inputs float64."""
    w = gamma_wide + float(np.float32(offset))
    s = rstd64[:, None] * (np.abs(dy_wide * w) + np.abs(v_wide * rstd64[:, None]) * (np.abs(c64) + sabs64)[:, None])
    if dh_wide is not None:
        s = s + np.abs(dh_wide)
    return s
