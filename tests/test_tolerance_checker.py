"""The parity checker accepts exact answers and rejects planted errors (CPU only)."""

import numpy as np

import oracle
from rmsnorm_inputs import bf16_bits_to_f32
from tolerance import (DGAMMA_TOL, check_bf16, check_f16, check_f32, dgamma_error,
                       rel_l2, ulp_bf16, ulp_f16)


def test_ulp_bf16_values():
    assert ulp_bf16(1.0) == 2.0 ** -7
    assert ulp_bf16(1.99) == 2.0 ** -7
    assert ulp_bf16(2.0) == 2.0 ** -6
    assert ulp_bf16(-0.75) == 2.0 ** -8
    assert ulp_bf16(2.0 ** -130) == 2.0 ** -133
    assert ulp_bf16(0.0) == 2.0 ** -133


def test_bf16_rule_accepts_exact_and_one_ulp():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal(10000)
    bits = oracle.round_to(ref, "bf16")
    assert check_bf16("exact", bits, ref).ok
    # one ulp up everywhere is still within 2 ulp
    assert check_bf16("1ulp", (bits.astype(np.int32) + np.where(ref >= 0, 1, 1)).astype(np.uint16), ref).ok


def test_bf16_rule_rejects_three_ulp_at_one_element():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal(5000) + 3.0  # positive, away from binade edges issues
    bits = oracle.round_to(ref, "bf16").copy()
    bits[1234] += 3
    r = check_bf16("planted", bits, ref)
    assert not r.ok and r.fails == 1 and r.worst_index == 1234


def test_bf16_floor_only_relaxes_cancelling_elements():
    ref = np.array([1e-6, 1.0])
    scale = np.array([1.0, 1.0])
    got = oracle.round_to(ref + np.array([3e-7, 0.0]), "bf16")  # 30% error on a value cancelled 1e6-fold
    assert not check_bf16("nofloor", got, ref).ok
    r = check_bf16("floor", got, ref, scale=scale)
    assert r.ok and r.floor_active == 1 and r.pure_fails == 1
    # beyond the floor's own 2 ulp it fails again
    worse = oracle.round_to(ref + np.array([2e-6, 0.0]), "bf16")
    assert not check_bf16("floor2", worse, ref, scale=scale).ok


def test_f32_rule():
    ref = np.array([1.0, -2.0, 1e-3])
    assert check_f32("ok", (ref * (1 + 5e-6)).astype(np.float32), ref).ok
    assert not check_f32("bad", (ref * (1 + 2e-5)).astype(np.float32), ref).ok
    assert not check_f32("nan", np.array([np.nan, -2.0, 1e-3], np.float32), ref).ok


def test_dgamma_rules():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal(4096) * 30
    good = oracle.round_to(ref, "bf16")
    assert dgamma_error(good, ref, "bf16") == 0.0
    scaled = oracle.round_to(ref * (1 + 2e-3), "bf16")
    assert dgamma_error(scaled, ref, "bf16") > DGAMMA_TOL["bf16"]
    assert dgamma_error(ref.astype(np.float32), ref, "f32") < DGAMMA_TOL["f32"]
    assert dgamma_error((ref * (1 + 2e-5)).astype(np.float32), ref, "f32") > DGAMMA_TOL["f32"]
    # the unrounded fp64 reference would be the wrong target for bf16 (final rounding alone ~1e-3)
    assert rel_l2(bf16_bits_to_f32(good), ref) > 1e-3


def test_ulp_f16_values():
    assert ulp_f16(1.0) == 2.0 ** -10
    assert ulp_f16(1.99) == 2.0 ** -10
    assert ulp_f16(65504.0) == 32.0
    assert ulp_f16(-0.75) == 2.0 ** -11
    assert ulp_f16(2.0 ** -20) == 2.0 ** -24
    assert ulp_f16(0.0) == 2.0 ** -24


def test_f16_rule():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal(5000) + 3.0
    got = oracle.round_to(ref, "f16")
    assert check_f16("exact", got, ref).ok
    pats = got.view(np.uint16).copy()
    assert check_f16("1ulp", (pats + 1).view(np.float16), ref).ok
    pats[77] += 3
    r = check_f16("planted", pats.view(np.float16), ref)
    assert not r.ok and r.fails == 1 and r.worst_index == 77
    # the cancellation floor: a 30% error on a value cancelled 1e6-fold passes with scale 1 only
    ref2 = np.array([1e-6, 1.0])
    bad = oracle.round_to(ref2 + np.array([3e-7, 0.0]), "f16")
    assert not check_f16("nofloor", bad, ref2).ok
    assert check_f16("floor", bad, ref2, scale=np.ones(2)).ok
    worse = oracle.round_to(ref2 + np.array([2e-6, 0.0]), "f16")
    assert not check_f16("floor2", worse, ref2, scale=np.ones(2)).ok


def test_f16_dgamma_rule():
    rng = np.random.default_rng(4)
    ref = rng.standard_normal(1) * 3  # a single column: one ulp off must still pass
    one = oracle.round_to(ref, "f16")
    up = (one.view(np.uint16) + 1).view(np.float16)
    assert dgamma_error(up, ref, "f16") <= DGAMMA_TOL["f16"]
    assert dgamma_error((one.view(np.uint16) + 3).view(np.float16), ref, "f16") > DGAMMA_TOL["f16"]


def test_floors_give_every_type_the_same_absolute_allowance():
    """At a cancelling element (|dx| far below s) each storage type's rule
    allows the same absolute error, 2^-20 s: the float32 error of the
    difference does not depend on the storage type."""
    from tolerance import BF16_FLOOR, F16_FLOOR, F32_FLOOR, F32_REL

    s = 4.0  # a power of two: the 16-bit spacings are exact there
    assert 2 * ulp_bf16(BF16_FLOOR * s) == 2 * ulp_f16(F16_FLOOR * s) == 2.0 ** -20 * s
    assert abs(F32_REL * F32_FLOOR * s - 2.0 ** -20 * s) <= 1e-15 * 2.0 ** -20 * s
    # float32: an error just inside 2^-20 s passes at a cancelling element, just outside fails
    from gpu_util_cpu import check_values_cpu

    ref = np.array([1e-9, 1.0])
    scale = np.array([s, 1.0])
    inside = np.array([1e-9 + 0.9 * 2.0 ** -20 * s, 1.0])
    outside = np.array([1e-9 + 1.1 * 2.0 ** -20 * s, 1.0])
    assert check_values_cpu(inside, ref, "f32", scale).ok
    assert not check_values_cpu(outside, ref, "f32", scale).ok


def test_floor_budget_counts_elements_the_floor_decides():
    """floor_used counts the elements that pass only because of the floor; the
    budget bounds it (a fraction of the elements plus two); rows of at most
    four elements are not bounded."""
    from tolerance import FLOOR_BUDGET, budget_for, floor_within_budget

    assert budget_for(FLOOR_BUDGET, "bf16", 4096) == 1e-3 and budget_for(FLOOR_BUDGET, "f32", 4096) == 5e-3
    assert budget_for(FLOOR_BUDGET, "f32", 4) is None and budget_for(None, "f32", 4096) is None
    assert budget_for(0.25, "bf16", 100) == 0.25

    n = 20000
    ref = np.ones(n)
    scale = np.ones(n)
    got = ref.copy()
    k = 30  # 30 elements at 1e-4 relative error: beyond 1e-5, inside the floor 2^-20 / 1e-5 * s
    ref[:k] = 1e-4
    got[:k] = 1e-4 + 5e-7
    r = check_f32("budget", got.astype(np.float64), ref, scale=scale * (2.0 ** -20 / 1e-5))
    assert r.ok and r.floor_used == k and r.pure_fails == k
    assert not floor_within_budget(r, 1e-3)  # 30 > 0.001 * 20000 + 2
    assert floor_within_budget(r, 1e-2) and floor_within_budget(r, None)
    got[k - 10:k] = ref[k - 10:k]  # 20 left
    r = check_f32("budget", got, ref, scale=scale * (2.0 ** -20 / 1e-5))
    assert r.floor_used == 20 and floor_within_budget(r, 1e-3)
