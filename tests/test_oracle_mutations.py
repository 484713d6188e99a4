"""The pins have teeth: each plausible mistake planted in a copy of the
reference (dropped term, wrong sign, wrong index, swapped operand, wrong
rounding) is caught by at least one pin.  CPU only; the planted copies are
compiled into a temporary directory and never touch the real build."""

import os
import subprocess

import pytest

import oracle
import oracle_pins

# (name, original text, mutated text, replace-all)
MUTATIONS = [
    ("eps_dropped", "return 1.0 / sqrt(ms + eps);", "return 1.0 / sqrt(ms);", False),
    ("divisor_n_minus_1", "double ms = ss / (double)N;", "double ms = ss / (double)(N > 1 ? N - 1 : N);", False),
    ("offset_dropped_fwd", "y64[i * N + j] = load_elem(dt, v, i * N + j) * rstd * w;",
     "y64[i * N + j] = load_elem(dt, v, i * N + j) * rstd * (w - off);", False),
    ("dx_sign", "double d = rstd[i] * (g - xhat * c);", "double d = rstd[i] * (g + xhat * c);", False),
    ("c_missing_mean", "double c = dot / (double)N;", "double c = dot;", False),
    ("dx_missing_rstd", "double d = rstd[i] * (g - xhat * c);", "double d = (g - xhat * c);", False),
    ("dgamma_unnormalised", "dgamma64[j] += load_elem(dt, dy, i * N + j) * (load_elem(dt, v, i * N + j) * rstd[i]);",
     "dgamma64[j] += load_elem(dt, dy, i * N + j) * load_elem(dt, v, i * N + j);", False),
    ("g_uses_v_not_dy", "double g = load_elem(dt, dy, i * N + j) * w;", "double g = load_elem(dt, v, i * N + j) * w;", True),
    ("rstd_reads_row0", "double a = load_elem(dt, v, row * N + j);", "double a = load_elem(dt, v, j);", False),
    ("dgamma_wrong_row_rstd", "(load_elem(dt, v, i * N + j) * rstd[i]);", "(load_elem(dt, v, i * N + j) * rstd[0]);", False),
    ("dh_sign", "d += load_elem(dt, dh, i * N + j);", "d -= load_elem(dt, dh, i * N + j);", False),
    ("fused_subtracts", "load_elem(dt, x, i * N + j) + load_elem(dt, r, i * N + j)",
     "load_elem(dt, x, i * N + j) - load_elem(dt, r, i * N + j)", False),
    ("ties_away", "double r = nearbyint(v / spacing) * spacing;", "double r = round(v / spacing) * spacing;", False),
    ("bf16_truncates", "double r = nearbyint(v / spacing) * spacing;", "double r = trunc(v / spacing) * spacing;", False),
    ("bf16_widen_shift", "uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;",
     "uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 15;", False),
    ("subnormal_spacing", "if (q < -126)\n        q = -126;", "if (q < -149)\n        q = -149;", False),
    # binary16 storage
    ("f16_ties_away", "const double rounded = nearbyint(a / step) * step;",
     "const double rounded = round(a / step) * step;", False),
    ("f16_subnormal_spacing", "if (lg < -14)\n        lg = -14;", "if (lg < -15)\n        lg = -15;", False),
    ("f16_overflow_edge", "if (rounded >= 65536.0)", "if (rounded >= 131072.0)", False),
    ("f16_fraction_offset", "(int)(ldexp(rounded, 10 - lr)) - 1024;", "(int)(ldexp(rounded, 10 - lr)) - 1023;", False),
    ("f16_widen_bias", "ldexp((double)(1024 + frac), field - 25)", "ldexp((double)(1024 + frac), field - 24)", False),
    ("f16_widen_subnormal", "return sign * ldexp((double)frac, -24);", "return sign * ldexp((double)frac, -25);", False),
    ("non_affine_scale", "return gamma ? load_elem(dt, gamma, j) + off : 1.0;", "return gamma ? load_elem(dt, gamma, j) + off : 1.0 + off + 0.5;", False),
    # fp8 E4M3 output
    ("e4m3_ties_away", "const double r = nearbyint(a / spacing) * spacing;", "const double r = round(a / spacing) * spacing;", False),
    ("e4m3_exponent_bias", "((E + 7) << 3) | m", "((E + 8) << 3) | m", False),
    ("e4m3_no_saturation", "if (a >= 448.0)\n        return (uint8_t)(sign | 0x7E);",
     "if (a >= 464.0)\n        return (uint8_t)(sign | 0x7F);", False),
    ("e4m3_subnormal_boundary", "if (q < -6)\n        q = -6;", "if (q < -7)\n        q = -7;", False),
    ("e4m3_mantissa_offset", "const int m = (int)(r / ldexp(1.0, E - 3)) - 8;", "const int m = (int)(r / ldexp(1.0, E - 3)) - 7;", False),
    ("e4m3_decode_bias", "return s * ldexp(1.0 + m / 8.0, e - 7);", "return s * ldexp(1.0 + m / 8.0, e - 8);", False),
    ("fp8_amax_after_scale", "else if (fabs(y) > amax)\n                amax = fabs(y);", "else if (fabs(t) > amax)\n                amax = fabs(t);", False),
    ("fp8_amax_drops_nan", "*amax64 = any_nan ? NAN : amax;", "*amax64 = amax;", False),
    ("fp8_scale_dropped", "const double t = y * sc;", "const double t = y;", False),
    ("fp8_bracket_swapped", "const double lo = t < 0 ? t * (1.0 + tol) : t * (1.0 - tol);",
     "const double lo = t < 0 ? t * (1.0 - tol) : t * (1.0 + tol);", False),
    # LayerNorm
    ("ln_mean_dropped", "const double m = s / (double)N;", "const double m = 0.0 * s;", False),
    ("ln_var_divisor", "*rstd = 1.0 / sqrt(q / (double)N + eps);", "*rstd = 1.0 / sqrt(q / (double)(N > 1 ? N - 1 : N) + eps);", False),
    ("ln_beta_dropped", "+ (beta ? load_elem(dt, beta, j) : 0.0);", "+ 0.0;", False),
    ("ln_c1_dropped", "double d = rs[i] * (g - c1 - xhat * c2);", "double d = rs[i] * (g - xhat * c2);", False),
    ("ln_c2_sign", "double d = rs[i] * (g - c1 - xhat * c2);", "double d = rs[i] * (g - c1 + xhat * c2);", False),
    ("ln_dbeta_scaled", "dbeta64[j] += d;", "dbeta64[j] += d * scale_w(dt, gamma, j, off);", False),
    ("ln_dgamma_unnormalised", "dgamma64[j] += d * ((load_elem(dt, v, i * N + j) - mu[i]) * rs[i]);",
     "dgamma64[j] += d * (load_elem(dt, v, i * N + j) - mu[i]);", False),
    ("ln_wrong_row_mean", "const double xhat = (load_elem(dt, v, i * N + j) - mu[i]) * rs[i];",
     "const double xhat = (load_elem(dt, v, i * N + j) - mu[0]) * rs[i];", True),
    # the magnitudes behind the tests' cancellation floor
    ("sabs_missing_mean", "sabs64[i] = dabs / (double)N;", "sabs64[i] = dabs;", False),
    ("sabs_signed", "dabs += fabs(g * xhat);", "dabs += g * xhat;", False),
    ("sabs_drops_rstd", "dabs += fabs(g * xhat);", "dabs += fabs(g * load_elem(dt, v, i * N + j));", False),
    ("ln_abs_g_unnormalised", "stats64[4 * i + 2] = ag / (double)N;", "stats64[4 * i + 2] = ag;", False),
    ("ln_abs_gx_unnormalised", "stats64[4 * i + 3] = agx / (double)N;", "stats64[4 * i + 3] = agx;", False),
    ("ln_abs_g_signed", "ag += fabs(g);", "ag += g;", False),
    ("ln_abs_stats_swapped", "stats64[4 * i + 2] = ag / (double)N;\n            stats64[4 * i + 3] = agx / (double)N;",
     "stats64[4 * i + 2] = agx / (double)N;\n            stats64[4 * i + 3] = ag / (double)N;", False),
    ("ln_dh_sign", "double d = rs[i] * (g - c1 - xhat * c2);\n                if (dh)\n                    d += load_elem",
     "double d = rs[i] * (g - c1 - xhat * c2);\n                if (dh)\n                    d -= load_elem", False),
]

# fast pins first so a mutant usually fails within a second
PIN_ORDER = [
    oracle_pins.golden, oracle_pins.e4m3_brute_force, oracle_pins.e4m3_torch, oracle_pins.fp8_forward,
    oracle_pins.closed_form_n1, oracle_pins.constant_row, oracle_pins.rms_invariant,
    oracle_pins.orthogonality, oracle_pins.offset_equivalence, oracle_pins.scale_invariance,
    oracle_pins.fused_reductions, oracle_pins.storage_widening, oracle_pins.rounding, oracle_pins.binary16,
    oracle_pins.torch_fp64,
    oracle_pins.non_affine, oracle_pins.finite_differences,
    oracle_pins.ln_closed_forms, oracle_pins.ln_identities, oracle_pins.ln_torch_fp64, oracle_pins.ln_finite_differences,
    oracle_pins.floor_magnitudes,
]


@pytest.mark.parametrize("name,old,new,replace_all", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new, replace_all):
    src = open(oracle.SOURCE).read()
    assert old in src, f"mutation site for {name} no longer present in the reference source"
    mutated = src.replace(old, new) if replace_all else src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.run(oracle.compile_command(str(path), lib_path), check=True, capture_output=True)
    lib = oracle.load(lib_path)
    caught_by = None
    for pin in PIN_ORDER:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught_by = pin.__name__
            break
    assert caught_by is not None, f"mutation {name} passed every pin"
