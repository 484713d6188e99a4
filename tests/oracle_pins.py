"""Pins of the fp64 CPU reference against facts fixed outside it.

Each pin takes a loaded reference library (so the mutation tests can run the
same pins against deliberately broken builds) and raises AssertionError on a
mismatch.  What pins what:

  finite_differences   backward and fused-add backward (dx, dgamma, d/dresidual)
  rms_invariant        forward: RMS_j(y_ij / w_j) = sqrt(ms / (ms + eps))
  orthogonality        dx: sum_j v_j dx_j = eps * rstd^3 * sum_j v_j g_j
  closed_form_n1       forward and backward at N = 1
  constant_row         forward on a constant row
  scale_invariance     eps = 0: y(a v) = y(v), dx(a v) = dx(v) / a, dgamma(a v) = dgamma(v)
  offset_equivalence   (gamma, offset) gives the same as (gamma + offset, 0)
  fused_reductions     fused-add with r = 0 / dh = 0 reduces to the plain op
  torch_fp64           torch.nn.functional.rms_norm in float64 with autograd
  golden               hand-worked fixtures (tests/golden/hand_worked.txt)
  storage_widening     bf16/f16/f32 storage widened exactly (same answers as f64 storage)
  rounding             nearest-even rounding vs torch casts and brute force
  binary16             IEEE binary16 storage: exact widening, round trip, numpy casts, brute force
  non_affine           no gamma: finite differences, RMS invariant, gamma = 1 equivalence
  e4m3_brute_force     fp8 E4M3 encoder vs an exhaustive nearest-code search
  e4m3_torch           fp8 E4M3 encoder vs torch's float8_e4m3fn cast; code round trip
  fp8_forward          fp8-output forward = plain forward then the encoder; amax; brackets
  ln_finite_differences  LayerNorm backward (dx, dgamma, dbeta, d/dresidual) vs central differences
  ln_identities        LayerNorm: sum dx = 0, sum xhat dx = N c2 rstd^3 eps, normalised mean / mean square
  ln_closed_forms      LayerNorm: N = 1, constant rows, shift invariance, offset, no gamma/beta
  ln_torch_fp64        torch.nn.functional.layer_norm in float64 with autograd
  floor_magnitudes     the row magnitudes behind the tolerance floor (c, S; LayerNorm's four
                       row statistics): triangle-inequality bounds and their equality cases,
                       scaling in dy and v (their exact values are in the golden fixtures)
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import oracle
from rmsnorm_inputs import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.txt")

# float32 draws to each storage type, and storage back to float64 (exact)
_CONV = {"f64": lambda a: a.astype(np.float64), "f32": lambda a: a.astype(np.float32), "bf16": f32_to_bf16_bits,
         "f16": lambda a: a.astype(np.float16)}
_WIDEN = {"f64": lambda a: a, "f32": lambda a: a.astype(np.float64),
          "bf16": lambda a: bf16_bits_to_f32(a).astype(np.float64), "f16": lambda a: a.astype(np.float64)}


def _f32(x: float) -> float:
    """The value the reference sees for a float argument (widened float32)."""
    return float(np.float32(x))


def _rand(rng, shape, scale=1.0):
    return (scale * rng.standard_normal(shape)).astype(np.float64)


def _loss(lib, v, gamma, dy, eps, offset):
    y, _ = oracle.fwd(v, gamma, "f64", eps, offset, lib=lib)
    return float(np.sum(dy * y))


def _cancel_scale(v, gamma, dy, eps, offset, out):
    """s_ij = rstd_i (|g_ij| + |xhat_ij| (|c_i| + S_i)): size of the terms that cancel in dx."""
    w = gamma + _f32(offset)
    rstd = 1.0 / np.sqrt(np.mean(v * v, axis=1) + _f32(eps))
    g = dy * w
    xhat = v * rstd[:, None]
    return rstd[:, None] * (np.abs(g) + np.abs(xhat) * (np.abs(out["c64"]) + out["sabs64"])[:, None])


def finite_differences(lib):
    rng = np.random.default_rng(11)
    worst = 0.0
    for M in (1, 2, 3):
        for N in (1, 2, 3, 7, 8, 16):
            for eps in (1e-6, 0.5):
                for offset in (0.0, 1.0):
                    v = _rand(rng, (M, N))
                    gamma = _rand(rng, (N,), 0.5) + 1.0
                    dy = _rand(rng, (M, N))
                    out = oracle.bwd(dy, v, gamma, "f64", eps, offset, lib=lib)
                    s = _cancel_scale(v, gamma, dy, eps, offset, out)
                    for i in range(M):
                        for j in range(N):
                            h = 1e-6 * max(1.0, abs(v[i, j]))
                            vp, vm = v.copy(), v.copy()
                            vp[i, j] += h
                            vm[i, j] -= h
                            fd = (_loss(lib, vp, gamma, dy, eps, offset) - _loss(lib, vm, gamma, dy, eps, offset)) / (vp[i, j] - vm[i, j])
                            ref = out["dx64"][i, j]
                            tol = 1e-7 * max(abs(ref), s[i, j])
                            err = abs(fd - ref)
                            worst = max(worst, err / max(abs(ref), s[i, j]))
                            assert err <= tol, f"dx FD M={M} N={N} eps={eps} off={offset} ({i},{j}): fd={fd} ref={ref}"
                    for j in range(N):
                        h = 1e-6 * max(1.0, abs(gamma[j]))
                        gp, gm = gamma.copy(), gamma.copy()
                        gp[j] += h
                        gm[j] -= h
                        fd = (_loss(lib, v, gp, dy, eps, offset) - _loss(lib, v, gm, dy, eps, offset)) / (gp[j] - gm[j])
                        ref = out["dgamma64"][j]
                        rstd = 1.0 / np.sqrt(np.mean(v * v, axis=1) + _f32(eps))
                        scale = max(abs(ref), float(np.sum(np.abs(dy[:, j] * v[:, j] * rstd))))
                        assert abs(fd - ref) <= 1e-7 * scale, f"dgamma FD M={M} N={N} j={j}: fd={fd} ref={ref}"
    # fused-add: L = sum dy * y(h) + sum dh * h with h = x + r; dL/dx = dL/dr = dx
    for M, N in ((1, 1), (2, 3), (3, 8)):
        for eps in (1e-6, 0.5):
            x = _rand(rng, (M, N))
            r = _rand(rng, (M, N))
            gamma = _rand(rng, (N,), 0.5) + 1.0
            dy = _rand(rng, (M, N))
            dh = _rand(rng, (M, N))

            def loss(xa, ra):
                hh, y, _ = oracle.fused_add_fwd(xa, ra, gamma, "f64", eps, 0.0, lib=lib)
                return float(np.sum(dy * y) + np.sum(dh * hh))

            h_store, _, _ = oracle.fused_add_fwd(x, r, gamma, "f64", eps, 0.0, lib=lib)
            out = oracle.bwd(dy, h_store, gamma, "f64", eps, 0.0, dh=dh, lib=lib)
            s = _cancel_scale(h_store, gamma, dy, eps, 0.0, out) + np.abs(dh)
            for i in range(M):
                for j in range(N):
                    for which in ("x", "r"):
                        a = x if which == "x" else r
                        hstep = 1e-6 * max(1.0, abs(a[i, j]))
                        ap, am = a.copy(), a.copy()
                        ap[i, j] += hstep
                        am[i, j] -= hstep
                        if which == "x":
                            fd = (loss(ap, r) - loss(am, r)) / (ap[i, j] - am[i, j])
                        else:
                            fd = (loss(x, ap) - loss(x, am)) / (ap[i, j] - am[i, j])
                        ref = out["dx64"][i, j]
                        assert abs(fd - ref) <= 1e-7 * max(abs(ref), s[i, j]), f"fused FD d{which} ({i},{j}): fd={fd} ref={ref}"
    return worst


def rms_invariant(lib):
    rng = np.random.default_rng(12)
    for N in (1, 5, 64, 1000):
        for eps in (1e-6, 0.25):
            v = _rand(rng, (4, N), 2.0)
            gamma = _rand(rng, (N,), 0.1) + 1.0
            y, rstd = oracle.fwd(v, gamma, "f64", eps, 0.0, lib=lib)
            ms = np.mean(v * v, axis=1)
            lhs = np.sqrt(np.mean((y / gamma) ** 2, axis=1))
            rhs = np.sqrt(ms / (ms + _f32(eps)))
            assert np.all(np.abs(lhs - rhs) <= 1e-13 * rhs), (N, eps, lhs, rhs)
            assert np.all(np.abs(rstd - 1.0 / np.sqrt(ms + _f32(eps))) <= 1e-13 * rstd)


def orthogonality(lib):
    rng = np.random.default_rng(13)
    for N in (1, 3, 64, 777):
        for eps in (1e-6, 0.3):
            for offset in (0.0, 1.0):
                v = _rand(rng, (5, N))
                gamma = _rand(rng, (N,), 0.3) + (0.0 if offset else 1.0)
                dy = _rand(rng, (5, N))
                out = oracle.bwd(dy, v, gamma, "f64", eps, offset, lib=lib)
                w = gamma + _f32(offset)
                g = dy * w
                ms = np.mean(v * v, axis=1)
                rstd = 1.0 / np.sqrt(ms + _f32(eps))
                lhs = np.sum(v * out["dx64"], axis=1)
                rhs = _f32(eps) * rstd ** 3 * np.sum(v * g, axis=1)
                s = _cancel_scale(v, gamma, dy, eps, offset, out)
                bound = 1e-12 * np.sum(np.abs(v) * s, axis=1)
                assert np.all(np.abs(lhs - rhs) <= bound), (N, eps, offset, lhs, rhs)


def closed_form_n1(lib):
    rng = np.random.default_rng(14)
    for eps in (1e-6, 0.5, 2.0):
        v = _rand(rng, (6, 1), 3.0)
        gamma = np.array([0.7])
        dy = _rand(rng, (6, 1))
        e = _f32(eps)
        y, rstd = oracle.fwd(v, gamma, "f64", eps, 0.0, lib=lib)
        out = oracle.bwd(dy, v, gamma, "f64", eps, 0.0, lib=lib)
        den = v * v + e
        np.testing.assert_allclose(y, v * 0.7 / np.sqrt(den), rtol=1e-14, atol=0)
        np.testing.assert_allclose(rstd, 1.0 / np.sqrt(den[:, 0]), rtol=1e-14, atol=0)
        dx_ref = dy * 0.7 * e / den ** 1.5
        scale = np.abs(dy * 0.7) / np.sqrt(den)  # size of the cancelling terms
        assert np.all(np.abs(out["dx64"] - dx_ref) <= 1e-13 * np.maximum(np.abs(dx_ref), scale)), (out["dx64"], dx_ref)
        np.testing.assert_allclose(out["dgamma64"], [np.sum(dy * v / np.sqrt(den))], rtol=1e-13)


def constant_row(lib):
    for a in (0.5, -3.0, 1e-3):
        for N in (1, 4, 1000):
            v = np.full((1, N), a)
            gamma = np.linspace(0.5, 1.5, N)
            eps = 1e-6
            y, rstd = oracle.fwd(v, gamma, "f64", eps, 0.0, lib=lib)
            r = 1.0 / np.sqrt(a * a + _f32(eps))
            np.testing.assert_allclose(rstd, [r], rtol=1e-14)
            np.testing.assert_allclose(y[0], a * r * gamma, rtol=1e-14)


def scale_invariance(lib):
    rng = np.random.default_rng(15)
    for N in (2, 17, 256):
        v = _rand(rng, (3, N))
        gamma = _rand(rng, (N,), 0.2) + 1.0
        dy = _rand(rng, (3, N))
        y1, _ = oracle.fwd(v, gamma, "f64", 0.0, 0.0, lib=lib)
        o1 = oracle.bwd(dy, v, gamma, "f64", 0.0, 0.0, lib=lib)
        for alpha in (4.0, 0.37):
            y2, _ = oracle.fwd(alpha * v, gamma, "f64", 0.0, 0.0, lib=lib)
            o2 = oracle.bwd(dy, alpha * v, gamma, "f64", 0.0, 0.0, lib=lib)
            np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-15)
            s = _cancel_scale(v, gamma, dy, 0.0, 0.0, o1)
            assert np.all(np.abs(o2["dx64"] * alpha - o1["dx64"]) <= 1e-13 * np.maximum(np.abs(o1["dx64"]), s))
            np.testing.assert_allclose(o2["dgamma64"], o1["dgamma64"], rtol=1e-12, atol=1e-13)


def offset_equivalence(lib):
    rng = np.random.default_rng(16)
    v = _rand(rng, (4, 33))
    gamma = _rand(rng, (33,), 0.1)
    dy = _rand(rng, (4, 33))
    for off in (1.0, 0.5, -2.0):
        y1, r1 = oracle.fwd(v, gamma, "f64", 1e-6, off, lib=lib)
        y2, r2 = oracle.fwd(v, gamma + off, "f64", 1e-6, 0.0, lib=lib)
        np.testing.assert_array_equal(y1, y2)
        np.testing.assert_array_equal(r1, r2)
        o1 = oracle.bwd(dy, v, gamma, "f64", 1e-6, off, lib=lib)
        o2 = oracle.bwd(dy, v, gamma + off, "f64", 1e-6, 0.0, lib=lib)
        np.testing.assert_array_equal(o1["dx64"], o2["dx64"])
        np.testing.assert_array_equal(o1["dgamma64"], o2["dgamma64"])
        # dgamma does not depend on the offset at all
        o0 = oracle.bwd(dy, v, gamma, "f64", 1e-6, 0.0, lib=lib)
        np.testing.assert_array_equal(o1["dgamma64"], o0["dgamma64"])


def fused_reductions(lib):
    rng = np.random.default_rng(17)
    for dt in ("f64", "f32", "bf16", "f16"):
        M, N = 3, 40
        x64 = rng.standard_normal((M, N)).astype(np.float32)
        g64 = (1 + 0.1 * rng.standard_normal(N)).astype(np.float32)
        dy32 = rng.standard_normal((M, N)).astype(np.float32)
        dh32 = rng.standard_normal((M, N)).astype(np.float32)
        conv = _CONV[dt]
        x, gamma, dy, dh = conv(x64), conv(g64), conv(dy32), conv(dh32)
        zero = np.zeros_like(x)
        h, yf, rf = oracle.fused_add_fwd(x, zero, gamma, dt, 1e-6, 0.0, lib=lib)
        yp, rp = oracle.fwd(x, gamma, dt, 1e-6, 0.0, lib=lib)
        np.testing.assert_array_equal(h, x)
        np.testing.assert_array_equal(yf, yp)
        np.testing.assert_array_equal(rf, rp)
        op = oracle.bwd(dy, x, gamma, dt, 1e-6, 0.0, lib=lib)
        oz = oracle.bwd(dy, x, gamma, dt, 1e-6, 0.0, dh=zero, lib=lib)
        np.testing.assert_array_equal(op["dx64"], oz["dx64"])
        od = oracle.bwd(dy, x, gamma, dt, 1e-6, 0.0, dh=dh, lib=lib)
        dh_wide = _WIDEN[dt](dh)
        np.testing.assert_allclose(od["dx64"] - op["dx64"], dh_wide, rtol=1e-12, atol=1e-15)
        np.testing.assert_array_equal(od["dgamma64"], op["dgamma64"])


def torch_fp64(lib):
    import torch

    rng = np.random.default_rng(18)
    for M, N, eps, offset in ((4, 64, 1e-6, 0.0), (3, 1000, 1e-5, 1.0), (2, 7, 0.5, 0.0), (5, 1, 1e-6, 0.0)):
        v = _rand(rng, (M, N))
        gamma = _rand(rng, (N,), 0.1) + (0.0 if offset else 1.0)
        dy = _rand(rng, (M, N))
        y, rstd = oracle.fwd(v, gamma, "f64", eps, offset, lib=lib)
        out = oracle.bwd(dy, v, gamma, "f64", eps, offset, lib=lib)
        tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
        tw = torch.tensor(gamma + _f32(offset), dtype=torch.float64, requires_grad=True)
        ty = torch.nn.functional.rms_norm(tv, (N,), weight=tw, eps=_f32(eps))
        ty.backward(torch.tensor(dy, dtype=torch.float64))
        np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-14)
        s = _cancel_scale(v, gamma, dy, eps, offset, out)
        assert np.all(np.abs(out["dx64"] - tv.grad.numpy()) <= 1e-12 * np.maximum(np.abs(out["dx64"]), s))
        np.testing.assert_allclose(out["dgamma64"], tw.grad.numpy(), rtol=1e-11, atol=1e-12)


def _e4m3_value(c: int) -> float:
    """Value of an E4M3 (OCP FN) code from the format's definition (NaN codes excluded by callers)."""
    sign = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    return sign * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def _e4m3_brute(t: float) -> int:
    """Nearest finite E4M3 code by exhaustive search; ties to the even mantissa;
    beyond the largest finite value, the largest finite value of that sign."""
    neg = t < 0 or (t == 0 and np.signbit(t))
    a = abs(t)
    best_c, best_d = None, None
    for c in range(0x7F):  # non-negative finite codes 0x00..0x7E
        d = abs(_e4m3_value(c) - a)
        if best_d is None or d < best_d or (d == best_d and (c & 1) == 0):
            best_c, best_d = c, d
    return best_c | (0x80 if neg else 0)


def _e4m3_probe_values(rng):
    pos = sorted({_e4m3_value(c) for c in range(0x7F)})
    vals = []
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        vals += [a, mid, np.nextafter(mid, 0.0), np.nextafter(mid, 1e9)]
    vals += [448.0, 449.0, 463.9, 464.0, 464.1, 480.0, 1e4, 2.0 ** -10, 2.0 ** -11, 1e-12, 0.0]
    vals += list(np.exp(rng.uniform(np.log(2.0 ** -12), np.log(600.0), 400)))
    vals = np.array(vals, dtype=np.float64)
    return np.concatenate([vals, -vals])


def e4m3_brute_force(lib):
    """The oracle's E4M3 encoder against an exhaustive nearest-code search."""
    vals = _e4m3_probe_values(np.random.default_rng(23))
    got = oracle.e4m3_encode(vals, lib=lib)
    want = np.array([_e4m3_brute(float(v)) for v in vals], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]


def e4m3_torch(lib):
    """Against torch's float8_e4m3fn cast (nearest, ties to even) of float32
    values inside +-448, and the code round trip of every finite code."""
    import torch

    # float32 inputs: torch's cast from float64 goes through float32 and so
    # rounds twice; from float32 it rounds once.  Midpoints +- one float32 ulp.
    pos = sorted({_e4m3_value(c) for c in range(0x7F)})
    v32 = []
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)
        v32 += [np.float32(a), mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))]
    v32 += list(np.exp(np.random.default_rng(29).uniform(np.log(2.0 ** -12), np.log(448.0), 400)).astype(np.float32))
    v32 = np.array(v32, dtype=np.float32)
    v32 = np.concatenate([v32, -v32])
    v32 = v32[np.abs(v32) <= 448.0]
    t = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v32.astype(np.float64), lib=lib)
    assert np.array_equal(got, t), np.nonzero(got != t)[0][:8]
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    dec = oracle.e4m3_decode(codes, lib=lib)
    assert np.array_equal(dec, [_e4m3_value(int(c)) for c in codes])
    assert np.array_equal(oracle.e4m3_encode(dec, lib=lib), codes)
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8), lib=lib)).all()


def fp8_forward(lib):
    """The fp8 forward is the plain forward followed by the encoder: codes of
    y64 * scale, amax = max |y64|, and the tolerance brackets around them."""
    rng = np.random.default_rng(31)
    M, N = 5, 37
    for dt, gemma, scale in (("f32", False, 1.0), ("bf16", True, 37.5), ("bf16", None, 300.0)):
        conv = (lambda a: a.astype(np.float32)) if dt == "f32" else f32_to_bf16_bits
        x = conv(rng.standard_normal((M, N)).astype(np.float32))
        gamma = None if gemma is None else conv(((0.1 if gemma else 1.0) * rng.standard_normal(N) + (0 if gemma else 1)).astype(np.float32))
        off = 1.0 if gemma else 0.0
        y, rstd = oracle.fwd(x, gamma, dt, 1e-6, off, lib=lib)
        out = oracle.fwd_fp8(x, gamma, dt, 1e-6, off, scale, tol=1e-5, lib=lib)
        assert np.array_equal(out["code"], oracle.e4m3_encode(y * np.float64(np.float32(scale)), lib=lib))
        assert np.array_equal(out["rstd64"], rstd)
        assert out["amax64"] == np.abs(y).max()
        t = y * np.float64(np.float32(scale))
        dec = lambda c: oracle.e4m3_decode(c, lib=lib)
        # brackets, checked exactly with a window wide enough that they usually differ
        wide = oracle.fwd_fp8(x, gamma, dt, 1e-6, off, scale, tol=0.05, lib=lib)
        lo_v, hi_v = np.where(t < 0, t * 1.05, t * 0.95), np.where(t < 0, t * 0.95, t * 1.05)
        assert np.array_equal(wide["code_lo"], oracle.e4m3_encode(lo_v, lib=lib))
        assert np.array_equal(wide["code_hi"], oracle.e4m3_encode(hi_v, lib=lib))
        assert np.mean(dec(wide["code_lo"]) < dec(wide["code_hi"])) > 0.3
        assert np.all(dec(out["code_lo"]) <= dec(out["code"])) and np.all(dec(out["code"]) <= dec(out["code_hi"]))
        # correct rounding: no finite code is nearer to t than the chosen one
        grid = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8), lib=lib)
        ts = np.clip(np.abs(t), 0, 448).ravel()
        nearest = np.min(np.abs(grid[None, :] - ts[:, None]), axis=1)
        assert np.all(np.abs(np.abs(dec(out["code"])).ravel() - ts) <= nearest)
    # a NaN input: IEEE propagation makes its row's rstd and every y of the row
    # NaN, so the row's codes are NaN codes (0x7F / 0xFF) and amax is NaN;
    # the other rows are unchanged
    x = rng.standard_normal((3, 8))
    x[1, 5] = np.nan
    out = oracle.fwd_fp8(x, None, "f64", 1e-6, 0.0, 4.0, lib=lib)
    assert np.isnan(out["amax64"]) and np.isnan(out["rstd64"][1]) and not np.isnan(out["rstd64"][[0, 2]]).any()
    assert np.all((out["code"][1] & 0x7F) == 0x7F)
    rest = oracle.fwd_fp8(x[[0, 2]], None, "f64", 1e-6, 0.0, 4.0, lib=lib)
    assert np.array_equal(out["code"][[0, 2]], rest["code"]) and rest["amax64"] == np.abs(
        oracle.fwd(x[[0, 2]], None, "f64", 1e-6, 0.0, lib=lib)[0]).max()


def _ln_loss_grads(x, gamma, beta, dy, eps, off, lib, r=None):
    """Central differences of L = sum dy * y (LayerNorm; fused: y of h = x + r)."""
    def loss(xx, gg, bb, rr):
        v = xx if rr is None else xx + rr
        y, _, _ = oracle.ln_fwd(v, gg, bb, "f64", eps, off, lib=lib)
        return float(np.sum(dy * y))

    def central(arr, idx, f):
        h = 1e-6 * max(1.0, abs(arr[idx]))
        a = arr.copy(); a[idx] += h
        b = arr.copy(); b[idx] -= h
        return (f(a) - f(b)) / (2 * h)

    dxn = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        dxn[idx] = central(x, idx, lambda a: loss(a, gamma, beta, r))
    dgn = np.array([central(gamma, (j,), lambda a: loss(x, a, beta, r)) for j in range(gamma.size)])
    dbn = np.array([central(beta, (j,), lambda a: loss(x, gamma, a, r)) for j in range(beta.size)])
    drn = None
    if r is not None:
        drn = np.zeros_like(r)
        for idx in np.ndindex(*r.shape):
            drn[idx] = central(r, idx, lambda a: loss(x, gamma, beta, a))
    return dxn, dgn, dbn, drn


def ln_finite_differences(lib):
    """LayerNorm backward (dx, dgamma, dbeta, d/dresidual) against fp64 central differences."""
    rng = np.random.default_rng(37)
    for M, N in ((1, 2), (2, 3), (3, 7), (2, 16)):
        for eps in (1e-6, 0.5):
            for off in (0.0, 1.0):
                x = rng.standard_normal((M, N))
                gamma = rng.standard_normal(N) * 0.5 + (0.0 if off else 1.0)
                beta = rng.standard_normal(N)
                dy = rng.standard_normal((M, N))
                out = oracle.ln_bwd(dy, x, gamma, "f64", eps, off, lib=lib)
                dxn, dgn, dbn, _ = _ln_loss_grads(x, gamma, beta, dy, eps, off, lib)
                rstd = oracle.ln_fwd(x, gamma, beta, "f64", eps, off, want_y=False, lib=lib)[2]
                st = out["stats64"]
                w = gamma + off
                xhat = (x - x.mean(1, keepdims=True)) * rstd[:, None]
                s = rstd[:, None] * (np.abs(dy * w) + st[:, 2:3] + np.abs(xhat) * (np.abs(st[:, 1:2]) + st[:, 3:4]))
                assert np.all(np.abs(out["dx64"] - dxn) <= 1e-7 * np.maximum(np.abs(out["dx64"]), s)), (M, N, eps, off)
                np.testing.assert_allclose(out["dgamma64"], dgn, rtol=1e-6, atol=1e-7)
                np.testing.assert_allclose(out["dbeta64"], dbn, rtol=1e-6, atol=1e-7)
                # fused: the residual's gradient equals x's
                r = rng.standard_normal((M, N))
                h = x + r
                dh = rng.standard_normal((M, N))
                fo = oracle.ln_bwd(dy, h, gamma, "f64", eps, off, dh=dh, lib=lib)
                _, _, _, drn = _ln_loss_grads(x, gamma, beta, dy, eps, off, lib, r=r)
                np.testing.assert_allclose(fo["dx64"] - dh, drn, rtol=1e-5, atol=1e-6)


def ln_identities(lib):
    """sum_j dx_j = 0; sum_j xhat_j dx_j = N * mean(g xhat) * rstd^3 * eps; the
    normalised output has mean 0 and mean square var / (var + eps)."""
    rng = np.random.default_rng(41)
    M, N = 6, 33
    x = rng.standard_normal((M, N)) * 3 + 1.5
    gamma = rng.standard_normal(N) * 0.3 + 1
    beta = rng.standard_normal(N)
    dy = rng.standard_normal((M, N))
    for eps in (1e-6, 0.25):
        y, mu, rstd = oracle.ln_fwd(x, gamma, beta, "f64", eps, 0.0, lib=lib)
        z = (y - beta) / gamma
        np.testing.assert_allclose(z.mean(1), 0, atol=1e-14)
        var = ((x - x.mean(1, keepdims=True)) ** 2).mean(1)
        np.testing.assert_allclose((z ** 2).mean(1), var / (var + eps), rtol=1e-13)
        out = oracle.ln_bwd(dy, x, gamma, "f64", eps, 0.0, lib=lib)
        dx = out["dx64"]
        scale = np.abs(dx).sum(1)
        assert np.all(np.abs(dx.sum(1)) <= 1e-13 * scale)
        xhat = (x - mu[:, None]) * rstd[:, None]
        want = N * out["stats64"][:, 1] * rstd ** 3 * eps
        np.testing.assert_allclose((xhat * dx).sum(1), want, rtol=1e-9, atol=1e-13 * scale.max())


def ln_closed_forms(lib):
    """N = 1 (y = beta, dx = 0, dbeta = dy, dgamma = 0); a constant row
    (y = beta, dx = rstd (g - mean g) with rstd = 1/sqrt(eps) = 4); shift
    invariance; (gamma, offset) = (gamma + offset, 0); no gamma / beta."""
    rng = np.random.default_rng(43)
    x = rng.standard_normal((5, 1))
    g, b = np.array([1.7]), np.array([-0.3])
    dy = rng.standard_normal((5, 1))
    y, _, _ = oracle.ln_fwd(x, g, b, "f64", 1e-6, 0.0, lib=lib)
    np.testing.assert_array_equal(y, np.full((5, 1), -0.3))
    out = oracle.ln_bwd(dy, x, g, "f64", 1e-6, 0.0, lib=lib)
    np.testing.assert_array_equal(out["dx64"], 0)
    np.testing.assert_array_equal(out["dgamma64"], 0)
    np.testing.assert_allclose(out["dbeta64"], dy.sum(0), rtol=1e-15)
    N = 9
    xc = np.full((2, N), 2.5)
    gamma = rng.standard_normal(N)
    beta = rng.standard_normal(N)
    dyc = rng.standard_normal((2, N))
    eps = 0.0625  # exact in float32: rstd = 1/sqrt(eps) = 4
    y, mu, rstd = oracle.ln_fwd(xc, gamma, beta, "f64", eps, 0.0, lib=lib)
    np.testing.assert_allclose(y, np.broadcast_to(beta, y.shape), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(rstd, 4.0)
    dx = oracle.ln_bwd(dyc, xc, gamma, "f64", eps, 0.0, lib=lib)["dx64"]
    gg = dyc * gamma
    np.testing.assert_allclose(dx, 4.0 * (gg - gg.mean(1, keepdims=True)), rtol=1e-13, atol=1e-14)
    xs = rng.standard_normal((3, 20))
    gs, bs, dys = rng.standard_normal(20), rng.standard_normal(20), rng.standard_normal((3, 20))
    y0, _, _ = oracle.ln_fwd(xs, gs, bs, "f64", 1e-3, 0.0, lib=lib)
    y1, _, _ = oracle.ln_fwd(xs + 7.25, gs, bs, "f64", 1e-3, 0.0, lib=lib)
    np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-12)
    y2, _, _ = oracle.ln_fwd(xs, gs - 1.0, bs, "f64", 1e-3, 1.0, lib=lib)
    np.testing.assert_allclose(y2, y0, rtol=1e-14, atol=1e-15)
    o0 = oracle.ln_bwd(dys, xs, gs, "f64", 1e-3, 0.0, lib=lib)
    o2 = oracle.ln_bwd(dys, xs, gs - 1.0, "f64", 1e-3, 1.0, lib=lib)
    np.testing.assert_allclose(o2["dx64"], o0["dx64"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o2["dgamma64"], o0["dgamma64"], rtol=1e-14)
    yn, _, _ = oracle.ln_fwd(xs, None, None, "f64", 1e-3, 0.0, lib=lib)
    yo, _, _ = oracle.ln_fwd(xs, np.ones(20), np.zeros(20), "f64", 1e-3, 0.0, lib=lib)
    np.testing.assert_array_equal(yn, yo)
    on = oracle.ln_bwd(dys, xs, None, "f64", 1e-3, 0.0, lib=lib)
    oo = oracle.ln_bwd(dys, xs, np.ones(20), "f64", 1e-3, 0.0, lib=lib)
    np.testing.assert_array_equal(on["dx64"], oo["dx64"])
    assert on["dgamma64"] is None


def ln_torch_fp64(lib):
    """torch.nn.functional.layer_norm in float64 with autograd."""
    import torch

    rng = np.random.default_rng(47)
    for M, N, eps, off in ((4, 64, 1e-6, 0.0), (3, 129, 0.1, 1.0), (2, 1000, 1e-5, 0.0)):
        x = rng.standard_normal((M, N)) * 2 - 0.5
        gamma = rng.standard_normal(N) * 0.2 + (0.0 if off else 1.0)
        beta = rng.standard_normal(N)
        dy = rng.standard_normal((M, N))
        y, _, _ = oracle.ln_fwd(x, gamma, beta, "f64", eps, off, lib=lib)
        out = oracle.ln_bwd(dy, x, gamma, "f64", eps, off, lib=lib)
        tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        tw = torch.tensor(gamma + _f32(off), dtype=torch.float64, requires_grad=True)
        tb = torch.tensor(beta, dtype=torch.float64, requires_grad=True)
        ty = torch.nn.functional.layer_norm(tx, (N,), weight=tw, bias=tb, eps=_f32(eps))
        ty.backward(torch.tensor(dy, dtype=torch.float64))
        np.testing.assert_allclose(y, ty.detach().numpy(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(out["dx64"], tx.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(out["dgamma64"], tw.grad.numpy(), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(out["dbeta64"], tb.grad.numpy(), rtol=1e-13, atol=1e-13)


def load_golden(path: str = GOLDEN):
    cases, cur = {}, None
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case "):
                cur = {}
                cases[line[5:].strip()] = cur
                continue
            key, _, val = line.partition(":")
            toks = val.split()
            if key.strip() in ("bits", "codes"):
                cur[key.strip()] = [int(t, 16) for t in toks]
            else:
                cur[key.strip()] = [float(t) for t in toks]
    return cases


def golden(lib):
    cases = load_golden()
    for name, c in cases.items():
        if name in ("bf16_round", "f16_round"):
            dt = name.split("_")[0]
            got = oracle.round_to(np.array(c["values"]), dt, lib=lib)
            got = got.view(np.uint16)
            assert list(map(int, got)) == c["bits"], (name, [hex(int(b)) for b in got])
            continue
        if "codes" in c:  # fp8 output
            N = int(c["N"][0])
            out = oracle.fwd_fp8(np.array(c["x"]).reshape(-1, N), np.array(c["gamma"]), "f64", c["eps"][0],
                                 c["offset"][0], c["scale"][0], lib=lib)
            assert list(map(int, out["code"].ravel())) == c["codes"], (name, [hex(int(b)) for b in out["code"].ravel()])
            np.testing.assert_allclose(out["rstd64"], c["rstd"], rtol=1e-15, err_msg=name)
            np.testing.assert_allclose(out["amax64"], c["amax"][0], rtol=1e-15, err_msg=name)
            continue
        if "mean" in c:  # LayerNorm
            N = int(c["N"][0])
            eps, off = c["eps"][0], c["offset"][0]
            x = np.array(c["x"]).reshape(-1, N)
            gamma, beta = np.array(c["gamma"]), np.array(c["beta"])
            dy = np.array(c["dy"]).reshape(-1, N)
            dh = None
            if "r" in c:
                h, _, _ = oracle.fused_add_fwd(x, np.array(c["r"]).reshape(-1, N), gamma, "f64", eps, off, lib=lib)
                np.testing.assert_allclose(h.ravel(), c["h"], rtol=0, atol=0)
                x = h
                dh = np.array(c["dh"]).reshape(-1, N)
            y, mu, rstd = oracle.ln_fwd(x, gamma, beta, "f64", eps, off, lib=lib)
            out = oracle.ln_bwd(dy, x, gamma, "f64", eps, off, dh=dh, lib=lib)
            np.testing.assert_allclose(mu, c["mean"], rtol=1e-15, atol=1e-16, err_msg=name)
            np.testing.assert_allclose(rstd, c["rstd"], rtol=1e-15, err_msg=name)
            np.testing.assert_allclose(y.ravel(), c["y"], rtol=1e-14, atol=1e-15, err_msg=name)
            np.testing.assert_allclose(out["dx64"].ravel(), c["dx"], rtol=1e-14, atol=1e-15, err_msg=name)
            np.testing.assert_allclose(out["dgamma64"], c["dgamma"], rtol=1e-14, atol=1e-15, err_msg=name)
            np.testing.assert_allclose(out["dbeta64"], c["dbeta"], rtol=0, atol=0, err_msg=name)
            np.testing.assert_allclose(out["stats64"].ravel(), c["stats"], rtol=1e-14, atol=1e-15, err_msg=name)
            continue
        N = int(c["N"][0])
        eps, off = c["eps"][0], c["offset"][0]
        x = np.array(c["x"]).reshape(-1, N)
        gamma = np.array(c["gamma"])
        dy = np.array(c["dy"]).reshape(-1, N)
        if "r" in c:
            r = np.array(c["r"]).reshape(-1, N)
            h, y, rstd = oracle.fused_add_fwd(x, r, gamma, "f64", eps, off, lib=lib)
            np.testing.assert_allclose(h.ravel(), c["h"], rtol=0, atol=0)
            v = h
            dh = np.array(c["dh"]).reshape(-1, N)
        else:
            y, rstd = oracle.fwd(x, gamma, "f64", eps, off, lib=lib)
            v, dh = x, None
        out = oracle.bwd(dy, v, gamma, "f64", eps, off, dh=dh, lib=lib)
        np.testing.assert_allclose(rstd, c["rstd"], rtol=1e-15, err_msg=name)
        np.testing.assert_allclose(y.ravel(), c["y"], rtol=1e-15, atol=1e-16, err_msg=name)
        np.testing.assert_allclose(out["dx64"].ravel(), c["dx"], rtol=1e-14, atol=1e-16, err_msg=name)
        np.testing.assert_allclose(out["dgamma64"], c["dgamma"], rtol=1e-15, atol=1e-16, err_msg=name)
        np.testing.assert_allclose(out["c64"], c["c"], rtol=1e-15, atol=1e-16, err_msg=name)
        np.testing.assert_allclose(out["sabs64"], c["S"], rtol=1e-15, atol=1e-16, err_msg=name)


def floor_magnitudes(lib):
    """The magnitudes behind the tests' cancellation floor, by properties that
    fix them: S = mean_j |g xhat| is at least |c| = |mean_j g xhat| (triangle
    inequality) and equals it when every g xhat has one sign (dy = v, w > 0);
    both scale with |dy| (S(a dy) = |a| S(dy)) and do not depend on the scale
    of v at eps = 0.  LayerNorm's (mean |g|, mean |g xhat|) bound (|mean g|,
    |mean g xhat|) the same way, with equality when g >= 0 and g xhat >= 0."""
    rng = np.random.default_rng(41)
    M, N = 6, 29
    v = _rand(rng, (M, N))
    dy = _rand(rng, (M, N))
    gamma = np.abs(_rand(rng, (N,), 0.3)) + 0.5  # w > 0
    out = oracle.bwd(dy, v, gamma, "f64", 1e-6, 0.0, lib=lib)
    c, S = out["c64"], out["sabs64"]
    assert np.all(S >= np.abs(c)) and np.all(S > 1.05 * np.abs(c)), (S, c)
    same = oracle.bwd(v, v, gamma, "f64", 1e-6, 0.0, lib=lib)  # g xhat = w v^2 rstd >= 0
    np.testing.assert_allclose(same["sabs64"], same["c64"], rtol=1e-14)
    for a in (-3.0, 0.25):
        sc = oracle.bwd(a * dy, v, gamma, "f64", 1e-6, 0.0, lib=lib)
        np.testing.assert_allclose(sc["sabs64"], abs(a) * S, rtol=1e-14)
        np.testing.assert_allclose(sc["c64"], a * c, rtol=1e-13)
    big = oracle.bwd(dy, 8.0 * v, gamma, "f64", 0.0, 0.0, lib=lib)
    small = oracle.bwd(dy, v, gamma, "f64", 0.0, 0.0, lib=lib)
    np.testing.assert_allclose(big["sabs64"], small["sabs64"], rtol=1e-14)
    # LayerNorm
    st = oracle.ln_bwd(dy, v, gamma, "f64", 1e-5, 0.0, lib=lib)["stats64"]
    assert np.all(st[:, 2] >= np.abs(st[:, 0])) and np.all(st[:, 3] >= np.abs(st[:, 1]))
    assert np.all(st[:, 2] > 1.05 * np.abs(st[:, 0])) and np.all(st[:, 3] > 1.05 * np.abs(st[:, 1]))
    dy_pos = np.abs(dy)
    st_pos = oracle.ln_bwd(dy_pos, v, gamma, "f64", 1e-5, 0.0, lib=lib)["stats64"]
    np.testing.assert_allclose(st_pos[:, 2], st_pos[:, 0], rtol=1e-14)  # g >= 0
    # g xhat >= 0 when dy has the sign of (v - mean): dy = v - mean(v)
    dy_al = v - v.mean(axis=1, keepdims=True)
    st_al = oracle.ln_bwd(dy_al, v, gamma, "f64", 1e-5, 0.0, lib=lib)["stats64"]
    np.testing.assert_allclose(st_al[:, 3], st_al[:, 1], rtol=1e-13)
    st2 = oracle.ln_bwd(-2.0 * dy, v, gamma, "f64", 1e-5, 0.0, lib=lib)["stats64"]
    np.testing.assert_allclose(st2[:, 2:], 2.0 * st[:, 2:], rtol=1e-14)
    np.testing.assert_allclose(st2[:, :2], -2.0 * st[:, :2], rtol=1e-13)


def storage_widening(lib):
    rng = np.random.default_rng(19)
    M, N = 3, 50
    for dt in ("f32", "bf16", "f16"):
        conv, widen = _CONV[dt], _WIDEN[dt]
        x = conv(rng.standard_normal((M, N)).astype(np.float32))
        r = conv(rng.standard_normal((M, N)).astype(np.float32))
        gamma = conv((1 + 0.1 * rng.standard_normal(N)).astype(np.float32))
        dy = conv(rng.standard_normal((M, N)).astype(np.float32))
        y_s, r_s = oracle.fwd(x, gamma, dt, 1e-6, 0.5, lib=lib)
        y_d, r_d = oracle.fwd(widen(x), widen(gamma), "f64", 1e-6, 0.5, lib=lib)
        np.testing.assert_array_equal(y_s, y_d)
        np.testing.assert_array_equal(r_s, r_d)
        o_s = oracle.bwd(dy, x, gamma, dt, 1e-6, 0.5, dh=r, lib=lib)
        o_d = oracle.bwd(widen(dy), widen(x), widen(gamma), "f64", 1e-6, 0.5, dh=widen(r), lib=lib)
        np.testing.assert_array_equal(o_s["dx64"], o_d["dx64"])
        np.testing.assert_array_equal(o_s["dgamma64"], o_d["dgamma64"])
        # the fused-add residual sum in storage precision: nearest to the exact sum
        h, _, _ = oracle.fused_add_fwd(x, r, gamma, dt, 1e-6, 0.0, lib=lib)
        exact = widen(x) + widen(r)  # exact in float64 for these magnitudes
        np.testing.assert_array_equal(h, oracle.round_to(exact, dt, lib=lib))
        np.testing.assert_array_equal(widen(h), _brute_round(exact.ravel(), dt).reshape(h.shape))


def _bf16_neighbours(v: float):
    """All bf16 values adjacent to v (brute force over the bit patterns near it)."""
    f = np.float32(v)
    b = int(f32_to_bf16_bits(np.array([f]))[0])
    cands = []
    for d in range(-2, 3):
        bb = (b + d) & 0xFFFF
        val = float(bf16_bits_to_f32(np.array([bb], np.uint16))[0])
        if np.isfinite(val):
            cands.append(val)
    return cands


def _f16_neighbours(v: float):
    """binary16 values around v: the patterns within 2 of the pattern of the
    float32 image of v, clamped to the finite range."""
    f = np.float32(min(max(v, -65504.0), 65504.0))
    b = int(np.array([f], np.float32).astype(np.float16).view(np.uint16)[0])
    cands = []
    for d in range(-2, 3):
        bb = (b + d) & 0xFFFF
        val = float(np.array([bb], np.uint16).view(np.float16)[0])
        if np.isfinite(val):
            cands.append(val)
    return cands


def _brute_round(vals, dt):
    """Nearest representable value, ties to the even significand, by exact rational search."""
    out = []
    for v in vals:
        v = float(v)
        if dt == "f32":
            cands = [float(np.float32(v)), float(np.nextafter(np.float32(v), np.float32(np.inf))),
                     float(np.nextafter(np.float32(v), np.float32(-np.inf)))]
            bits = lambda c: int(np.array([c], np.float32).view(np.uint32)[0])
        elif dt == "f16":
            cands = _f16_neighbours(v)
            bits = lambda c: int(np.array([c], np.float16).view(np.uint16)[0])
        else:
            cands = _bf16_neighbours(v)
            bits = lambda c: int(f32_to_bf16_bits(np.array([c], np.float32))[0])
        fv = Fraction(v)
        best = min(cands, key=lambda c: (abs(Fraction(c) - fv), bits(c) & 1))
        out.append(best)
    return np.array(out)


def rounding(lib):
    import torch

    rng = np.random.default_rng(20)
    # float32-representable values: torch's float32 -> bfloat16 cast rounds to nearest even
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.3895314e38, 1e-40, -1e-41,
                  1.1754944e-38, np.float32(2.0) ** -133, np.float32(2.0) ** -134, np.inf, -np.inf], np.float32),
    ])
    # bf16/float32 subnormals and the normal/subnormal boundary, mostly off the bf16 grid
    sub = (rng.integers(1, 1 << 23, 4000).astype(np.uint32)).view(np.float32)
    sub = np.concatenate([sub, -sub, sub * np.float32(1.9)])
    f = np.concatenate([f, sub])
    f = f[np.isfinite(f) | np.isinf(f)]
    got = oracle.round_to(f.astype(np.float64), "bf16", lib=lib)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    # float64 values that float32 cannot hold (double rounding through float32 would be wrong)
    d = np.array([1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -8 - 2.0 ** -30, -(1 + 3 * 2.0 ** -8 - 2.0 ** -40),
                  0.2, 1.4, np.pi, -np.e * 1e20, 2.0 ** -130 * 1.25])
    d = np.concatenate([d, rng.standard_normal(300) * 7.0])
    got = oracle.round_to(d, "bf16", lib=lib)
    np.testing.assert_array_equal(bf16_bits_to_f32(got).astype(np.float64), _brute_round(d, "bf16"))
    # float32 storage rounding
    got32 = oracle.round_to(d, "f32", lib=lib)
    np.testing.assert_array_equal(got32.astype(np.float64), _brute_round(d, "f32"))
    # NaN stays NaN
    assert np.isnan(bf16_bits_to_f32(oracle.round_to(np.array([np.nan]), "bf16", lib=lib)))[0]


def binary16(lib):
    """IEEE binary16 storage: every finite pattern widens exactly and rounds
    back to itself; rounding of float64 values (ties, subnormals, overflow,
    bits beyond float32) agrees with numpy's float64 -> float16 cast and with
    an exact nearest-value search."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = pats.view(np.float16)
    fin = pats[np.isfinite(vals)]  # 63488 patterns, +-0 included
    wide = fin.view(np.float16).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_to(wide, "f16", lib=lib).view(np.uint16), fin)
    # the reference's widening of stored binary16 against numpy's: identical forward results
    x = fin.view(np.float16).reshape(1024, 62)
    y_s, r_s = oracle.fwd(x, None, "f16", 1e-6, 0.0, lib=lib)
    y_d, r_d = oracle.fwd(x.astype(np.float64), None, "f64", 1e-6, 0.0, lib=lib)
    np.testing.assert_array_equal(y_s, y_d)
    np.testing.assert_array_equal(np.signbit(y_s), np.signbit(y_d))
    np.testing.assert_array_equal(r_s, r_d)
    # float64 values: midpoints of adjacent binary16 values (exact ties), points
    # just off them, random magnitudes over the whole range, the overflow edge
    rng = np.random.default_rng(22)
    pos = np.sort(wide[wide > 0])
    k = rng.integers(0, pos.size - 1, 3000)
    mid = (pos[k] + pos[k + 1]) / 2
    d = np.concatenate([
        mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid,
        rng.standard_normal(4000) * 2.0 ** rng.integers(-28, 17, 4000),
        np.array([65504.0, 65519.0, 65520.0, 65519.99999999999, 70000.0, 1e300, -65520.0, 2.0 ** -25,
                  2.0 ** -25 * (1 + 2.0 ** -40), 2.0 ** -26, 2.0 ** -14 - 2.0 ** -25, 1 + 2.0 ** -11 + 2.0 ** -40,
                  0.0, -0.0, np.inf, -np.inf]),
    ])
    with np.errstate(over="ignore"):
        want = d.astype(np.float16).view(np.uint16)
    got = oracle.round_to(d, "f16", lib=lib).view(np.uint16)
    np.testing.assert_array_equal(got, want)
    sub = np.concatenate([d[:200], d[-16:-2], d[12000:12200]])
    sub = sub[np.abs(sub) < 65504.0]
    np.testing.assert_array_equal(oracle.round_to(sub, "f16", lib=lib).astype(np.float64), _brute_round(sub, "f16"))
    assert np.isnan(oracle.round_to(np.array([np.nan]), "f16", lib=lib)[0])


def non_affine(lib):
    """Without gamma: the finite-difference gradient of sum dy * y, the RMS
    invariant with w = 1, and (gamma = 1, offset = 0) giving the same values."""
    rng = np.random.default_rng(21)
    for M, N, eps in ((2, 1, 1e-6), (3, 5, 0.5), (2, 16, 1e-6)):
        v = _rand(rng, (M, N))
        dy = _rand(rng, (M, N))
        y, rstd = oracle.fwd(v, None, "f64", eps, 0.0, lib=lib)
        ms = np.mean(v * v, axis=1)
        np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + _f32(eps))), rtol=1e-13)
        out = oracle.bwd(dy, v, None, "f64", eps, 0.0, lib=lib)
        assert out["dgamma64"] is None
        s = _cancel_scale(v, np.ones(N), dy, eps, 0.0, out)
        for i in range(M):
            for j in range(N):
                h = 1e-6 * max(1.0, abs(v[i, j]))
                vp, vm = v.copy(), v.copy()
                vp[i, j] += h
                vm[i, j] -= h
                lp = float(np.sum(dy * oracle.fwd(vp, None, "f64", eps, 0.0, lib=lib)[0]))
                lm = float(np.sum(dy * oracle.fwd(vm, None, "f64", eps, 0.0, lib=lib)[0]))
                fd = (lp - lm) / (vp[i, j] - vm[i, j])
                ref = out["dx64"][i, j]
                assert abs(fd - ref) <= 1e-7 * max(abs(ref), s[i, j]), (M, N, i, j, fd, ref)
        y1, _ = oracle.fwd(v, np.ones(N), "f64", eps, 0.0, lib=lib)
        np.testing.assert_array_equal(y, y1)
        np.testing.assert_array_equal(out["dx64"], oracle.bwd(dy, v, np.ones(N), "f64", eps, 0.0, lib=lib)["dx64"])
    try:
        oracle.fwd(np.ones((1, 2)), None, "f64", 1e-6, 1.0, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("offset without gamma must be refused")


ALL_PINS = [
    finite_differences, rms_invariant, orthogonality, closed_form_n1, constant_row, scale_invariance,
    offset_equivalence, fused_reductions, torch_fp64, golden, storage_widening, rounding, binary16, non_affine,
    e4m3_brute_force, e4m3_torch, fp8_forward,
    ln_finite_differences, ln_identities, ln_closed_forms, ln_torch_fp64, floor_magnitudes,
]
