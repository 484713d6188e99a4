"""The seeded input generator is deterministic and packs bf16 by nearest-even (CPU only)."""

import numpy as np
import torch

import rmsnorm_inputs as ri


def test_deterministic_and_ordered():
    a = ri.make_inputs(8, 16, "bf16", fused=True, seed=0)
    b = ri.make_inputs(8, 16, "bf16", fused=True, seed=0)
    assert list(a) == ["x", "residual", "dy", "dh", "gamma"]
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    c = ri.make_inputs(8, 16, "bf16", fused=True, seed=1)
    assert not np.array_equal(a["x"], c["x"])


def test_sampled_rows_match_full_draw():
    full = ri.make_inputs(50, 24, "f32", gemma=True)
    rows = ri.sample_rows(50, 7)
    part = ri.make_inputs(50, 24, "f32", gemma=True, rows=rows)
    assert rows[0] == 0 and rows[-1] == 49
    for k in ("x", "dy"):
        np.testing.assert_array_equal(part[k], full[k][rows])
    np.testing.assert_array_equal(part["gamma"], full["gamma"])


def test_bf16_packing_matches_torch():
    rng = np.random.default_rng(5)
    f = rng.standard_normal(100000).astype(np.float32) * 3
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ri.f32_to_bf16_bits(f), want)


def test_gamma_recipes():
    g = ri.bf16_bits_to_f32(ri.make_inputs(4, 4096, "bf16")["gamma"])
    assert abs(float(g.mean()) - 1.0) < 0.01 and 0.08 < float(g.std()) < 0.12
    g2 = ri.make_inputs(4, 4096, "f32", gemma=True)["gamma"]
    assert abs(float(g2.mean())) < 0.01 and 0.08 < float(g2.std()) < 0.12


def test_algorithmic_bytes():
    assert ri.algorithmic_bytes("fwd", 4096, 4096, 2) == 67_133_440
    assert ri.algorithmic_bytes("bwd", 4096, 4096, 2) == 100_696_064
    assert ri.algorithmic_bytes("fused_fwd", 16384, 7168, 2) == 939_603_968
    assert ri.algorithmic_bytes("bwd", 16384, 6144, 4) == 1_208_074_240
