"""The fp64 reference against facts fixed outside it (CPU only)."""

import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


def test_rejects_bad_arguments(oracle_lib):
    v = np.zeros((2, 3))
    with pytest.raises(ValueError):
        oracle_lib_call = oracle.fwd(v[:, :0], np.zeros(0), "f64", 1e-6, 0.0, lib=oracle_lib)  # N = 0
    with pytest.raises(TypeError):
        oracle.fwd(v.astype(np.float32), np.zeros(3), "f64", 1e-6, 0.0, lib=oracle_lib)
    src, dst = np.zeros(4), np.zeros(4, np.uint16)
    assert oracle_lib.oracle_round(4, src.ctypes.data, 4, dst.ctypes.data) != 0  # unknown storage code
    assert oracle_lib.oracle_round(3, src.ctypes.data, 4, dst.ctypes.data) == 0  # binary16


def test_zero_rows(oracle_lib):
    y, rstd = oracle.fwd(np.zeros((0, 5)), np.ones(5), "f64", 1e-6, 0.0, lib=oracle_lib)
    assert y.shape == (0, 5) and rstd.shape == (0,)
    out = oracle.bwd(np.zeros((0, 5)), np.zeros((0, 5)), np.ones(5), "f64", 1e-6, 0.0, lib=oracle_lib)
    np.testing.assert_array_equal(out["dgamma64"], np.zeros(5))


def test_thread_count_does_not_change_results(oracle_lib):
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 300))
    dy = rng.standard_normal((64, 300))
    g = 1 + 0.1 * rng.standard_normal(300)
    n0 = oracle.num_threads(oracle_lib)
    try:
        oracle.set_num_threads(1, oracle_lib)
        a = oracle.bwd(dy, v, g, "f64", 1e-6, 0.0, lib=oracle_lib)
        oracle.set_num_threads(max(n0, 3), oracle_lib)
        b = oracle.bwd(dy, v, g, "f64", 1e-6, 0.0, lib=oracle_lib)
    finally:
        oracle.set_num_threads(n0, oracle_lib)
    for k in ("dx64", "dgamma64", "c64", "sabs64"):
        np.testing.assert_array_equal(a[k], b[k])
