"""Pins for the comparison rule: the bound 2e-2 * D / sqrt(K) + 1e-3 and the
half-ulp allowance of the output dtype."""

import numpy as np

from oracle.tolerance import tolerance, compare


def test_bound_closed_form():
    assert tolerance(64.0, 64) == 2e-2 * 64.0 / 8.0 + 1e-3
    assert tolerance(0.0, 4096) == 1e-3
    assert np.allclose(tolerance(np.array([1.0, 2.0]), 4), [0.011, 0.021])


def test_compare_counts():
    y_ref = np.array([[1.0, 8.0, 0.0, 100.0]])
    D = np.zeros_like(y_ref)        # bound is exactly 1e-3
    K = 16
    y = y_ref + np.array([[5e-4, 2e-2, 2e-3, 0.0]])
    r = compare(y, y_ref, D, K, "bf16")
    # 1.0 + 5e-4 passes strict; 8.02 fails strict but is within half a bf16
    # ulp at 8 (0.03125); 0.002 at 0 fails both; 100.0 passes
    assert r["strict_fail"] == 2
    assert r["allowed_fail"] == 1
    r = compare(np.array([[np.nan]]), np.array([[0.0]]), np.zeros((1, 1)), K, "f32")
    assert r["strict_fail"] == 1 and r["allowed_fail"] == 1
