"""Pins for the oracle's percentile-clipped per-row int8 quantizer."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int8 as oi8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_cases():
    with open(os.path.join(GOLDEN, "int8_clip_worked.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        w = np.array(c["w"], dtype=np.float32)
        q, s = oi8.quantize_rows_int8_clip(w, c["p"])
        clip = oi8.row_percentile(np.abs(w), c["p"])
        clip = np.where(clip == 0, np.abs(w).max(axis=1), clip)
        assert np.array_equal(clip, np.array(c["clip"], dtype=np.float32)), c["note"]
        assert np.array_equal(s, np.array(c["scale"], dtype=np.float32)), c["note"]
        assert np.array_equal(q, np.array(c["q"], dtype=np.int8)), c["note"]


@pytest.mark.parametrize("K", [1, 2, 7, 100, 1000, 4096])
def test_percentile_is_numpys(K):
    """The fp32 steps equal NumPy's own percentile (the routine the pages
    call) bit for bit."""
    rng = np.random.default_rng(K)
    v = np.abs(rng.standard_normal((40, K)) * rng.uniform(1e-3, 1e3, size=(40, 1))).astype(np.float32)
    v[0] = 0
    v[1, : K // 2] = 0
    for p in (0.0, 0.1, 1.0, 25.0, 33.3, 50.0, 66.7, 75.0, 99.0, 99.9, 99.99, 100.0):
        ref = np.percentile(v, p, axis=1)
        assert ref.dtype == np.float32
        assert np.array_equal(oi8.row_percentile(v, p).view(np.uint32), ref.view(np.uint32)), p


def test_percentile_100_is_the_absmax_quantizer():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    w[4] = 0
    q1, s1 = oi8.quantize_rows_int8_clip(w, 100.0)
    q2, s2 = oi8.quantize_rows_int8(w)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_clipped_elements_saturate_and_others_are_nearest():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((6, 200)).astype(np.float32)
    w[:, 7] *= 50                                            # outliers above the clip
    q, s = oi8.quantize_rows_int8_clip(w, 99.0)
    clip = oi8.row_percentile(np.abs(w), 99.0)
    for r in range(6):
        for k in range(200):
            x = w[r, k]
            if abs(x) >= clip[r]:
                assert abs(int(q[r, k])) == 127 and np.sign(q[r, k]) == np.sign(x)
            else:
                t = Fraction(float(np.float32(x) / np.float32(s[r])))     # the fp32 quotient
                best = min(range(-128, 128), key=lambda c: (abs(t - c), c % 2))
                assert int(q[r, k]) == best


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oi8.quantize_rows_int8_clip(np.zeros((2, 4), np.float32), 101.0)
    w = np.zeros((2, 4), np.float32)
    w[0, 1] = np.nan
    with pytest.raises(ValueError):
        oi8.quantize_rows_int8_clip(w, 50.0)
