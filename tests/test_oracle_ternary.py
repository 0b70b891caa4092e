"""Pins for the oracle's ternary BitLinear pack / decode / forward."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ternary

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "ternary_worked.json")) as f:
        return json.load(f)


def test_layout_golden():
    g = _golden()
    t = np.array(g["t"], dtype=np.int8)
    packed = np.array(g["packed"], dtype=np.uint8)
    assert np.array_equal(ternary.ternary_pack(t), packed)
    assert np.array_equal(ternary.ternary_unpack(packed, t.shape[0]), t)


def test_forward_golden_multiply_and_invert():
    g = _golden()
    packed = np.array(g["packed"], dtype=np.uint8)
    x = np.array(g["x"])
    y, _ = ternary.ternary_forward(x, packed, 8, g["weight_scale"], invert=False)
    assert np.array_equal(y, np.array(g["y_multiply"]))
    y, _ = ternary.ternary_forward(x, packed, 8, g["weight_scale"], invert=True)
    assert np.array_equal(y, np.array(g["y_invert"]))


def test_roundtrip_and_value_set():
    rng = np.random.default_rng(20)
    t = rng.integers(-1, 2, size=(36, 40)).astype(np.int8)
    packed = ternary.ternary_pack(t)
    assert packed.shape == (9, 40) and packed.dtype == np.uint8
    d = ternary.ternary_unpack(packed, 36)
    assert set(np.unique(d)) <= {-1, 0, 1}
    assert np.array_equal(d, t)
    # the packer never emits code 3
    for j in range(4):
        assert (((packed >> (2 * j)) & 3) != 3).all()


def test_code_three_decodes_literally():
    packed = np.full((1, 5), 0xFF, dtype=np.uint8)
    assert (ternary.ternary_unpack(packed, 4) == 2).all()


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        ternary.ternary_pack(np.zeros((6, 4), dtype=np.int8))
    with pytest.raises(ValueError):
        ternary.ternary_pack(np.full((4, 4), 2, dtype=np.int8))


def test_brute_force_fractions():
    """M=2, K=16, N=8, fields decoded by plain Python bit arithmetic."""
    rng = np.random.default_rng(21)
    M, K, N = 2, 16, 8
    x = rng.standard_normal((M, K)).astype(np.float32)
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    bias = rng.standard_normal(N).astype(np.float32)
    packed = ternary.ternary_pack(t)
    for invert in (False, True):
        ws = 0.050048828125
        y, D = ternary.ternary_forward(x, packed, N, ws, invert=invert, bias=bias)
        sigma = 1 / Fraction(ws) if invert else Fraction(ws)
        R = N // 4
        for n in range(N):
            r, j = n % R, n // R
            vals = [((int(packed[r, k]) >> (2 * j)) & 3) - 1 for k in range(K)]
            for m in range(M):
                acc = sum(Fraction(float(x[m, k])) * vals[k] for k in range(K))
                exact = sigma * acc + Fraction(float(bias[n]))
                dex = sigma * sum(abs(Fraction(float(x[m, k])) * vals[k]) for k in range(K))
                assert abs(y[m, n] - float(exact)) <= 1e-12 * (float(dex) + 1)
                assert abs(D[m, n] - float(dex)) <= 1e-12 * (float(dex) + 1e-300)


def test_identities():
    rng = np.random.default_rng(22)
    N, K = 12, 20
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    packed = ternary.ternary_pack(t)
    ws = 0.25
    bias = rng.standard_normal(N)
    # one-hot x picks sigma * t[:, k]
    for k in (0, 7, 19):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        y, _ = ternary.ternary_forward(e, packed, N, ws)
        assert np.array_equal(y[0], ws * t[:, k].astype(np.float64))
    # all codes 1 (value 0) -> y = bias
    zero_pack = ternary.ternary_pack(np.zeros((N, K), dtype=np.int8))
    y, _ = ternary.ternary_forward(rng.standard_normal((3, K)), zero_pack, N, ws, bias=bias)
    assert np.array_equal(y, np.broadcast_to(bias, (3, N)))
    # x = ones -> sigma * (#plus - #minus), exact
    y, _ = ternary.ternary_forward(np.ones((1, K)), packed, N, ws)
    want = ws * ((t == 1).sum(axis=1) - (t == -1).sum(axis=1))
    assert np.array_equal(y[0], want.astype(np.float64))
