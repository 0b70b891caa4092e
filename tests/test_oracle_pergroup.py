"""Pins for the oracle's per-group int8 quantizer and per-group linear."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int8 as oi8
from oracle import pergroup as opg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "pergroup_worked.json")) as f:
        return json.load(f)


def test_golden_quantizer():
    g = _golden()
    q, s = opg.quantize_groups_int8(np.array(g["w"], dtype=np.float32), g["group_size"])
    assert np.array_equal(q, np.array(g["q"], dtype=np.int8))
    assert np.array_equal(s, np.array(g["scale"], dtype=np.float32))


@pytest.mark.parametrize("xk,yk", [("x1", "y1"), ("x2", "y2")])
def test_golden_forward_both_branches(xk, yk):
    g = _golden()
    y, _ = opg.pergroup_forward(np.array(g[xk], dtype=np.float32), np.array(g["q"], dtype=np.int8),
                                np.array(g["scale"], dtype=np.float32), g["group_size"],
                                bias=np.array(g["bias"], dtype=np.float32))
    assert np.array_equal(y, np.array(g[yk]))


def test_one_group_is_the_row_quantizer():
    rng = np.random.default_rng(40)
    w = (rng.standard_normal((9, 256)) * rng.uniform(1e-3, 10, size=(9, 1))).astype(np.float32)
    w[3] = 0
    q, s = opg.quantize_groups_int8(w, 256)
    q_r, s_r = oi8.quantize_rows_int8(w)
    assert np.array_equal(q, q_r) and np.array_equal(s[0], s_r)


@pytest.mark.parametrize("G", [64, 128, 256])
def test_groups_are_independent_row_quantizations(G):
    rng = np.random.default_rng(41 + G)
    w = (rng.standard_normal((7, 4 * G)) * rng.uniform(1e-2, 1e2, size=(7, 4 * G))).astype(np.float32)
    w[2, G:2 * G] = 0                      # one all-zero group
    q, s = opg.quantize_groups_int8(w, G)
    assert s.shape == (4, 7)
    for g in range(4):
        q_r, s_r = oi8.quantize_rows_int8(w[:, g * G:(g + 1) * G])
        assert np.array_equal(q[:, g * G:(g + 1) * G], q_r)
        assert np.array_equal(s[g], s_r)
    assert s[1, 2] == 1.0


def test_single_group_forward_is_w8a8():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((5, 128)).astype(np.float32)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    q, s = opg.quantize_groups_int8(w, 128)
    y, D = opg.pergroup_forward(x, q, s, 128)
    _, _, _, y8, D8 = oi8.w8a8_forward(x, q, s[0])
    np.testing.assert_allclose(y, y8, rtol=1e-14, atol=0)
    np.testing.assert_allclose(D, D8, rtol=1e-14, atol=0)


def _brute(x, q, s, G, bias):
    """Exact rational forward of the definition, loops only."""
    M, K = x.shape
    N = q.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    if M == 1:
        for n in range(N):
            y[0][n] = sum(Fraction(float(x[0, k])) * int(q[n, k]) * Fraction(float(s[k // G, n]))
                          for k in range(K))
    else:
        xq, sx = oi8.quantize_rows_int8(x)
        for m in range(M):
            for n in range(N):
                tot = Fraction(0)
                for g in range(K // G):
                    acc = sum(int(xq[m, k]) * int(q[n, k]) for k in range(g * G, (g + 1) * G))
                    tot += acc * Fraction(float(s[g, n]))
                y[m][n] = tot * Fraction(float(sx[m]))
    return [[float(v + Fraction(float(bias[n]))) for n, v in enumerate(r)] for r in y]


@pytest.mark.parametrize("M", [1, 3])
def test_forward_against_exact_rationals(M):
    rng = np.random.default_rng(43 + M)
    K, G, N = 8, 4, 3
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    q, s = opg.quantize_groups_int8(w, G)
    y, _ = opg.pergroup_forward(x, q, s, G, bias=bias)
    np.testing.assert_allclose(y, np.array(_brute(x, q, s, G, bias)), rtol=1e-12, atol=1e-12)


def test_D_bounds_the_product():
    rng = np.random.default_rng(44)
    for M in (1, 4):
        x = rng.standard_normal((M, 256)).astype(np.float32)
        q, s = opg.quantize_groups_int8(rng.standard_normal((5, 256)).astype(np.float32), 64)
        y, D = opg.pergroup_forward(x, q, s, 64)
        assert (np.abs(y) <= D * (1 + 1e-12)).all()


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        opg.quantize_groups_int8(np.zeros((2, 100), np.float32), 64)
    with pytest.raises(ValueError):
        opg.quantize_groups_int8(np.full((2, 64), np.inf, np.float32), 64)
