"""Pins for the oracle's row int8 quantizer, int8 matmul and W8A8 forward."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int8 as oi8

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "int8_worked.json")) as f:
        return json.load(f)


def test_quantize_rows_golden():
    g = _golden()
    q, s = oi8.quantize_rows_int8(np.array(g["rows"], dtype=np.float32))
    assert np.array_equal(q, np.array(g["q"], dtype=np.int8))
    assert np.array_equal(s, np.array(g["scale"], dtype=np.float32))


def test_matmul_golden():
    g = _golden()
    c = oi8.int8_matmul_int32(np.array(g["a"]), np.array(g["b"]))
    assert np.array_equal(c, np.array(g["c"]))


def test_matmul_against_python_ints():
    rng = np.random.default_rng(30)
    a = rng.integers(-128, 128, size=(5, 37)).astype(np.int8)
    b = rng.integers(-128, 128, size=(3, 37)).astype(np.int8)
    c = oi8.int8_matmul_int32(a, b)
    for i in range(5):
        for j in range(3):
            assert c[i, j] == sum(int(a[i, k]) * int(b[j, k]) for k in range(37))


def test_overflow_bound_closed_form():
    # |acc| <= 128*128*K; the extreme is reached by -128 * -128 everywhere
    K = 4096
    a = np.full((1, K), -128, dtype=np.int8)
    c = oi8.int8_matmul_int32(a, a)
    assert c[0, 0] == 128 * 128 * K == 2 ** 26


def test_quantizer_invariants():
    rng = np.random.default_rng(31)
    v = (rng.standard_normal((64, 300)) * rng.uniform(1e-3, 1e3, size=(64, 1))).astype(np.float32)
    v[5] = 0.0
    q, s = oi8.quantize_rows_int8(v)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(q.astype(np.int32)).max() <= 127        # -128 unreachable with absmax
    assert s[5] == 1.0 and (q[5] == 0).all()
    # the absmax element of every non-zero row maps to +-127
    nz = np.abs(v).max(axis=1) > 0
    assert (np.abs(q[nz].astype(np.int32)).max(axis=1) == 127).all()
    # round-trip error <= s (1/2 + 127.5 * 2^-23)
    err = np.abs(v.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert (err <= s[:, None] * (0.5 + 127.5 * 2.0 ** -23)).all()


def test_quantizer_nearest_brute_force():
    rng = np.random.default_rng(32)
    v = rng.standard_normal((6, 50)).astype(np.float32)
    q, s = oi8.quantize_rows_int8(v)
    cands = np.arange(-128, 128, dtype=np.float64)
    for r in range(6):
        for k in range(50):
            d = np.abs(float(v[r, k]) - cands * float(s[r]))
            best = cands[d == d.min()]
            t = float(v[r, k]) / float(s[r])
            if abs(abs(t - np.floor(t)) - 0.5) < 2.0 ** -18:
                continue    # within fp32 rounding of a tie: either neighbour
            assert q[r, k] in best


def test_w8a8_brute_force_fractions():
    rng = np.random.default_rng(33)
    M, K, N = 2, 16, 8
    x = rng.standard_normal((M, K)).astype(np.float32)
    wq = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sw = (rng.random(N) * 0.01 + 1e-3).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    xq, sx, acc, y, D = oi8.w8a8_forward(x, wq, sw, bias=bias)
    for m in range(M):
        for n in range(N):
            a = sum(int(xq[m, k]) * int(wq[n, k]) for k in range(K))
            assert acc[m, n] == a
            exact = Fraction(a) * Fraction(float(sx[m])) * Fraction(float(sw[n])) + Fraction(float(bias[n]))
            assert abs(y[m, n] - float(exact)) <= 1e-12 * (abs(float(exact)) + 1)
            dex = sum(abs(int(xq[m, k]) * int(wq[n, k])) for k in range(K)) * float(sx[m]) * float(sw[n])
            assert abs(D[m, n] - dex) <= 1e-12 * (dex + 1e-300)


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        oi8.quantize_rows_int8(np.array([[1.0, np.nan]], dtype=np.float32))


def test_exact_int_matmul_both_routes_against_python_ints():
    # the fp64 route (bound below 2^53) and the int64 route (bound above it)
    # must both give the exact integer sums
    rng = np.random.default_rng(34)
    a = rng.integers(-128, 128, size=(4, 300)).astype(np.int64)
    b = rng.integers(-128, 128, size=(300, 5)).astype(np.int64)
    big_a = a * (1 << 20)
    big_b = b * (1 << 20)        # 2^27 * 2^27 * 300 > 2^53: int64 route, still < 2^63
    for x, y in ((a, b), (big_a, big_b)):
        c = oi8.exact_int_matmul(x, y)
        assert c.dtype == np.int64
        for i in range(4):
            for j in range(5):
                assert int(c[i, j]) == sum(int(x[i, k]) * int(y[k, j]) for k in range(300))


def test_exact_int_matmul_cancelling_sums():
    # products near 2^40 that cancel pairwise, leaving a sum whose low bits
    # an inexact product would lose
    K = 64
    a = np.full((1, K), (1 << 20) + 1, dtype=np.int64)
    b = np.full((K, 1), (1 << 20) - 1, dtype=np.int64)
    b[::2] = -((1 << 20) - 1)
    b[0] = (1 << 20) + 3
    want = sum(int(a[0, k]) * int(b[k, 0]) for k in range(K))
    assert int(oi8.exact_int_matmul(a, b)[0, 0]) == want


def test_workload_sized_int8_product_matches_int64():
    # the fp64 route on a 64 x 4096 x 64 block of int8 extremes equals int64
    rng = np.random.default_rng(35)
    a = rng.choice(np.array([-128, 127, -127, 0], dtype=np.int8), size=(64, 4096))
    b = rng.choice(np.array([-128, 127, 1, -1], dtype=np.int8), size=(64, 4096))
    assert np.array_equal(oi8.int8_matmul_int32(a, b), a.astype(np.int64) @ b.astype(np.int64).T)
