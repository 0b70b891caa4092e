"""Pins for the oracle's per-column int4 packer and W4A8 linear."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int8 as oi8
from oracle import w4a8 as ow4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "w4a8_worked.json")) as f:
        return json.load(f)


def test_golden_pack():
    g = _golden()
    packed, s = ow4.pack_weight_int4(np.array(g["w"], dtype=np.float32))
    assert np.array_equal(packed, np.array(g["packed"], dtype=np.uint8))
    assert np.array_equal(s, np.array(g["scale"], dtype=np.float32))
    assert np.array_equal(ow4.unpack_weight_int4(packed), np.array(g["codes"], dtype=np.uint8))


def test_golden_forward():
    g = _golden()
    xq, sx, acc, y, _ = ow4.w4a8_forward(np.array(g["x"], dtype=np.float32),
                                         np.array(g["packed"], dtype=np.uint8),
                                         np.array(g["scale"], dtype=np.float32))
    assert np.array_equal(xq, np.array(g["xq"], dtype=np.int8))
    assert np.array_equal(sx, np.array(g["sx"], dtype=np.float32))
    assert np.array_equal(acc, np.array(g["acc"], dtype=np.int64))
    assert np.array_equal(y, np.array(g["y"]))


def _nearest_code(r):
    """Brute force: the code c in 0..15 whose value c - 8 is nearest to the
    exact rational r, ties to the even value."""
    best = None
    for c in range(16):
        d = abs(Fraction(r) - (c - 8))
        key = (d, (c - 8) % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_codes_are_nearest_by_brute_force():
    rng = np.random.default_rng(11)
    K, N = 24, 7
    w = (rng.standard_normal((K, N)) * rng.uniform(1e-3, 50, size=(1, N))).astype(np.float32)
    w[5, 2] = -w[:, 2].max() * 1.0   # make a column's absmax negative
    w[:, 4] = 0.0
    packed, s = ow4.pack_weight_int4(w)
    codes = ow4.unpack_weight_int4(packed)
    for n in range(N):
        for k in range(K):
            r = np.float32(w[k, n]) / np.float32(s[n])          # the fp32 quotient
            assert codes[k, n] == _nearest_code(float(r)), (k, n)


def test_column_extreme_maps_to_seven_and_no_code_is_zero():
    rng = np.random.default_rng(12)
    w = rng.standard_normal((64, 33)).astype(np.float32)
    packed, s = ow4.pack_weight_int4(w)
    codes = ow4.unpack_weight_int4(packed).astype(int)
    am = np.argmax(np.abs(w), axis=0)
    for n in range(w.shape[1]):
        assert codes[am[n], n] - 8 == (7 if w[am[n], n] > 0 else -7)
    assert codes.min() >= 1 and codes.max() <= 15    # |w| / s <= 7: value -8 never used


def test_round_trip_bound():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((128, 40)) * 0.02).astype(np.float32)
    packed, s = ow4.pack_weight_int4(w)
    wd = (ow4.unpack_weight_int4(packed).astype(np.float64) - 8) * s.astype(np.float64)[None, :]
    err = np.abs(wd - w.astype(np.float64))
    assert (err <= s.astype(np.float64)[None, :] * (0.5 + 1e-6)).all()


def test_nibble_order_even_k_high():
    w = np.zeros((4, 1), dtype=np.float32)
    w[:, 0] = [7.0, 1.0, -7.0, 0.0]    # scale 1: codes 15, 9, 1, 8
    packed, _ = ow4.pack_weight_int4(w)
    assert packed[:, 0].tolist() == [0xF9, 0x18]


def test_forward_is_w8a8_on_unpacked_values():
    """W4A8 equals the (separately pinned) W8A8 oracle run on the int8 values
    code - 8 in the [N, K] layout with the same per-column scales."""
    rng = np.random.default_rng(14)
    M, K, N = 5, 96, 11
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((K, N)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    packed, s = ow4.pack_weight_int4(w)
    w8 = (ow4.unpack_weight_int4(packed).astype(np.int16) - 8).T.astype(np.int8)
    a = ow4.w4a8_forward(x, packed, s, bias=bias)
    b = oi8.w8a8_forward(x, w8, s, bias=bias)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("M", [1, 3])
def test_forward_against_exact_rationals(M):
    rng = np.random.default_rng(20 + M)
    K, N = 10, 6
    x = (rng.standard_normal((M, K)) * 3).astype(np.float16).astype(np.float32)
    w = rng.standard_normal((K, N)).astype(np.float32)
    packed, s = ow4.pack_weight_int4(w)
    xq, sx, acc, y, D = ow4.w4a8_forward(x, packed, s)
    codes = ow4.unpack_weight_int4(packed)
    for m in range(M):
        for n in range(N):
            tot = sum(int(xq[m, k]) * (int(codes[k, n]) - 8) for k in range(K))
            assert acc[m, n] == tot
            exact = Fraction(tot) * Fraction(float(sx[m])) * Fraction(float(s[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 50)
            dex = sum(abs(int(xq[m, k])) * abs(int(codes[k, n]) - 8) for k in range(K))
            assert D[m, n] == pytest.approx(dex * float(sx[m]) * float(s[n]), rel=1e-14)


def test_zero_input_gives_bias():
    w = np.random.default_rng(15).standard_normal((32, 8)).astype(np.float32)
    packed, s = ow4.pack_weight_int4(w)
    bias = np.arange(8, dtype=np.float32)
    _, _, acc, y, _ = ow4.w4a8_forward(np.zeros((2, 32), np.float32), packed, s, bias=bias)
    assert not acc.any()
    assert np.array_equal(y, np.broadcast_to(bias.astype(np.float64), (2, 8)))


def test_rejects_bad_inputs():
    with pytest.raises(ValueError):
        ow4.pack_weight_int4(np.zeros((3, 4), np.float32))
    w = np.zeros((4, 4), np.float32)
    w[1, 1] = np.inf
    with pytest.raises(ValueError):
        ow4.pack_weight_int4(w)
