"""Pins for the oracle's affine quantize / pack / unpack / dequantize / forward.

Each check compares the oracle with something other than itself: values
worked by hand (tests/golden), exact rational arithmetic on tiny inputs,
brute-force searches over every code, closed-form bounds and identities.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import affine, codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- bit order
def test_bit_order_golden():
    for case in _load("affine_bitorder.json")["cases"]:
        bits = case["bits"]
        codes = np.array([case["codes"]], dtype=np.uint8)
        words = np.array([[int(h, 16) for h in case["words_hex"]]], dtype=np.uint32)
        assert np.array_equal(affine.affine_pack(codes, bits), words), case
        assert np.array_equal(affine.affine_unpack(words, codes.shape[1], bits), codes), case


def test_pack_unpack_bijection_random_words():
    rng = np.random.default_rng(1)
    for bits in (1, 2, 3, 4, 5, 6, 8):
        words = rng.integers(0, 1 << 32, size=(5, 7 * bits), dtype=np.uint64).astype(np.uint32)
        codes = affine.affine_unpack(words, 7 * 32, bits)
        assert codes.max() < 2 ** bits
        assert np.array_equal(affine.affine_pack(codes, bits), words)


def test_bitstream_golden():
    with open(os.path.join(GOLDEN, "affine_bitstream.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        bits = case["bits"]
        codes = np.array([case["codes"]], dtype=np.uint8)
        words = np.array([[int(h, 16) for h in case["words_hex"]]], dtype=np.uint32)
        assert np.array_equal(affine.affine_pack(codes, bits), words), case["note"]
        assert np.array_equal(affine.affine_unpack(words, codes.shape[1], bits), codes), case["note"]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
def test_pack_matches_big_integer_stream(bits):
    """A row as one Python integer: sum_k q_k * 2^(bits*k); word i is bits
    32 i .. 32 i + 31 of it."""
    rng = np.random.default_rng(bits)
    K = 96
    codes = rng.integers(0, 2 ** bits, size=(3, K)).astype(np.uint8)
    words = affine.affine_pack(codes, bits)
    for n in range(3):
        v = sum(int(codes[n, k]) << (bits * k) for k in range(K))
        ref = [(v >> (32 * i)) & 0xFFFFFFFF for i in range(K * bits // 32)]
        assert [int(u) for u in words[n]] == ref


def _python_unpack(word_row, K, bits):
    """Independent per-element bit extraction, plain Python ints: the row's
    words as one integer, code k = its bits bits*k .. bits*k + bits - 1."""
    v = sum(int(u) << (32 * i) for i, u in enumerate(word_row))
    return [(v >> (bits * k)) & ((1 << bits) - 1) for k in range(K)]


# --------------------------------------------------------- worked quantization
def test_worked_quantization_golden():
    g = _load("affine_quant_worked.json")
    w = np.array(g["w"], dtype=np.float32)
    for sb in ("f32", "bf16", "f16"):   # every parameter is exact in all three
        q, s, b = affine.affine_quantize(w, g["bits"], g["group_size"], sb)
        assert np.array_equal(q, np.array(g["codes"], dtype=np.uint8)), sb
        assert np.array_equal(s, np.array(g["scales"], dtype=np.float32)), sb
        assert np.array_equal(b, np.array(g["biases"], dtype=np.float32)), sb
        words = affine.affine_pack(q, g["bits"])
        assert [f"{int(v):08X}" for v in words[0]] == g["words_hex"][0]
        deq = affine.affine_dequantize(q, s, b, g["group_size"])
        assert np.array_equal(deq, np.array(g["dequantized"]))
        fx = g["forward"]
        y, _ = affine.affine_forward(np.array(fx["x"]), q, s, b, g["group_size"],
                                     bias=np.array(fx["bias"]))
        assert np.array_equal(y, np.array(fx["y"]))


# ------------------------------------------------------- quantizer properties
CASES = [(4, 64, "f32"), (4, 64, "bf16"), (4, 128, "bf16"), (4, 32, "f16"),
         (2, 64, "bf16"), (8, 128, "f32"), (8, 32, "bf16"), (1, 32, "f32"),
         (3, 64, "bf16"), (3, 32, "f32"), (5, 128, "f16"), (6, 64, "bf16"), (6, 32, "f32")]


def _weights(seed, N=24, K=256, std=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K)) * std).astype(np.float32)


@pytest.mark.parametrize("bits,G,sb", CASES)
def test_shapes_and_code_range(bits, G, sb):
    w = _weights(2)
    q, s, b = affine.affine_quantize(w, bits, G, sb)
    assert q.shape == w.shape and q.dtype == np.uint8
    assert s.shape == (w.shape[0], w.shape[1] // G) and b.shape == s.shape
    assert q.max() <= 2 ** bits - 1
    assert affine.affine_pack(q, bits).shape == (w.shape[0], w.shape[1] * bits // 32)
    # stored parameters are representable in the storage dtype
    assert np.array_equal(codecs.round_to_dtype(s, sb), s)
    assert np.array_equal(codecs.round_to_dtype(b, sb), b)
    # every group reaches code 0 (its minimum maps to about 0) for f32 storage
    if sb == "f32":
        assert (q.reshape(w.shape[0], -1, G).min(axis=2) == 0).all()


@pytest.mark.parametrize("bits,G,sb", CASES)
def test_nearest_code_brute_force(bits, G, sb):
    """q minimises |w - (s*c + b)| over every c, ties to the even c.

    Exact fp64 distances are computed for every candidate code.  The oracle's
    two fp32 roundings may only differ from the exact argmin where the exact
    quotient lies within 2^-20 of a tie.
    """
    w = _weights(3, N=8, K=128 if G <= 128 else G)
    q, s, b = affine.affine_quantize(w, bits, G, sb)
    N, K = w.shape
    sr = np.repeat(s.astype(np.float64), G, axis=1)
    br = np.repeat(b.astype(np.float64), G, axis=1)
    cands = np.arange(2 ** bits, dtype=np.float64)
    dist = np.abs(w.astype(np.float64)[:, :, None] - (sr[:, :, None] * cands + br[:, :, None]))
    best = dist.min(axis=2)
    is_best = dist <= best[:, :, None]
    # among tied minimisers prefer the even code
    even_pref = np.where(is_best, (cands % 2 == 0) * 2 + 1, 0)
    want = np.argmax(even_pref, axis=2)
    exact_t = (w.astype(np.float64) - br) / sr
    near_tie = np.abs(np.abs(exact_t - np.floor(exact_t)) - 0.5) < 2.0 ** -20
    ok = (q == want) | near_tie
    assert ok.all()


@pytest.mark.parametrize("bits,G,sb", CASES)
def test_roundtrip_error_bound(bits, G, sb):
    """|w - (s q + b)| <= s (1/2 + (2^b - 1/2) 2^-23) for unclamped elements."""
    w = _weights(4)
    q, s, b = affine.affine_quantize(w, bits, G, sb)
    sr = np.repeat(s.astype(np.float64), G, axis=1)
    br = np.repeat(b.astype(np.float64), G, axis=1)
    err = np.abs(w.astype(np.float64) - (sr * q + br))
    t = (w.astype(np.float64) - br) / sr
    unclamped = (t > -0.5) & (t < 2 ** bits - 0.5)
    bound = sr * (0.5 + (2 ** bits - 0.5) * 2.0 ** -23)
    assert (err[unclamped] <= bound[unclamped]).all()
    # clamped elements come only from rounding the parameters to the storage
    # dtype: |b32 - b| + (2^b - 1)|s32 - s| <= 2^-8 (|min| + (max - min))
    groups = w.reshape(w.shape[0], -1, G).astype(np.float64)
    mn = np.repeat(groups.min(axis=2), G, axis=1)
    mx = np.repeat(groups.max(axis=2), G, axis=1)
    pbound = 2.0 ** -8 * (np.abs(mn) + (mx - mn)) + bound
    assert (err <= pbound).all()
    # with fp32 parameters, or few enough codes that (2^b - 1) 2^-9 < 1/2,
    # zero-centred data clamps nothing
    if sb == "f32" or bits <= 4:
        assert unclamped.all()


def test_clamped_error_bound_adversarial_group():
    """A group far from zero: bf16 rounding of the bias exceeds s/2, so some
    elements clamp; their error stays within the parameter-rounding bound."""
    rng = np.random.default_rng(5)
    w = (1.004 + 0.01 * rng.random((4, 64))).astype(np.float32)
    bits, G = 4, 64
    q, s, b = affine.affine_quantize(w, bits, G, "bf16")
    mn = w.min(axis=1, keepdims=True).astype(np.float64)
    mx = w.max(axis=1, keepdims=True).astype(np.float64)
    err = np.abs(w - (s.astype(np.float64) * q + b.astype(np.float64)))
    bound = 2.0 ** -8 * (np.abs(mn) + (mx - mn)) + s.astype(np.float64) * (0.5 + 2.0 ** -18)
    assert (err <= bound).all()
    assert (err > s.astype(np.float64) / 2).any()   # the case really is adversarial


def test_degenerate_group_takes_unit_scale():
    w = np.full((2, 64), 0.375, dtype=np.float32)
    w[1, :] = -3.0
    for sb in ("f32", "bf16", "f16"):
        q, s, b = affine.affine_quantize(w, 4, 64, sb)
        assert (s == 1.0).all() and (q == 0).all()
        assert np.array_equal(affine.affine_dequantize(q, s, b, 64), w.astype(np.float64))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
def test_idempotent_on_exact_groups(bits):
    """Groups built as s*q + b with s a power of two, b a multiple of s and
    both extreme codes present re-quantize to the same codes and parameters."""
    rng = np.random.default_rng(6)
    N, K, G = 6, 128, 32
    qmax = 2 ** bits - 1
    q = rng.integers(0, qmax + 1, size=(N, K)).astype(np.uint8)
    q[:, ::G] = 0
    q[:, 1::G] = qmax
    s = (2.0 ** rng.integers(-9, -3, size=(N, K // G))).astype(np.float32)
    b = (s * rng.integers(-40, 40, size=(N, K // G))).astype(np.float32)
    w = affine.affine_dequantize(q, s, b, G).astype(np.float32)
    for sb in ("f32", "bf16"):
        q2, s2, b2 = affine.affine_quantize(w, bits, G, sb)
        assert np.array_equal(q2, q) and np.array_equal(s2, s) and np.array_equal(b2, b)


def test_rejects_bad_input():
    w = np.zeros((2, 64), dtype=np.float32)
    with pytest.raises(ValueError):
        affine.affine_quantize(w, 4, 48, "f32")
    with pytest.raises(ValueError):
        affine.affine_quantize(w, 7, 32, "f32")      # 7 bits is not a layer width
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        affine.affine_quantize(w, 4, 32, "f32")
    big = np.full((1, 32), 1e5, dtype=np.float32)
    big[0, 0] = -1e5
    with pytest.raises(ValueError):       # bias and scale overflow fp16
        affine.affine_quantize(big, 4, 32, "f16")


def test_dequantize_single_rounding_matches_fp32_fma():
    """fp32(s q + b computed exactly) == fma in fp32: checked against exact
    rational arithmetic element by element."""
    w = _weights(9, N=4, K=64)
    q, s, b = affine.affine_quantize(w, 4, 32, "bf16")
    deq32 = affine.affine_dequantize(q, s, b, 32).astype(np.float32)
    for n in range(4):
        for k in range(0, 64, 7):
            g = k // 32
            exact = Fraction(float(s[n, g])) * int(q[n, k]) + Fraction(float(b[n, g]))
            assert float(deq32[n, k]) == float(np.float32(float(exact)))


# --------------------------------------------------------------- forward pins
@pytest.mark.parametrize("bits,G", [(2, 8), (4, 8), (8, 8), (4, 16), (3, 32), (5, 32), (6, 16), (1, 32)])
def test_forward_brute_force_fractions(bits, G):
    """M=2, K=16 or 32, N=8: packed words unpacked by plain bit arithmetic
    and the product summed in exact rationals."""
    rng = np.random.default_rng(10 + bits)
    M, K, N = 2, max(16, G), 8
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    q, s, b = affine.affine_quantize(w, bits, G, "f32")
    words = affine.affine_pack(q, bits)
    y, D = affine.affine_forward(x, affine.affine_unpack(words, K, bits), s, b, G, bias=bias)
    for n in range(N):
        codes = _python_unpack(words[n], K, bits)
        wn = [Fraction(float(s[n, k // G])) * codes[k] + Fraction(float(b[n, k // G])) for k in range(K)]
        for m in range(M):
            exact = sum(Fraction(float(x[m, k])) * wn[k] for k in range(K)) + Fraction(float(bias[n]))
            dexact = sum(abs(Fraction(float(x[m, k])) * wn[k]) for k in range(K))
            assert abs(y[m, n] - float(exact)) <= 1e-12 * float(dexact) + 1e-300
            assert abs(D[m, n] - float(dexact)) <= 1e-12 * float(dexact)


def test_forward_one_hot_zero_and_linearity():
    rng = np.random.default_rng(11)
    M, K, N, G = 3, 64, 10, 32
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    q, s, b = affine.affine_quantize(w, 4, G, "bf16")
    deq = affine.affine_dequantize(q, s, b, G)
    for k in (0, 17, 63):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        y, _ = affine.affine_forward(e, q, s, b, G, bias=bias)
        assert np.array_equal(y[0], deq[:, k] + bias.astype(np.float64))
    y0, D0 = affine.affine_forward(np.zeros((2, K)), q, s, b, G, bias=bias)
    assert np.array_equal(y0, np.broadcast_to(bias.astype(np.float64), (2, N)))
    assert (D0 == 0).all()
    x1 = rng.standard_normal((M, K))
    x2 = rng.standard_normal((M, K))
    f = lambda xx: affine.affine_forward(xx, q, s, b, G)[0]
    assert np.allclose(f(2.5 * x1 + x2), 2.5 * f(x1) + f(x2), rtol=1e-12, atol=1e-12)
    # transposition check: a non-square product keeps [M, N]
    assert f(x1).shape == (M, N)
