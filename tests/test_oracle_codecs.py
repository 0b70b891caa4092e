"""Pins for the oracle's dtype codecs and its ulp helper.

The codecs are pinned against library routines (torch's CPU conversions,
NumPy's IEEE float16) and against closed-form spacings; none of these checks
retypes the oracle's own formula.
"""

import numpy as np
import torch

from oracle import codecs


def test_bf16_all_patterns_roundtrip():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = codecs.bf16_bits_to_f32(b)
    finite = np.isfinite(f)
    back = codecs.f32_to_bf16_bits(f[finite])
    assert np.array_equal(back, b[finite])
    # widening agrees with torch's own bf16 -> fp32
    t = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(t.view(np.uint32)[finite], f.view(np.uint32)[finite])


def _torch_bf16_bits(a):
    t = torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_narrowing_matches_torch_random_and_ties():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    a = u.view(np.float32)
    a = a[np.isfinite(a)]
    assert np.array_equal(codecs.f32_to_bf16_bits(a), _torch_bf16_bits(a))
    # exact ties on both parities, and values one ulp either side of a tie
    hi = rng.integers(0, 0x7F7F, size=20000, dtype=np.uint32)
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        v = ((hi << 16) | low).astype(np.uint32).view(np.float32)
        v = np.concatenate([v, -v])
        v = v[np.isfinite(v)]
        assert np.array_equal(codecs.f32_to_bf16_bits(v), _torch_bf16_bits(v))


def test_round_to_dtype_matches_torch():
    rng = np.random.default_rng(8)
    a = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(200_000) * 1e-6).astype(np.float32),
        (rng.standard_normal(200_000) * 3e4).astype(np.float32),
    ])
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        ref = torch.from_numpy(a).to(tdt).to(torch.float32).numpy()
        got = codecs.round_to_dtype(a, dt)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), dt


def test_half_ulp_closed_forms():
    # bf16 has 8 significant bits: spacing at 1.0 is 2^-7, at 8.0 it is 2^-4
    assert codecs.half_ulp(1.0, "bf16") == 2.0 ** -8
    assert codecs.half_ulp(8.0, "bf16") == 2.0 ** -5
    assert codecs.half_ulp(-9.5, "bf16") == 2.0 ** -5
    # fp16: 11 significant bits; fp32: 24
    assert codecs.half_ulp(1.0, "f16") == 2.0 ** -11
    assert codecs.half_ulp(1.0, "f32") == 2.0 ** -24
    # subnormal range: fp16 spacing bottoms out at 2^-24
    assert codecs.half_ulp(1e-7, "f16") == 2.0 ** -25
    # zero takes the smallest (subnormal) spacing of the dtype
    assert codecs.half_ulp(0.0, "bf16") == 2.0 ** -134
    assert codecs.half_ulp(0.0, "f16") == 2.0 ** -25
    # a value just below a power of two is given the wider spacing above it
    just_below = np.nextafter(np.float32(2.0), np.float32(0))
    assert codecs.half_ulp(float(just_below), "bf16") == 2.0 ** -7
