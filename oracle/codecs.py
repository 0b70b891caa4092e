"""Floating-point storage codecs used by the oracle (test infrastructure only).

The layer stores activations, outputs and quantization parameters in fp32,
fp16 or bf16 (the QuantizedLinear page stores scales and biases beside the
packed weight; the BitLinear page requires the input dtype to equal the
weight-scale dtype and returns that dtype).  Narrowing is round-to-nearest,
ties-to-even (RNE); widening is exact.

bf16 is the top half of an fp32 word, so RNE narrowing is the integer rule
``(u + 0x7FFF + ((u >> 16) & 1)) >> 16`` on the fp32 bit pattern ``u``.
fp16 narrowing uses NumPy's IEEE ``astype(np.float16)``.
"""

import numpy as np

DTYPES = ("f32", "f16", "bf16")

# significand bits (including the implicit one) and minimum normal exponent
_PRECISION = {"f32": (24, -126), "f16": (11, -14), "bf16": (8, -126)}


def f32_to_bf16_bits(a):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite by construction; NaN maps to the quiet NaN 0x7FC0.
    """
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b):
    """bf16 bit patterns (uint16) -> fp32 values (exact widening)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_dtype(a, dtype):
    """Round fp32 values to the storage dtype and widen back to fp32.

    The result holds exactly the values a tensor of ``dtype`` would store.
    """
    a = np.asarray(a, dtype=np.float32)
    if dtype == "f32":
        return a.copy()
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(a))
    if dtype == "f16":
        with np.errstate(over="ignore"):   # overflow to inf is the IEEE result
            return a.astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def half_ulp(v, dtype):
    """Half the spacing of ``dtype`` values around |v| (fp64 array).

    The spacing is taken from the binade of |v| enlarged by one part in
    2^precision, so a value just below a power of two that rounds up is given
    the wider spacing of the binade above it.
    """
    p, emin = _PRECISION[dtype]
    v = np.abs(np.asarray(v, dtype=np.float64)) * (1.0 + 2.0 ** -p)
    _, e = np.frexp(v)            # v = m * 2**e with m in [0.5, 1); 0 -> e = 0
    e = np.where(v == 0, emin, np.maximum(e - 1, emin))  # floor(log2 v), clamped
    return np.ldexp(0.5, e - (p - 1))
