"""Group-wise affine n-bit weights: quantize, pack, unpack, dequantize, forward.

Test infrastructure only (see the package docstring).

Sources on the pages:
  * "Struct QuantizedLinear" (nuvec-nn docs), Fields: ``weight`` is uint32
    ``[output_dims, input_dims*bits/32]``; ``scales`` holds one scale per group
    of ``group_size`` input values, ``[output_dims, input_dims/group_size]``;
    ``biases`` is shaped like ``scales``; ``bias`` is the optional layer bias.
  * same page, ``from_linear``: groups of 32, 64 or 128 input values, bits in
    1-6 or 8, the layer bias kept; ``dequantized_weight`` returns
    ``[output_dims, input_dims]``; ``forward`` is x W^T + b over the last axis.
  * "cider/ops.py", ``pergroup_linear`` docstring (MLX affine format):
    ``q = clip(round((w - biases)/scales), 0, 2^b - 1)`` and
    ``w = q*scale + bias``.

Readings where the pages are silent (all listed in the design notes):
  * scale = (max - min)/(2^b - 1) and bias = min per group, both computed in
    fp32 and then rounded (RNE) to the storage dtype; codes are computed
    against the *stored* scale and bias;
  * round() is half-to-even (the cider quantizers use ``np.round``);
  * a group whose stored scale is zero (max == min) takes scale 1, following
    the zero-scale guard of the cider quantizers, so its codes are all 0;
  * codes are packed LSB-first into one bit stream per row along K: code k
    occupies stream bits ``bits*k .. bits*k + bits - 1`` (its least
    significant bit first), and stream bit i is bit ``i mod 32`` of
    little-endian uint32 word ``i // 32``.  For widths that divide 32 this
    puts code k at bit ``bits*(k mod (32/bits))`` of word ``k // (32/bits)``;
    for 3, 5 and 6 bits a code may straddle two words (the packed width
    ``input_dims*bits/32`` implies dense packing).
"""

import numpy as np

from .codecs import round_to_dtype


BITS = (1, 2, 3, 4, 5, 6, 8)


def _check_bits(K, bits):
    if bits not in BITS:
        raise ValueError(f"bits={bits} not in {BITS}")
    if (K * bits) % 32:
        raise ValueError(f"K={K} does not fill whole uint32 words at {bits} bits")


def _check_shape(K, bits, group_size):
    if group_size <= 0 or K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    _check_bits(K, bits)


def affine_quantize(w, bits, group_size, sb_dtype):
    """Quantize fp32 weights ``[N, K]`` group-wise along K.

    Returns ``(codes uint8 [N, K], scales f32 [N, K/G], biases f32 [N, K/G])``;
    ``scales`` and ``biases`` hold exactly the values stored in ``sb_dtype``.
    Raises ValueError on non-finite weights or non-finite stored parameters.
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    _check_shape(K, bits, group_size)
    if not np.isfinite(w).all():
        raise ValueError("non-finite weight")
    qmax = 2 ** bits - 1
    groups = w.reshape(N, K // group_size, group_size)

    # 1. exact fp32 extremes of every group
    mn = groups.min(axis=2)
    mx = groups.max(axis=2)
    # 2. fp32 scale and bias:  scale = (max - min) / (2^b - 1),  bias = min
    s32 = (mx - mn) / np.float32(qmax)
    b32 = mn
    # 3. round both to the storage dtype
    s_st = round_to_dtype(s32, sb_dtype)
    b_st = round_to_dtype(b32, sb_dtype)
    if not (np.isfinite(s_st).all() and np.isfinite(b_st).all()):
        raise ValueError(f"scale or bias overflows {sb_dtype}")
    # 4. zero-scale guard
    s_st = np.where(s_st == 0, np.float32(1.0), s_st).astype(np.float32)
    # 5. q = clip(round((w - bias) / scale), 0, 2^b - 1), all in fp32
    t = (groups - b_st[:, :, None]) / s_st[:, :, None]
    q = np.clip(np.rint(t), 0, qmax).astype(np.uint8)
    return q.reshape(N, K), s_st, b_st


def affine_pack(codes, bits):
    """Pack codes ``[N, K]`` (each < 2^bits) into uint32 words ``[N, K*bits/32]``.

    Each code is spread into its ``bits`` bits (least significant first), the
    bits of a row are laid end to end, and every 32 consecutive stream bits
    form one word (stream bit i -> bit i mod 32 of word i // 32).
    """
    codes = np.asarray(codes)
    N, K = codes.shape
    _check_bits(K, bits)
    if codes.size and (int(codes.max()) >= 2 ** bits or int(codes.min()) < 0):
        raise ValueError("code out of range")
    t = np.arange(bits, dtype=np.uint32)
    stream = (codes.astype(np.uint32)[:, :, None] >> t) & np.uint32(1)        # [N, K, bits]
    stream = stream.reshape(N, K * bits // 32, 32)
    place = np.uint32(1) << np.arange(32, dtype=np.uint32)
    return (stream * place).sum(axis=2, dtype=np.uint64).astype(np.uint32)


def affine_unpack(words, K, bits):
    """Unpack uint32 words ``[N, K*bits/32]`` into codes uint8 ``[N, K]``."""
    words = np.asarray(words, dtype=np.uint32)
    N = words.shape[0]
    _check_bits(K, bits)
    if words.shape[1] * 32 != K * bits:
        raise ValueError("packed width does not match K")
    stream = (words[:, :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)   # [N, W, 32]
    stream = stream.reshape(N, K, bits).astype(np.uint32)
    weight = np.uint32(1) << np.arange(bits, dtype=np.uint32)
    return (stream * weight).sum(axis=2).astype(np.uint8)


def affine_dequantize(codes, scales, biases, group_size):
    """w' = scale * q + bias per group, in fp64 ``[N, K]``.

    The stored scale has at most 24 significant bits and q at most 8, so the
    product is exact in fp64; the sum is exact too unless |bias| and scale
    differ by more than about 2^21 in magnitude.  Rounding the result to fp32
    therefore gives the single-rounding fp32 value fma(scale, q, bias).
    """
    codes = np.asarray(codes)
    N, K = codes.shape
    s = np.repeat(np.asarray(scales, dtype=np.float64), group_size, axis=1)
    b = np.repeat(np.asarray(biases, dtype=np.float64), group_size, axis=1)
    if s.shape != (N, K):
        raise ValueError("scales do not match codes and group_size")
    return s * codes.astype(np.float64) + b


def affine_forward(x, codes, scales, biases, group_size, bias=None):
    """y = x . w'^T (+ bias) with w' the dequantized weight, in fp64.

    ``x`` is ``[M, K]`` holding the stored input values; ``bias`` is ``[N]`` or
    None.  Returns ``(y_ref [M, N], D [M, N])`` where ``D = sum_k |x||w'|`` is
    the denominator of the tolerance rule.
    """
    x = np.asarray(x, dtype=np.float64)
    w = affine_dequantize(codes, scales, biases, group_size)
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    D = np.abs(x) @ np.abs(w).T
    return y, D
