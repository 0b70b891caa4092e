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
  * codes are packed LSB-first into little-endian uint32 words along K: code k
    sits at bit ``bits*(k mod (32/bits))`` of word ``k // (32/bits)``;
  * only widths that divide 32 (1, 2, 4, 8) are packed here.
"""

import numpy as np

from .codecs import round_to_dtype


def _check_shape(K, bits, group_size):
    if bits not in (1, 2, 4, 8):
        raise ValueError(f"bits={bits} does not divide 32")
    if group_size <= 0 or K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    if K % (32 // bits):
        raise ValueError(f"K={K} does not fill whole uint32 words at {bits} bits")


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
    """Pack codes ``[N, K]`` (each < 2^bits) into uint32 words ``[N, K*bits/32]``."""
    codes = np.asarray(codes)
    N, K = codes.shape
    per = 32 // bits
    if 32 % bits or K % per:
        raise ValueError("bits must divide 32 and K must fill whole words")
    if codes.size and int(codes.max()) >= 2 ** bits:
        raise ValueError("code out of range")
    c = codes.astype(np.uint32).reshape(N, K // per, per)
    words = np.zeros((N, K // per), dtype=np.uint32)
    for slot in range(per):
        words |= c[:, :, slot] << np.uint32(bits * slot)
    return words


def affine_unpack(words, K, bits):
    """Unpack uint32 words ``[N, K*bits/32]`` into codes uint8 ``[N, K]``."""
    words = np.asarray(words, dtype=np.uint32)
    N = words.shape[0]
    per = 32 // bits
    if words.shape[1] * per != K:
        raise ValueError("packed width does not match K")
    mask = np.uint32(2 ** bits - 1)
    codes = np.empty((N, K // per, per), dtype=np.uint8)
    for slot in range(per):
        codes[:, :, slot] = (words >> np.uint32(bits * slot)) & mask
    return codes.reshape(N, K)


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
