"""Per-column symmetric int4 weights and the W4A8 linear layer.

Test infrastructure only (see the package docstring).

Source: "cider/ops.py".
  * ``pack_weight_int4``: weights ``w [K, N]`` (K even, cast to fp32),
    per-column scale = colmax|w| / 7 in fp32, a zero scale becomes 1,
    codes ``clip(round(w / scale) + zero_point, 0, 15)`` with zero point 8;
    two codes per byte, ``packed [K // 2, N]`` uint8 with the even k in the
    high nibble and the odd k in the low nibble; ``scale_w [N]`` fp32.
  * ``w4a8_linear``: ``y = dequant(quant_a(x) @ unpack4(w))`` with x
    ``[M, K]`` fp16 (output in x's dtype) and per-column ``scale_w``.

Readings:
  * ``unpack4`` recovers the signed value ``code - zero_point`` of each
    nibble, so the weight multiplied is ``(code - 8) * scale_w[n]``;
  * ``quant_a`` is the per-row symmetric absmax/127 int8 quantizer used by
    W8A8 (the pages name it without defining it), and the reference output is
    the product of the dequantized operands,
    ``y[m, n] = sx[m] * scale_w[n] * sum_k xq[m, k] (code[k, n] - 8)``
    (+ bias[n]); the pages' function takes no bias, an optional one is added
    after the product.
"""

import numpy as np

from .int8 import exact_int_matmul, quantize_rows_int8

ZERO_POINT = 8


def pack_weight_int4(w, zero_point=ZERO_POINT):
    """Per-column symmetric int4 quantization and packing of ``w [K, N]``.

    Returns ``(packed uint8 [K // 2, N], scale f32 [N])``.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("expected a 2-D array")
    K, N = w.shape
    if K % 2:
        raise ValueError("K must be even")
    if not np.isfinite(w).all():
        raise ValueError("non-finite weight")
    a = np.abs(w).max(axis=0) if K else np.zeros(N, np.float32)   # [N] fp32
    s = (a / np.float32(7.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    r = np.rint(w / s[None, :]).astype(np.float32)                 # fp32 quotient, half to even
    codes = np.clip(r + np.float32(zero_point), 0, 15).astype(np.uint8)
    packed = ((codes[0::2, :] << 4) | codes[1::2, :]).astype(np.uint8)
    return packed, s


def unpack_weight_int4(packed):
    """Codes ``[K, N]`` (0..15) of ``packed [K // 2, N]``: row 2j is the high
    nibble of packed row j, row 2j + 1 the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    K2, N = p.shape
    codes = np.empty((2 * K2, N), dtype=np.uint8)
    codes[0::2, :] = p >> 4
    codes[1::2, :] = p & 0x0F
    return codes


def w4a8_forward(x, packed, scale_w, bias=None, zero_point=ZERO_POINT):
    """W4A8 linear in the dequantized-operand reading.

    ``x`` ``[M, K]`` holds the stored fp16/bf16 input values, ``packed``
    uint8 ``[K // 2, N]``, ``scale_w`` fp32 ``[N]``.  Returns
    ``(xq int8 [M, K], sx f32 [M], acc int64 [M, N], y_ref fp64 [M, N], D)``
    with ``acc = xq @ (codes - zero_point)``,
    ``y_ref = acc * sx[m] * scale_w[n] (+ bias[n])`` and
    ``D = sum_k |xq sx| |(code - zero_point) scale_w|``.
    """
    xq, sx = quantize_rows_int8(x)
    wv = unpack_weight_int4(packed).astype(np.int64) - zero_point     # [K, N]
    xi = xq.astype(np.int64)
    acc = exact_int_matmul(xi, wv)
    sx64 = sx.astype(np.float64)[:, None]
    sw64 = np.asarray(scale_w, dtype=np.float32).astype(np.float64)[None, :]
    y = acc.astype(np.float64) * sx64 * sw64
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    D = exact_int_matmul(np.abs(xi), np.abs(wv)).astype(np.float64) * sx64 * np.abs(sw64)
    return xq, sx, acc, y, D
