"""Per-row symmetric int8 quantization, int8 x int8 -> int32 matmul, W8A8.

Test infrastructure only (see the package docstring).

Source: "cider/ops.py".
  * ``quantize_weight_int8`` (absmax branch): cast to fp32,
    ``scale = rowmax|w| / 127``, a zero scale becomes 1.0,
    ``q = clip(round(w / scale), -128, 127)`` as int8, scale fp32 ``[N]``.
  * ``perchannel_linear``: ``y = dequant(quant_a(x) @ w_int8) + bias`` with x
    ``[M, K]`` fp16/bf16, w int8 ``[N, K]``, ``scale_w`` fp32 ``[N]``, output in
    the input dtype.
  * ``int8_matmul_int32``: int8 ``a [M, K]`` times int8 ``b [N, K]`` (the
    transposed weight layout) to int32 ``[M, N]``, bit-exact.

  * ``quantize_weight_int8`` with ``clip_percentile`` set: the row's scale
    comes from the given percentile of |w| instead of its maximum (a zero
    percentile falls back to the maximum), the row is clipped to
    [-clip, clip], then quantized with scale = clip / 127 as above.

Reading of the percentile: NumPy's default ("linear") percentile on the
fp32 array of |w| under NumPy 2 promotion rules, so every step stays in fp32:
the fraction q = fl32(p / 100), the virtual index v = fl32((K - 1) q), its
floor i and weight t = v - i, and with the sorted values a <= b at i and
i + 1: a + (b - a) t when t < 0.5, else b - (b - a)(1 - t), each operation
rounded to fp32; v >= K - 1 gives the largest value.  (Under NumPy 1 value
casting the same call computes in fp64.)

Reading: the pages name the activation quantizer ``quant_a`` without defining
it; it is taken to be the same per-row symmetric absmax/127 rule as the weight
quantizer, applied to each row of x.  The W8A8 reference output is the product
of the dequantized operands, ``acc * sx[m] * sw[n] (+ bias)``, not x W^T on the
unquantized values.
"""

import numpy as np


def quantize_rows_int8(v):
    """Per-row symmetric int8 quantization of ``[R, K]`` values (fp32 steps).

    Returns ``(q int8 [R, K], scale f32 [R])``.
    """
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("expected a 2-D array")
    if not np.isfinite(v).all():
        raise ValueError("non-finite value")
    a = np.abs(v).max(axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    s = (a / np.float32(127.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = np.clip(np.rint(v / s[:, None]), -128, 127).astype(np.int8)
    return q, s


def row_percentile(v, percentile):
    """fp32 percentile of each row of ``v`` (see the module reading)."""
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    srt = np.sort(v, axis=1)
    q = np.float32(np.float32(percentile) / np.float32(100.0))
    vi = np.float32(np.float32(K - 1) * q)
    if vi >= K - 1:
        return srt[:, K - 1].copy()
    i = int(np.floor(vi))
    t = np.float32(vi - np.float32(i))
    a, b = srt[:, i], srt[:, i + 1]
    d = (b - a).astype(np.float32)
    if t >= 0.5:
        return (b - (d * np.float32(np.float32(1.0) - t)).astype(np.float32)).astype(np.float32)
    return (a + (d * t).astype(np.float32)).astype(np.float32)


def quantize_rows_int8_clip(w, clip_percentile):
    """Per-row symmetric int8 with a percentile clip (fp32 steps).

    Returns ``(q int8 [R, K], scale f32 [R])``.
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] == 0:
        raise ValueError("expected a non-empty 2-D array")
    if not np.isfinite(w).all():
        raise ValueError("non-finite value")
    if not 0.0 <= clip_percentile <= 100.0:
        raise ValueError("percentile outside [0, 100]")
    aw = np.abs(w)
    clip = row_percentile(aw, clip_percentile)
    clip = np.where(clip == 0, aw.max(axis=1), clip).astype(np.float32)
    s = (clip / np.float32(127.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    wc = np.clip(w, -clip[:, None], clip[:, None])
    q = np.clip(np.rint(wc / s[:, None]), -128, 127).astype(np.int8)
    return q, s


def exact_int_matmul(a, b):
    """Exact integer product ``a [M, K] @ b [K, N]`` returned as int64.

    When ``max|a| * max|b| * K < 2^53`` every partial sum, in whatever order a
    library adds the terms, is an integer of magnitude below 2^53, which fp64
    holds exactly; the product is then taken as an fp64 matrix product.  Any
    larger bound takes the int64 product.
    """
    a = np.asarray(a)
    b = np.asarray(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("shapes do not chain")
    K = a.shape[1]
    amax = int(np.abs(a.astype(np.int64)).max()) if a.size else 0
    bmax = int(np.abs(b.astype(np.int64)).max()) if b.size else 0
    if amax * bmax * max(K, 1) < 2 ** 53:
        return (a.astype(np.float64) @ b.astype(np.float64)).astype(np.int64)
    return a.astype(np.int64) @ b.astype(np.int64)


def int8_matmul_int32(a, b):
    """Exact ``a [M, K] @ b [N, K]^T`` as int64 (equals int32 when it fits)."""
    a = np.asarray(a, dtype=np.int8)
    b = np.asarray(b, dtype=np.int8)
    return exact_int_matmul(a, b.T)


def w8a8_forward(x, wq, sw, bias=None):
    """W8A8 per-channel linear in the dequantized-operand reading.

    ``x`` ``[M, K]`` holds the stored fp16/bf16 input values, ``wq`` int8
    ``[N, K]``, ``sw`` fp32 ``[N]``.  Returns
    ``(xq int8 [M, K], sx f32 [M], acc int64 [M, N], y_ref fp64 [M, N], D)``
    with ``y_ref = acc * sx[m] * sw[n] (+ bias[n])`` and
    ``D = sum_k |xq sx| |wq sw|``.
    """
    xq, sx = quantize_rows_int8(x)
    acc = int8_matmul_int32(xq, wq)
    sx64 = sx.astype(np.float64)[:, None]
    sw64 = np.asarray(sw, dtype=np.float32).astype(np.float64)[None, :]
    y = acc.astype(np.float64) * sx64 * sw64
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    absacc = exact_int_matmul(np.abs(xq.astype(np.int64)), np.abs(np.asarray(wq, dtype=np.int64)).T)
    D = absacc.astype(np.float64) * sx64 * np.abs(sw64)
    return xq, sx, acc, y, D
