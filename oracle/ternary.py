"""Ternary BitLinear: pack, decode and forward.

Test infrastructure only (see the package docstring).

Source: "mlx-lm/mlx_lm/models/bitlinear_layers.py".
  * ``BitLinear.__init__``: the weight is uint8 ``[(out+3)//4, in]``, four
    2-bit values per byte; ``weight_scale`` has one element; ``bias`` ``[out]``.
  * ``make_bitlinear_kernel`` (the Metal source): byte ``(r, k)`` holds in bit
    field j (bits 2j..2j+1) the code of output row ``r + j*out/4`` at input k;
    a code c decodes to ``c - 1``; the per-row sum is multiplied by
    ``weight_scale`` or, with ``invert_weight_scales``, by its reciprocal.
  * ``execute_matmul_kernel`` / ``__call__``: the input dtype must equal the
    weight-scale dtype, the output has that dtype, and the layer bias is added
    after the scaled product.

Readings: ``out % 4 == 0`` is required (the page sizes the packed rows as
``(out+3)//4`` but indexes them with ``out/4``); code 3 decodes literally to
+2, as the kernel arithmetic does (the packer never emits it); the scale is the
*stored* weight_scale value (e.g. bf16(0.05) = 0.050048828125).
"""

import numpy as np


def ternary_pack(t):
    """Pack ternary values ``[N, K]`` in {-1, 0, 1} into uint8 ``[N/4, K]``.

    byte[r, k] = sum_j (t[r + j*N/4, k] + 1) << 2j
    """
    t = np.asarray(t)
    N, K = t.shape
    if N % 4:
        raise ValueError("N must be a multiple of 4")
    if t.size and (t.min() < -1 or t.max() > 1):
        raise ValueError("ternary value outside {-1, 0, 1}")
    R = N // 4
    codes = (t.astype(np.int16) + 1).astype(np.uint8)
    out = np.zeros((R, K), dtype=np.uint8)
    for j in range(4):
        out |= codes[j * R:(j + 1) * R, :] << np.uint8(2 * j)
    return out


def ternary_unpack(packed, N):
    """Decode packed bytes ``[N/4, K]`` to int8 values ``[N, K]`` (code - 1)."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, K = packed.shape
    if N != 4 * R:
        raise ValueError("N must equal 4 * packed rows")
    t = np.empty((N, K), dtype=np.int8)
    for j in range(4):
        c = (packed >> np.uint8(2 * j)) & np.uint8(3)
        t[j * R:(j + 1) * R, :] = c.astype(np.int8) - 1
    return t


def ternary_forward(x, packed, N, weight_scale, invert=False, bias=None):
    """y[m, n] = sigma * sum_k x[m, k] * t[n, k] (+ bias[n]) in fp64.

    ``sigma`` is the stored ``weight_scale`` value, or its reciprocal when
    ``invert`` is set.  Returns ``(y_ref [M, N], D [M, N])`` with
    ``D = sum_k |x||sigma t|``.
    """
    x = np.asarray(x, dtype=np.float64)
    t = ternary_unpack(packed, N).astype(np.float64)
    ws = float(np.float64(weight_scale))
    sigma = 1.0 / ws if invert else ws
    y = sigma * (x @ t.T)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    D = abs(sigma) * (np.abs(x) @ np.abs(t).T)
    return y, D
