"""Per-group symmetric int8 weights and the per-group int8 linear layer.

Test infrastructure only (see the package docstring).

Source: "cider/ops.py".
  * ``pergroup_linear``: x ``[M, K]`` fp16/bf16; int8 weights ``w [N, K]``
    quantized symmetrically per group of ``group_size`` (64, 128 or 256)
    consecutive input values; per-group scales ``[num_groups, N]`` fp32,
    stored transposed so that one group's scales for all outputs are
    contiguous; optional bias ``[N]``; output in x's dtype.  The function
    branches on M: for M > 1 it quantizes the activations and runs an int8
    product per group, for M == 1 it keeps the activations in floating point
    and dequantizes each weight as it is used.
  * ``quantize_weight_int8`` (absmax branch) fixes the symmetric rule a group
    follows: scale = absmax / 127 in fp32, a zero scale becomes 1, codes
    ``clip(round(w / scale), -128, 127)``.

Readings (the pages give the layout and the dispatch, not a per-group
quantizer):
  * a group is quantized exactly as ``quantize_weight_int8`` quantizes a row:
    fp32 absmax, fp32 quotient, round half to even;
  * M > 1: ``xq, sx`` = the per-row activation quantizer used by W8A8, and
    ``y[m, n] = sx[m] * sum_g s[g, n] * (sum_{k in g} xq[m, k] w[n, k])``
    (+ bias[n]);
  * M == 1: ``y[n] = sum_k x[k] * (w[n, k] * s[g(k), n])`` (+ bias[n]), with
    x as stored (no activation quantization).
"""

import numpy as np

from .int8 import exact_int_matmul, quantize_rows_int8


def quantize_groups_int8(w, group_size):
    """Per-group symmetric int8 quantization of fp32 weights ``w [N, K]``.

    Returns ``(q int8 [N, K], scale f32 [K / group_size, N])`` (scales stored
    group-major, the transposed layout of the pages).
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("expected a 2-D array")
    N, K = w.shape
    G = int(group_size)
    if G <= 0 or K % G:
        raise ValueError("K must be a multiple of group_size")
    if not np.isfinite(w).all():
        raise ValueError("non-finite weight")
    ng = K // G
    wg = w.reshape(N, ng, G)
    a = np.abs(wg).max(axis=2)                               # [N, ng] fp32
    s = (a / np.float32(127.0)).astype(np.float32)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    q = np.clip(np.rint(wg / s[:, :, None]), -128, 127).astype(np.int8)
    return q.reshape(N, K), np.ascontiguousarray(s.T)


def pergroup_forward(x, q, scale, group_size, bias=None):
    """Per-group int8 linear in the dequantized-operand reading.

    ``x`` ``[M, K]`` holds the stored input values, ``q`` int8 ``[N, K]``,
    ``scale`` fp32 ``[K / group_size, N]``.  Returns ``(y_ref fp64 [M, N],
    D fp64 [M, N])`` where D is ``sum_k |x_eff| |w_eff|`` over the operands
    the branch multiplies (quantized-and-rescaled x for M > 1, stored x for
    M == 1; dequantized weights in both).
    """
    x = np.asarray(x, dtype=np.float32)
    q = np.asarray(q, dtype=np.int8)
    M, K = x.shape
    N = q.shape[0]
    G = int(group_size)
    ng = K // G
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)  # [ng, N]
    qg = q.astype(np.int64).reshape(N, ng, G)
    if M == 1:
        wd = (qg.astype(np.float64) * s.T[:, :, None]).reshape(N, K)  # w * s, exact in fp64
        x64 = x.astype(np.float64)
        y = x64 @ wd.T
        D = np.abs(x64) @ np.abs(wd).T
    else:
        xq, sx = quantize_rows_int8(x)
        xg = xq.astype(np.int64).reshape(M, ng, G)
        y = np.zeros((M, N), dtype=np.float64)
        D = np.zeros((M, N), dtype=np.float64)
        for g in range(ng):                                    # one exact int8 sum per group
            acc = exact_int_matmul(xg[:, g, :], qg[:, g, :].T)  # [M, N]
            absacc = exact_int_matmul(np.abs(xg[:, g, :]), np.abs(qg[:, g, :]).T)
            y += acc.astype(np.float64) * s[g][None, :]
            D += absacc.astype(np.float64) * np.abs(s[g])[None, :]
        sx64 = sx.astype(np.float64)[:, None]
        y = y * sx64
        D = D * sx64
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y, D
