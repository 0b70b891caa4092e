"""Comparison rule for floating-point outputs (test infrastructure only).

The bound for a float output is ``|y - y_ref| <= 2e-2 * D / sqrt(K) + 1e-3``
with ``D = sum_k |x||w|`` over the operands the method multiplies.

Reading: the bound is taken to hold for the value *before* its final rounding
to the output dtype, so the pass rule adds half an ulp of the output dtype at
``y_ref``.  Both counts are reported: ``strict`` (without the allowance) and
``allowed`` (with it).  The allowance matters only where half an output ulp
exceeds the bound, e.g. bf16 outputs with |y| >= 8 and a small D.
"""

import numpy as np

from .codecs import half_ulp

REL = 2e-2
ABS = 1e-3


def tolerance(D, K):
    """2e-2 * D / sqrt(K) + 1e-3 (fp64)."""
    D = np.asarray(D, dtype=np.float64)
    return REL * D / np.sqrt(max(int(K), 1)) + ABS


def compare(y, y_ref, D, K, out_dtype):
    """Element-wise comparison of a float output against the oracle.

    Returns a dict with the number of elements outside the strict bound, the
    number outside the bound plus half an output ulp, and the largest ratio of
    error to the allowed bound.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.shape != y_ref.shape:
        raise ValueError(f"shape {y.shape} != {y_ref.shape}")
    err = np.abs(y - y_ref)
    tol = tolerance(D, K)
    allow = tol + half_ulp(y_ref, out_dtype)
    bad_strict = ~(err <= tol)          # NaN counts as a failure
    bad_allow = ~(err <= allow)
    return {
        "n": int(y.size),
        "strict_fail": int(bad_strict.sum()),
        "allowed_fail": int(bad_allow.sum()),
        "max_ratio_strict": float(np.max(err / tol)) if y.size else 0.0,
        "max_ratio_allowed": float(np.max(err / allow)) if y.size else 0.0,
    }
