"""Helpers shared by the GPU parity tests: host copies and the comparison rule.

Expected values always come from the CPU oracle (``oracle/``) on the same
seeded inputs; nothing here computes any part of the layer.
"""

import numpy as np
import torch

import oracle

ODT = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


def f32(t):
    """Exact fp32 NumPy copy of a stored tensor (any float dtype, any device)."""
    return t.detach().to("cpu").to(torch.float32).numpy()


def u32(t):
    return t.detach().to("cpu").numpy().view(np.uint32)


def dev():
    return torch.device("cuda:0")


def assert_close(y_gpu, y_ref, D, K, out_dtype, strict=False, label=""):
    """Float parity: every element within 2e-2*D/sqrt(K) + 1e-3 (+ half an
    output ulp unless ``strict``)."""
    r = oracle.compare(f32(y_gpu).astype(np.float64), y_ref, D, K, ODT[out_dtype])
    print(f"[parity] {label} n={r['n']} strict_fail={r['strict_fail']} allowed_fail={r['allowed_fail']} "
          f"max_ratio={r['max_ratio_strict']:.3f}", flush=True)
    assert r["allowed_fail"] == 0, r
    if strict:
        assert r["strict_fail"] == 0, r
    return r
