"""Seeded synthetic inputs for the quantized linear layer.

This module only draws random inputs and casts them to their storage dtype; it
holds none of the layer's arithmetic (no quantizer, no packing, no product).
Both the GPU tests and the CPU oracle take their inputs from here.

Recipe (one NumPy PCG64 generator per case, ``default_rng(seed)``, draws in a
fixed order: x, then W or ternary codes, then the layer bias, then outlier
positions; every draw is fp32 and is cast to the storage dtype by torch's CPU
round-to-nearest-even conversion):

  tiny_affine_4bit    x f32 [4,256] ~N(0,1); W f32 [128,256] ~N(0,0.02);
                      group 64, 4-bit, f32 scales/biases; bias f32 ~N(0,0.01)
  decode_gemv_4bit    x bf16 [1,4096] ~N(0,1); W [4096,4096] ~N(0,0.02);
                      group 64, 4-bit, bf16 scales/biases; no bias
  ternary_bitlinear   x bf16 [8,2560] ~N(0,1); codes uniform {0,1,2} -> t =
                      code-1, W [6912,2560]; weight_scale bf16(0.05), multiply
  prefill_gemm_4bit   x bf16 [2048,4096] ~N(0,1); W [11008,4096] ~N(0,0.02);
                      group 128, 4-bit, bf16 scales/biases; bias bf16 ~N(0,0.01)
  w8a8_perchannel     x f16 [1024,4096] ~N(0,1), exactly round(0.001*M*K)
                      distinct positions multiplied by 20 before the cast;
                      W f32 [4096,4096] ~N(0,0.02); no bias
  pergroup_int8_g128  the w8a8_perchannel recipe (x f16 [1024,4096] with the
                      same outliers, W f32 [4096,4096] ~N(0,0.02), no bias);
                      weights quantized per group of 128; its single-token
                      case draws x [1,4096] by the same recipe
  w4a8_perchannel     x f16 [1024,4096] by the w8a8_perchannel recipe (same
                      outlier count and factor); W f32 [K=4096, N=4096]
                      ~N(0,0.02) drawn in the [K, N] orientation the int4
                      packer takes; no bias
  decode_gemv_3bit    the decode_gemv_4bit recipe with 3-bit codes (a code
                      stream whose codes straddle words)
  prefill_gemm_3bit   the prefill_gemm_4bit recipe with 3-bit codes

The default seed of a workload is 1000 + its index in the list above (1..9).
Smaller parity cases reuse the same recipes at other shapes and seeds.
"""

import numpy as np
import torch

WORKLOADS = {
    "tiny_affine_4bit": dict(index=1, kind="affine", M=4, K=256, N=128, bits=4,
                             group_size=64, x_dtype="f32", sb_dtype="f32",
                             bias=True),
    "decode_gemv_4bit": dict(index=2, kind="affine", M=1, K=4096, N=4096, bits=4,
                             group_size=64, x_dtype="bf16", sb_dtype="bf16",
                             bias=False),
    "ternary_bitlinear": dict(index=3, kind="ternary", M=8, K=2560, N=6912,
                              x_dtype="bf16", weight_scale=0.05, invert=False,
                              bias=False),
    "prefill_gemm_4bit": dict(index=4, kind="affine", M=2048, K=4096, N=11008,
                              bits=4, group_size=128, x_dtype="bf16",
                              sb_dtype="bf16", bias=True),
    "w8a8_perchannel": dict(index=5, kind="w8a8", M=1024, K=4096, N=4096,
                            x_dtype="f16", bias=False, outlier_frac=0.001,
                            outlier_mult=20.0),
    "pergroup_int8_g128": dict(index=6, kind="w8a8", M=1024, K=4096, N=4096,
                               group_size=128, x_dtype="f16", bias=False,
                               outlier_frac=0.001, outlier_mult=20.0),
    "w4a8_perchannel": dict(index=7, kind="w4a8", M=1024, K=4096, N=4096,
                            x_dtype="f16", bias=False, outlier_frac=0.001,
                            outlier_mult=20.0),
    "decode_gemv_3bit": dict(index=8, kind="affine", M=1, K=4096, N=4096, bits=3,
                             group_size=64, x_dtype="bf16", sb_dtype="bf16",
                             bias=False),
    "prefill_gemm_3bit": dict(index=9, kind="affine", M=2048, K=4096, N=11008,
                              bits=3, group_size=128, x_dtype="bf16",
                              sb_dtype="bf16", bias=True),
}

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def default_seed(name):
    return 1000 + WORKLOADS[name]["index"]


def _cast(a32, dtype):
    """fp32 NumPy array -> torch CPU tensor of the storage dtype (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(TORCH_DTYPE[dtype])


def affine_inputs(M, K, N, x_dtype="bf16", bias=False, bias_dtype=None, seed=0,
                  w_std=0.02, bias_std=0.01):
    """x [M,K] (x_dtype), W [N,K] fp32, optional bias [N] (x_dtype)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    b = None
    if bias:
        b = (rng.standard_normal(N, dtype=np.float32) * np.float32(bias_std)).astype(np.float32)
    return {
        "x": _cast(x, x_dtype),
        "w": torch.from_numpy(w),
        "bias": None if b is None else _cast(b, bias_dtype or x_dtype),
    }


def ternary_inputs(M, K, N, x_dtype="bf16", weight_scale=0.05, bias=False, seed=0,
                   bias_std=0.01):
    """x [M,K], ternary t [N,K] int8 in {-1,0,1}, weight_scale [1], bias [N]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    codes = rng.integers(0, 3, size=(N, K), dtype=np.int8)
    b = None
    if bias:
        b = (rng.standard_normal(N, dtype=np.float32) * np.float32(bias_std)).astype(np.float32)
    return {
        "x": _cast(x, x_dtype),
        "t": torch.from_numpy((codes - 1).astype(np.int8)),
        "weight_scale": _cast(np.array([weight_scale], dtype=np.float32), x_dtype),
        "bias": None if b is None else _cast(b, x_dtype),
    }


def w8a8_inputs(M, K, N, x_dtype="f16", bias=False, seed=0, outlier_frac=0.001,
                outlier_mult=20.0, w_std=0.02, bias_std=0.01):
    """x [M,K] with outliers, W [N,K] fp32, optional bias [N]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    b = None
    if bias:
        b = (rng.standard_normal(N, dtype=np.float32) * np.float32(bias_std)).astype(np.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        pos = rng.choice(M * K, n_out, replace=False)
        flat = x.reshape(-1)
        flat[pos] = flat[pos] * np.float32(outlier_mult)
    return {
        "x": _cast(x, x_dtype),
        "w": torch.from_numpy(w),
        "bias": None if b is None else _cast(b, x_dtype),
    }


def w4a8_inputs(M, K, N, x_dtype="f16", bias=False, seed=0, outlier_frac=0.001,
                outlier_mult=20.0, w_std=0.02, bias_std=0.01):
    """x [M,K] with outliers, W [K,N] fp32 (the int4 packer's orientation),
    optional bias [N]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    w = (rng.standard_normal((K, N), dtype=np.float32) * np.float32(w_std)).astype(np.float32)
    b = None
    if bias:
        b = (rng.standard_normal(N, dtype=np.float32) * np.float32(bias_std)).astype(np.float32)
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        pos = rng.choice(M * K, n_out, replace=False)
        flat = x.reshape(-1)
        flat[pos] = flat[pos] * np.float32(outlier_mult)
    return {
        "x": _cast(x, x_dtype),
        "w": torch.from_numpy(w),
        "bias": None if b is None else _cast(b, x_dtype),
    }


def workload_inputs(name, seed=None, **shape):
    """Inputs of a named workload; ``shape`` may override M, K, N."""
    cfg = dict(WORKLOADS[name])
    cfg.update(shape)
    seed = default_seed(name) if seed is None else seed
    if cfg["kind"] == "affine":
        return affine_inputs(cfg["M"], cfg["K"], cfg["N"], x_dtype=cfg["x_dtype"],
                             bias=cfg["bias"], seed=seed)
    if cfg["kind"] == "ternary":
        return ternary_inputs(cfg["M"], cfg["K"], cfg["N"], x_dtype=cfg["x_dtype"],
                              weight_scale=cfg["weight_scale"], bias=cfg["bias"], seed=seed)
    if cfg["kind"] == "w8a8":
        return w8a8_inputs(cfg["M"], cfg["K"], cfg["N"], x_dtype=cfg["x_dtype"],
                           bias=cfg["bias"], seed=seed, outlier_frac=cfg["outlier_frac"],
                           outlier_mult=cfg["outlier_mult"])
    if cfg["kind"] == "w4a8":
        return w4a8_inputs(cfg["M"], cfg["K"], cfg["N"], x_dtype=cfg["x_dtype"],
                           bias=cfg["bias"], seed=seed, outlier_frac=cfg["outlier_frac"],
                           outlier_mult=cfg["outlier_mult"])
    raise ValueError(cfg["kind"])


def to_f32_numpy(t):
    """Exact widening of a stored torch tensor to an fp32 NumPy array."""
    return t.detach().to("cpu").to(torch.float32).numpy()
