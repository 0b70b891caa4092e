"""Randomized GPU parity: seeded random shapes, dtypes and options for every
forward entry point, each checked against the oracle by the tolerance rule
(and bit-exact where the operation is integer or byte work).  Shapes stay
within each entry point's documented limits and small enough for the oracle;
the seed of every case is in its id, so a failure names its case."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32

pytestmark = pytest.mark.gpu

SEEDS = list(range(48))
XDT = [torch.bfloat16, torch.float16]


def _rng(kind, seed):
    return np.random.default_rng(10_000 * kind + seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_affine_random(seed):
    rng = _rng(1, seed)
    bits = int(rng.choice([1, 2, 3, 4, 5, 6, 8]))
    G = int(rng.choice([32, 64, 128]))
    K = G * int(rng.integers(1, 9))
    if rng.random() < 0.7:
        K = ((K + 63) // 64) * 64 if K % 64 else K          # most cases can take the GEMM
        K = max(K, G)
        K -= K % G
    M = int(rng.integers(1, 160))
    N = int(rng.integers(1, 200))
    xdt = [torch.bfloat16, torch.float16, torch.float32][int(rng.integers(0, 3))]
    bias = bool(rng.random() < 0.5)
    inp = workloads.affine_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=seed)
    packed, scales, biases = qlq.qlq_pack(inp["w"].to(dev()), bits, G, xdt)
    codes, s_ref, b_ref = oracle.affine_quantize(inp["w"].numpy(), bits, G, ODT[xdt])
    assert np.array_equal(packed.cpu().numpy().view(np.uint32), oracle.affine_pack(codes, bits))
    y_ref, D = oracle.affine_forward(f32(inp["x"]), codes, s_ref, b_ref, G,
                                     bias=None if inp["bias"] is None else f32(inp["bias"]))
    old = qlq.qlq_get_skinny_max_m()
    try:
        for thr in (1 << 20, 0):                               # skinny, then the GEMM where it applies
            qlq.qlq_set_skinny_max_m(thr)
            y = qlq.qlq_linear_forward(inp["x"].to(dev()), packed, scales, biases, bits, G,
                                       bias=None if inp["bias"] is None else inp["bias"].to(dev()))
            assert_close(y, y_ref, D, K, xdt, label=f"affine seed={seed} bits={bits} G={G} "
                                                     f"M={M} K={K} N={N} {xdt} thr={thr}")
    finally:
        qlq.qlq_set_skinny_max_m(old)


@pytest.mark.parametrize("seed", SEEDS)
def test_ternary_random(seed):
    rng = _rng(2, seed)
    M = int(rng.integers(1, 40))
    K = 32 * int(rng.integers(1, 40))
    N = 4 * int(rng.integers(1, 120))
    xdt = [torch.bfloat16, torch.float16, torch.float32][int(rng.integers(0, 3))]
    invert = bool(rng.random() < 0.5)
    inp = workloads.ternary_inputs(M, K, N, x_dtype=ODT[xdt], weight_scale=float(rng.uniform(0.01, 2)),
                                   bias=bool(rng.random() < 0.5), seed=seed)
    packed = qlq.bitlinear_pack(inp["t"].to(dev()))
    ref_packed = oracle.ternary_pack(inp["t"].numpy())
    assert np.array_equal(packed.cpu().numpy(), ref_packed)
    y = qlq.bitlinear_forward(inp["x"].to(dev()), packed, N, inp["weight_scale"].to(dev()), invert,
                              bias=None if inp["bias"] is None else inp["bias"].to(dev()))
    y_ref, D = oracle.ternary_forward(f32(inp["x"]), ref_packed, N, float(f32(inp["weight_scale"])[0]), invert,
                                      bias=None if inp["bias"] is None else f32(inp["bias"]))
    assert_close(y, y_ref, D, K, xdt, label=f"ternary seed={seed} M={M} K={K} N={N} {xdt} invert={invert}")


@pytest.mark.parametrize("seed", SEEDS)
def test_int8_families_random(seed):
    """Per-channel W8A8, per-group int8 and W4A8 on one random shape each."""
    rng = _rng(3, seed)
    M = int(rng.choice([1, 2, 5, 8, 9, 33, 130, 200]))
    xdt = XDT[int(rng.integers(0, 2))]
    bias = bool(rng.random() < 0.5)
    # per-channel W8A8
    K = 16 * int(rng.integers(1, 80))
    N = int(rng.integers(1, 260))
    inp = workloads.w8a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=seed)
    wq, sw = qlq.qlq_quantize_rows_int8(inp["w"].to(dev()))
    wq_ref, sw_ref = oracle.quantize_rows_int8(inp["w"].numpy())
    assert np.array_equal(wq.cpu().numpy(), wq_ref) and np.array_equal(sw.cpu().numpy(), sw_ref)
    y = qlq.w8a8_linear_forward(inp["x"].to(dev()), wq, sw, bias=None if not bias else inp["bias"].to(dev()))
    *_, y_ref, D = oracle.w8a8_forward(f32(inp["x"]), wq_ref, sw_ref, bias=None if not bias else f32(inp["bias"]))
    assert_close(y, y_ref, D, K, xdt, label=f"w8a8 seed={seed} M={M} K={K} N={N}")
    # per-group int8
    G = int(rng.choice([64, 128, 256]))
    K = G * int(rng.integers(1, 12))
    inp = workloads.w8a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=seed + 1)
    q, sg = qlq.qlq_quantize_groups_int8(inp["w"].to(dev()), G)
    q_ref, sg_ref = oracle.quantize_groups_int8(inp["w"].numpy(), G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    y = qlq.pergroup_linear_forward(inp["x"].to(dev()), q, sg, G, bias=None if not bias else inp["bias"].to(dev()))
    y_ref, D = oracle.pergroup_forward(f32(inp["x"]), q_ref, sg_ref, G, bias=None if not bias else f32(inp["bias"]))
    assert_close(y, y_ref, D, K, xdt, label=f"pergroup seed={seed} M={M} K={K} N={N} G={G}")
    # W4A8 (both paths for M <= 8)
    K = 16 * int(rng.integers(1, 80))
    inp = workloads.w4a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=seed + 2)
    p4, s4 = qlq.w4a8_pack_weight_int4(inp["w"].to(dev()))
    p_ref, s4_ref = oracle.pack_weight_int4(inp["w"].numpy())
    assert np.array_equal(p4.cpu().numpy(), p_ref)
    *_, y_ref, D = oracle.w4a8_forward(f32(inp["x"]), p_ref, s4_ref, bias=None if not bias else f32(inp["bias"]))
    old = qlq.qlq_get_skinny_max_m()
    try:
        outs = []
        for thr in (8, 0):
            qlq.qlq_set_skinny_max_m(thr)
            y = qlq.w4a8_linear_forward(inp["x"].to(dev()), p4, s4, bias=None if not bias else inp["bias"].to(dev()))
            assert_close(y, y_ref, D, K, xdt, label=f"w4a8 seed={seed} M={M} K={K} N={N} thr={thr}")
            outs.append(y)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    finally:
        qlq.qlq_set_skinny_max_m(old)
