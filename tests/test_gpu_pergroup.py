"""GPU parity for per-group int8 weights: the group quantizer is bit-exact
against the oracle; both branches of the per-group linear (M > 1 with
quantized activations, M == 1 with float activations) are within the
tolerance rule."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wdt", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("G,K", [(64, 1088), (128, 640), (256, 2304), (64, 4096)])
def test_quantize_groups_bitexact(wdt, G, K):
    rng = np.random.default_rng(G + K)
    N = 37
    w = (rng.standard_normal((N, K)) * rng.uniform(1e-3, 1e2, size=(N, 1))).astype(np.float32)
    w[5, G:2 * G] = 0                                   # a zero group takes scale 1
    w[6, 3] = 1e-30 if wdt == torch.float32 else 0.0    # tiny magnitudes
    wt = torch.from_numpy(w).to(wdt)
    q, s = qlq.qlq_quantize_groups_int8(wt.to(dev()), G)
    q_ref, s_ref = oracle.quantize_groups_int8(f32(wt), G)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _case(M, K, N, G, xdt, seed, bias=True):
    inp = workloads.w8a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=seed, outlier_frac=0.01)
    q, s = qlq.qlq_quantize_groups_int8(inp["w"].to(dev()), G)
    b = None if inp["bias"] is None else inp["bias"].to(dev())
    y = qlq.pergroup_linear_forward(inp["x"].to(dev()), q, s, G, bias=b)
    q_ref, s_ref = oracle.quantize_groups_int8(inp["w"].numpy(), G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    y_ref, D = oracle.pergroup_forward(f32(inp["x"]), q_ref, s_ref, G,
                                       bias=None if inp["bias"] is None else f32(inp["bias"]))
    return y, y_ref, D


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", [(2, 256, 45, 64), (37, 640, 130, 128), (130, 2304, 257, 256),
                                   (1, 256, 45, 64), (1, 1088, 130, 64), (1, 2304, 257, 256),
                                   # one, two and four 256-wide k-iterations with groups of
                                   # 128 and 256 (the GEMM's per-group sums alternate between
                                   # two register sets per k-iteration)
                                   (5, 128, 33, 128), (67, 512, 129, 128), (3, 1024, 70, 256),
                                   (9, 256, 64, 256)])
def test_forward_ragged(xdt, shape):
    M, K, N, G = shape
    y, y_ref, D = _case(M, K, N, G, xdt, seed=M * 7 + K + N)
    assert_close(y, y_ref, D, K, xdt, label=f"pergroup {xdt} {shape}")


def test_forward_float_branch_full_size():
    # the workload's single-token case: M == 1 keeps x in floating point
    name = "pergroup_int8_g128"
    cfg = workloads.WORKLOADS[name]
    K, N, G = cfg["K"], cfg["N"], cfg["group_size"]
    inp = workloads.workload_inputs(name, M=1)
    q, s = qlq.qlq_quantize_groups_int8(inp["w"].to(dev()), G)
    y = qlq.pergroup_linear_forward(inp["x"].to(dev()), q, s, G)
    q_ref, s_ref = oracle.quantize_groups_int8(inp["w"].numpy(), G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    y_ref, D = oracle.pergroup_forward(f32(inp["x"]), q_ref, s_ref, G)
    assert_close(y, y_ref, D, K, torch.float16, strict=True, label=f"{name} M=1")


def test_forward_quantized_branch_full():
    """The full workload through the quantized-activation branch: the GPU
    group quantizer is bit-exact on the workload weights, and every output
    is compared against the oracle run on the oracle's own codes and scales."""
    name = "pergroup_int8_g128"
    cfg = workloads.WORKLOADS[name]
    M, K, N, G = cfg["M"], cfg["K"], cfg["N"], cfg["group_size"]
    inp = workloads.workload_inputs(name)
    q, s = qlq.qlq_quantize_groups_int8(inp["w"].to(dev()), G)
    q_ref, s_ref = oracle.quantize_groups_int8(inp["w"].numpy(), G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    y = qlq.pergroup_linear_forward(inp["x"].to(dev()), q, s, G)
    y_ref, D = oracle.pergroup_forward(f32(inp["x"]), q_ref, s_ref, G)
    assert y.shape == (M, N)
    assert_close(y, y_ref, D, K, torch.float16, strict=True, label=f"{name} full")


def test_zero_input_gives_bias():
    K, N, G = 512, 40, 128
    w = torch.randn(N, K, device=dev())
    q, s = qlq.qlq_quantize_groups_int8(w, G)
    bias = (torch.arange(N, device=dev(), dtype=torch.float32) / 8).to(torch.float16)
    for M in (1, 5):
        y = qlq.pergroup_linear_forward(torch.zeros(M, K, device=dev(), dtype=torch.float16), q, s, G, bias=bias)
        assert torch.equal(y, bias.expand(M, N)), M
