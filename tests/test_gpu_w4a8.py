"""GPU parity for per-column int4 weights with int8 activations: the packer is
bit-exact against the oracle; w4a8_linear_forward's int32 sums are exact, so
its outputs are within the tolerance rule on the full workload and on ragged
shapes (K tails, N not a multiple of 128 or of 4, M not a multiple of 128)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wdt", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("K,N", [(64, 37), (1088, 130), (4096, 256)])
def test_pack_bitexact(wdt, K, N):
    rng = np.random.default_rng(K + N)
    w = (rng.standard_normal((K, N)) * rng.uniform(1e-3, 1e2, size=(1, N))).astype(np.float32)
    w[:, 5] = 0                                          # a zero column takes scale 1
    w[3, 6] = 1e-30 if wdt == torch.float32 else 0.0
    wt = torch.from_numpy(w).to(wdt)
    packed, s = qlq.w4a8_pack_weight_int4(wt.to(dev()))
    p_ref, s_ref = oracle.pack_weight_int4(f32(wt))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(packed.cpu().numpy(), p_ref)


def test_pack_ties_and_extremes():
    # quotients exactly on .5 (round half to even) and at +-7
    col = np.array([7.0, -7.0, 2.5, -2.5, 0.5, -0.5, 3.5, -1.5], dtype=np.float32)
    w = np.stack([col, col * 2, np.zeros_like(col), col * 0.25], axis=1)
    packed, s = qlq.w4a8_pack_weight_int4(torch.from_numpy(w).to(dev()))
    p_ref, s_ref = oracle.pack_weight_int4(w)
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)


def _case(M, K, N, xdt, seed, bias=True):
    inp = workloads.w4a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=seed, outlier_frac=0.01)
    packed, s = qlq.w4a8_pack_weight_int4(inp["w"].to(dev()))
    b = None if inp["bias"] is None else inp["bias"].to(dev())
    y = qlq.w4a8_linear_forward(inp["x"].to(dev()), packed, s, bias=b)
    p_ref, s_ref = oracle.pack_weight_int4(inp["w"].numpy())
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    _, _, _, y_ref, D = oracle.w4a8_forward(f32(inp["x"]), p_ref, s_ref,
                                            bias=None if inp["bias"] is None else f32(inp["bias"]))
    return y, y_ref, D


SHAPES = [  # (M, K, N): tiles of 128 x 128 x 256; N % 4 != 0 takes byte loads
    (1, 256, 128), (3, 272, 132), (130, 512, 260), (129, 4096, 130), (300, 1040, 517),
    (17, 16, 4), (64, 784, 1), (257, 2048, 384),
]


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", SHAPES)
def test_forward_ragged(xdt, shape):
    M, K, N = shape
    y, y_ref, D = _case(M, K, N, xdt, seed=M * 7 + K + N, bias=(M % 2 == 1))
    assert_close(y, y_ref, D, K, xdt, label=f"w4a8 {xdt} {shape}")


@pytest.mark.parametrize("M", [1024, 1])
def test_forward_workload_full(M):
    """The full workload (and its single-token case): the packer is bit-exact
    on the workload weights and every output is compared against the oracle
    run on the oracle's own packed weights and scales."""
    name = "w4a8_perchannel"
    cfg = workloads.WORKLOADS[name]
    K, N = cfg["K"], cfg["N"]
    inp = workloads.workload_inputs(name, M=M)
    packed, s = qlq.w4a8_pack_weight_int4(inp["w"].to(dev()))
    p_ref, s_ref = oracle.pack_weight_int4(inp["w"].numpy())
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    y = qlq.w4a8_linear_forward(inp["x"].to(dev()), packed, s)
    _, _, _, y_ref, D = oracle.w4a8_forward(f32(inp["x"]), p_ref, s_ref)
    assert y.shape == (M, N)
    assert_close(y, y_ref, D, K, torch.float16, strict=True, label=f"{name} M={M}")


def test_forward_is_exact_integer_sum():
    """With x rows whose quantization is exact (absmax 127, integer values)
    and unit scales, y equals the exact integer product."""
    M, K, N = 130, 512, 136
    rng = np.random.default_rng(3)
    xi = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    xi[:, 0] = 127.0
    codes = rng.integers(1, 16, size=(K, N))
    codes[0, :] = 15                                     # column absmax 7 -> scale 1
    w = (codes - 8).astype(np.float32)
    packed, s = qlq.w4a8_pack_weight_int4(torch.from_numpy(w).to(dev()))
    assert torch.equal(s.cpu(), torch.ones(N))
    y = qlq.w4a8_linear_forward(torch.from_numpy(xi).to(dev()).to(torch.float16), packed, s)
    exact = xi.astype(np.int64) @ (codes - 8)
    assert np.abs(exact).max() < 65504                    # finite in fp16
    ref = torch.from_numpy(exact.astype(np.float32)).to(torch.float16)
    assert torch.equal(y.cpu(), ref)


def test_zero_input_gives_bias():
    K, N = 512, 40
    w = torch.randn(K, N, device=dev())
    packed, s = qlq.w4a8_pack_weight_int4(w)
    bias = (torch.arange(N, device=dev(), dtype=torch.float32) / 8).to(torch.float16)
    y = qlq.w4a8_linear_forward(torch.zeros(5, K, device=dev(), dtype=torch.float16), packed, s, bias=bias)
    assert torch.equal(y, bias.expand(5, N))


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,K,N", [
    (1, 4096, 4096), (2, 4096, 1024), (1, 8192, 64), (2, 16384, 32), (2, 272, 144), (1, 16, 16),
    (1, 1040, 4096), (1, 1040, 520), (2, 272, 132), (3, 1040, 517), (4, 128, 260), (5, 2048, 384), (8, 16, 4),
    (7, 784, 1)])
def test_skinny_and_gemm_paths_identical(xdt, M, K, N):
    """M <= 8 runs split over K; the GEMM gives the same exact int32 sums and
    the same epilogue, so the two outputs must be bit-identical."""
    inp = workloads.w4a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=True, seed=M + K + N, outlier_frac=0.01)
    packed, s = qlq.w4a8_pack_weight_int4(inp["w"].to(dev()))
    x, b = inp["x"].to(dev()), inp["bias"].to(dev())
    old = qlq.qlq_get_skinny_max_m()
    try:
        qlq.qlq_set_skinny_max_m(8)
        y_skinny = qlq.w4a8_linear_forward(x, packed, s, bias=b)
        qlq.qlq_set_skinny_max_m(0)
        y_gemm = qlq.w4a8_linear_forward(x, packed, s, bias=b)
    finally:
        qlq.qlq_set_skinny_max_m(old)
    assert torch.equal(y_skinny.view(torch.int16), y_gemm.view(torch.int16))
    p_ref, s_ref = oracle.pack_weight_int4(inp["w"].numpy())
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    _, _, _, y_ref, D = oracle.w4a8_forward(f32(inp["x"]), p_ref, s_ref, bias=f32(inp["bias"]))
    assert_close(y_skinny, y_ref, D, K, xdt, label=f"w4a8 skinny {xdt} {(M, K, N)}")
