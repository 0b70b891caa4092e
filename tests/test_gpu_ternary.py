"""GPU parity for ternary BitLinear: bitlinear_pack is bit-exact against the
oracle; bitlinear_forward is within the tolerance rule."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32

pytestmark = pytest.mark.gpu


def _case(inp, N, invert=False, rows=None):
    x, t = inp["x"], inp["t"]
    packed = qlq.bitlinear_pack(t.to(dev()))
    ref_packed = oracle.ternary_pack(t.numpy())
    assert np.array_equal(packed.cpu().numpy(), ref_packed)
    bias = inp["bias"]
    y = qlq.bitlinear_forward(x.to(dev()), packed, N, inp["weight_scale"].to(dev()), invert,
                              bias=None if bias is None else bias.to(dev()))
    torch.cuda.synchronize()
    y_ref, D = oracle.ternary_forward(f32(x), ref_packed, N, float(f32(inp["weight_scale"])[0]), invert,
                                      bias=None if bias is None else f32(bias))
    return y, y_ref, D


def test_forward_workload_full():
    name = "ternary_bitlinear"
    cfg = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name)
    # the stored scale is bf16(0.05), not 0.05
    assert float(inp["weight_scale"].float()[0]) == 0.050048828125
    y, y_ref, D = _case(inp, cfg["N"], cfg["invert"])
    assert_close(y, y_ref, D, cfg["K"], torch.bfloat16, label=name)


@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("M", [1, 3, 8, 16, 17, 40])
@pytest.mark.parametrize("invert", [False, True])
def test_forward_variants(xdt, M, invert):
    N, K = 4 * 37, 96
    inp = workloads.ternary_inputs(M, K, N, x_dtype=ODT[xdt], weight_scale=0.3, bias=(M % 2 == 1),
                                   seed=M * 7 + int(invert))
    y, y_ref, D = _case(inp, N, invert)
    assert_close(y, y_ref, D, K, xdt, label=f"ternary {xdt} M={M} invert={invert}")


def test_forward_large_k_ragged_rows():
    N, K, M = 4 * 45, 4096, 5
    inp = workloads.ternary_inputs(M, K, N, seed=11, bias=True)
    y, y_ref, D = _case(inp, N)
    assert_close(y, y_ref, D, K, torch.bfloat16, label="ternary K=4096")


def test_forward_many_blocks_ragged():
    # a grid of 129 x 4 blocks with a ragged last block in both directions
    # (R = 2053 packed rows, M = 61)
    N, K, M = 4 * 2053, 128, 61
    inp = workloads.ternary_inputs(M, K, N, seed=12, bias=True)
    y, y_ref, D = _case(inp, N)
    assert_close(y, y_ref, D, K, torch.bfloat16, label="ternary wide blocks")


def test_pack_rejects_out_of_set():
    t = torch.zeros(8, 32, dtype=torch.int8, device=dev())
    t[3, 4] = 2
    with pytest.raises(qlq.QLQError) as e:
        qlq.bitlinear_pack(t)
    assert e.value.code == qlq.QLQ_ERR_DATA


def test_code_three_decodes_literally():
    """A byte the packer never emits (all fields = 3) decodes to +2."""
    M, K, N = 2, 64, 8
    packed_host = np.full((N // 4, K), 0xFF, dtype=np.uint8)
    packed = torch.from_numpy(packed_host).to(dev())
    x = torch.ones(M, K, dtype=torch.bfloat16, device=dev())
    ws = torch.ones(1, dtype=torch.bfloat16, device=dev())
    y = qlq.bitlinear_forward(x, packed, N, ws)
    y_ref, _ = oracle.ternary_forward(np.ones((M, K)), packed_host, N, 1.0)
    assert np.array_equal(f32(y), y_ref.astype(np.float32))
    assert (y_ref == 2 * K).all()


def test_identities():
    """x = ones gives sigma * (#plus - #minus) exactly; all-zero weights give the bias."""
    N, K = 4 * 9, 128
    t = torch.from_numpy(np.random.default_rng(3).integers(-1, 2, size=(N, K)).astype(np.int8))
    packed = qlq.bitlinear_pack(t.to(dev()))
    ws = torch.tensor([0.25], dtype=torch.bfloat16, device=dev())
    y = qlq.bitlinear_forward(torch.ones(1, K, dtype=torch.bfloat16, device=dev()), packed, N, ws)
    want = 0.25 * ((t == 1).sum(1) - (t == -1).sum(1)).float()
    assert torch.equal(y.float().cpu()[0], want.to(torch.bfloat16).float())
    # all-zero weights: the kernel's sum x*(OFF + 1) - (OFF + 1)*sum x cancels
    # only up to fp32 rounding, so this case is held to the tolerance rule
    zero_t = np.zeros((N, K), dtype=np.int8)
    zero = qlq.bitlinear_pack(torch.from_numpy(zero_t).to(dev()))
    bias = torch.randn(N, device=dev()).to(torch.bfloat16)
    x = torch.randn(3, K, device=dev()).to(torch.bfloat16)
    y = qlq.bitlinear_forward(x, zero, N, ws, bias=bias)
    y_ref, D = oracle.ternary_forward(f32(x), oracle.ternary_pack(zero_t), N, 0.25, bias=f32(bias))
    assert np.array_equal(y_ref, np.broadcast_to(f32(bias), (3, N)))
    assert_close(y, y_ref, D, K, torch.bfloat16, label="ternary zero weights")


@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("M,K,N", [(3, 5120, 4 * 37), (17, 2560, 4 * 21), (8, 2560, 4 * 1728)])
def test_forward_unmasked_windows(xdt, M, K, N):
    # K a multiple of 128 whose 128-k windows split evenly over the waves:
    # the kernel variant with no masking; ragged packed rows and x rows
    inp = workloads.ternary_inputs(M, K, N, x_dtype=ODT[xdt], weight_scale=0.05, bias=True, seed=M + K)
    y, y_ref, D = _case(inp, N)
    assert_close(y, y_ref, D, K, xdt, label=f"ternary unmasked {xdt} {(M, K, N)}")
