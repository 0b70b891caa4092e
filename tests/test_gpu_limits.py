"""GPU parity at the documented limits: the largest K each int8 path accepts
with inputs that drive the int32 sums to their extreme (every product at its
largest magnitude, one sign), the per-group matrix-vector kernel at its K
cap, a long-K affine decode, and empty batches through every binding."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import assert_close, dev, f32

pytestmark = pytest.mark.gpu

KMAX16 = 131071 - 131071 % 16      # largest K a 16-aligned int8 path accepts


def test_w8a8_extreme_sum_at_max_k():
    # x rows of +-1 (quantize to +-127), weights +-1 (quantize to +-127):
    # |acc| = 127 * 127 * K, the largest the path can meet
    M, K, N = 3, KMAX16, 24
    x = torch.ones(M, K, dtype=torch.bfloat16)      # outputs near 1.3e5: beyond fp16
    x[1] = -1.0
    x[2, ::2] = -1.0
    w = torch.ones(N, K)
    w[5] = -1.0
    wq, sw = qlq.qlq_quantize_rows_int8(w.to(dev()))
    wq_ref, sw_ref = oracle.quantize_rows_int8(w.numpy())
    xq_ref, _ = oracle.quantize_rows_int8(f32(x))
    assert np.array_equal(wq.cpu().numpy(), wq_ref) and np.array_equal(sw.cpu().numpy(), sw_ref)
    acc = qlq.qlq_int8_matmul_int32(qlq.qlq_quantize_rows_int8(x.to(dev()))[0], wq)
    ref = oracle.int8_matmul_int32(xq_ref, wq_ref)
    assert np.abs(ref).max() == 127 * 127 * K < 2 ** 31
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref)
    y = qlq.w8a8_linear_forward(x.to(dev()), wq, sw)
    *_, y_ref, D = oracle.w8a8_forward(f32(x), wq_ref, sw_ref)
    assert_close(y, y_ref, D, K, torch.bfloat16, label="w8a8 K max")  # half an output ulp exceeds the strict bound here


@pytest.mark.parametrize("M", [1, 8, 9])                      # skinny path, both sides of its bound
def test_w4a8_extreme_sum_at_max_k(M):
    # x = +-1 (xq = +-127), int4 codes 1 (value -7) or 15 (+7): the kernels
    # carry 16 (code - 8), so their int32 sums reach 127 * 16 * 7 * K
    K, N = KMAX16, 20
    x = torch.ones(M, K, dtype=torch.bfloat16)      # outputs near 9e5: beyond fp16
    x[0, 1::3] = -1.0
    w = torch.full((K, N), -7.0)
    w[:, 3] = 7.0
    packed, s = qlq.w4a8_pack_weight_int4(w.to(dev()))
    p_ref, s_ref = oracle.pack_weight_int4(w.numpy())
    assert np.array_equal(packed.cpu().numpy(), p_ref)
    *_, acc_ref, y_ref, D = oracle.w4a8_forward(f32(x), p_ref, s_ref)
    assert 16 * np.abs(acc_ref).max() < 2 ** 31
    old = qlq.qlq_get_skinny_max_m()
    try:
        outs = []
        for thr in (8, 0):
            qlq.qlq_set_skinny_max_m(thr)
            y = qlq.w4a8_linear_forward(x.to(dev()), packed, s)
            assert_close(y, y_ref, D, K, torch.bfloat16, label=f"w4a8 K max M={M} thr={thr}")
            outs.append(y)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    finally:
        qlq.qlq_set_skinny_max_m(old)


def test_pergroup_mv_at_k_cap():
    K, N, G = 16384, 96, 256
    inp = workloads.w8a8_inputs(1, K, N, x_dtype="bf16", bias=True, seed=77)
    q, sg = qlq.qlq_quantize_groups_int8(inp["w"].to(dev()), G)
    q_ref, s_ref = oracle.quantize_groups_int8(inp["w"].numpy(), G)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sg.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    y = qlq.pergroup_linear_forward(inp["x"].to(dev()), q, sg, G, bias=inp["bias"].to(dev()))
    y_ref, D = oracle.pergroup_forward(f32(inp["x"]), q_ref, s_ref, G, bias=f32(inp["bias"]))
    assert_close(y, y_ref, D, K, torch.bfloat16, strict=True, label="pergroup M=1 K cap")
    with pytest.raises(qlq.QLQError) as e:
        qlq.pergroup_linear_forward(torch.zeros(1, K + G, dtype=torch.bfloat16, device=dev()),
                                    torch.zeros(N, K + G, dtype=torch.int8, device=dev()),
                                    torch.ones((K + G) // G, N, device=dev()), G)
    assert e.value.code == qlq.QLQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("bits", [3, 4])
def test_affine_long_k_decode(bits):
    M, K, N, G = 2, 32768, 64, 128
    inp = workloads.affine_inputs(M, K, N, x_dtype="bf16", bias=True, seed=88 + bits)
    packed, scales, biases = qlq.qlq_pack(inp["w"].to(dev()), bits, G, torch.bfloat16)
    y = qlq.qlq_linear_forward(inp["x"].to(dev()), packed, scales, biases, bits, G, bias=inp["bias"].to(dev()))
    codes, s_ref, b_ref = oracle.affine_quantize(inp["w"].numpy(), bits, G, "bf16")
    y_ref, D = oracle.affine_forward(f32(inp["x"]), codes, s_ref, b_ref, G, bias=f32(inp["bias"]))
    assert_close(y, y_ref, D, K, torch.bfloat16, strict=True, label=f"affine K={K} bits={bits}")


def test_empty_batches():
    d = dev()
    w = torch.randn(64, 256, device=d)
    packed, scales, biases = qlq.qlq_pack(w, 4, 64, torch.bfloat16)
    y = qlq.qlq_linear_forward(torch.zeros(0, 256, dtype=torch.bfloat16, device=d), packed, scales, biases, 4, 64)
    assert y.shape == (0, 64)
    tp = qlq.bitlinear_pack(torch.zeros(64, 256, dtype=torch.int8, device=d))
    ws = torch.ones(1, dtype=torch.bfloat16, device=d)
    assert qlq.bitlinear_forward(torch.zeros(0, 256, dtype=torch.bfloat16, device=d), tp, 64, ws).shape == (0, 64)
    wq, sw = qlq.qlq_quantize_rows_int8(w)
    x0 = torch.zeros(0, 256, dtype=torch.float16, device=d)
    assert qlq.w8a8_linear_forward(x0, wq, sw).shape == (0, 64)
    q, sg = qlq.qlq_quantize_groups_int8(w, 128)
    assert qlq.pergroup_linear_forward(x0, q, sg, 128).shape == (0, 64)
    p4, s4 = qlq.w4a8_pack_weight_int4(w.T.contiguous())
    assert qlq.w4a8_linear_forward(x0, p4, s4).shape == (0, 64)
