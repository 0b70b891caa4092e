"""GPU checks beyond parity: device check, guard bands around outputs,
non-default streams and run-to-run determinism."""

import numpy as np
import pytest
import torch

import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import dev

pytestmark = pytest.mark.gpu

PAD = 64  # elements of guard band on each side (keeps 16-byte alignment)


def test_device_check():
    assert qlq.qlq_device_check(0) == 0
    assert qlq.qlq_device_check(63) == qlq.QLQ_ERR_DEVICE


def _guarded(M, N, dtype):
    buf = torch.full((M * N + 2 * PAD,), -7.0, dtype=dtype, device=dev())
    return buf, buf[PAD:PAD + M * N].view(M, N)


def _guard_ok(buf, M, N):
    g = torch.cat([buf[:PAD], buf[PAD + M * N:]]).float()
    return bool((g == -7.0).all())


@pytest.mark.parametrize("M", [1, 5, 200])
def test_linear_guard_bands(M):
    K, N = 256, 129
    inp = workloads.affine_inputs(M, K, N, bias=True, seed=M)
    packed, scales, biases = qlq.qlq_pack(inp["w"].to(dev()), 4, 64, torch.bfloat16)
    buf, y = _guarded(M, N, torch.bfloat16)
    qlq.qlq_linear_forward(inp["x"].to(dev()), packed, scales, biases, 4, 64, bias=inp["bias"].to(dev()), out=y)
    torch.cuda.synchronize()
    assert _guard_ok(buf, M, N)
    assert torch.isfinite(y.float()).all()


def test_ternary_and_w8a8_guard_bands():
    M, K, N = 19, 128, 4 * 33
    t = workloads.ternary_inputs(M, K, N, seed=1)
    packed = qlq.bitlinear_pack(t["t"].to(dev()))
    buf, y = _guarded(M, N, torch.bfloat16)
    qlq.bitlinear_forward(t["x"].to(dev()), packed, N, t["weight_scale"].to(dev()), out=y)
    torch.cuda.synchronize()
    assert _guard_ok(buf, M, N)
    w = workloads.w8a8_inputs(M, K, N, seed=2)
    wq, sw = qlq.qlq_quantize_rows_int8(w["w"].to(dev()))
    buf, y = _guarded(M, N, torch.float16)
    qlq.w8a8_linear_forward(w["x"].to(dev()), wq, sw, out=y)
    torch.cuda.synchronize()
    assert _guard_ok(buf, M, N)


def test_non_default_stream_and_determinism():
    inp = workloads.affine_inputs(300, 512, 260, bias=True, seed=5)
    packed, scales, biases = qlq.qlq_pack(inp["w"].to(dev()), 4, 128, torch.bfloat16)
    x = inp["x"].to(dev())
    b = inp["bias"].to(dev())
    y0 = qlq.qlq_linear_forward(x, packed, scales, biases, 4, 128, bias=b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y1 = qlq.qlq_linear_forward(x, packed, scales, biases, 4, 128, bias=b)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    a = torch.randint(-128, 128, (70, 256), dtype=torch.int8, device=dev())
    bb = torch.randint(-128, 128, (90, 256), dtype=torch.int8, device=dev())
    c0 = qlq.qlq_int8_matmul_int32(a, bb)
    c1 = qlq.qlq_int8_matmul_int32(a, bb)
    assert torch.equal(c0, c1)
