"""The allocation-free W8A8 entry point (w8a8_linear_forward_noalloc), called
through the C ABI: on two calls in a row, the second with a smaller input, its
output is bit-identical to w8a8_linear_forward's (same kernels, same int32
sums, same epilogue) and within the tolerance rule of the oracle, which runs
on its own quantized weights."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32

pytestmark = pytest.mark.gpu


def _noalloc_c(x, wq, sw, bias, y):
    """One call of the C entry point on torch's current stream."""
    M, K = x.shape
    N = wq.shape[0]
    vp = ctypes.c_void_p
    st = qlq.lib().w8a8_linear_forward_noalloc(
        vp(x.data_ptr()), qlq.DTYPE_CODE[x.dtype], M, K, vp(wq.data_ptr()), vp(sw.data_ptr()), N,
        None if bias is None else vp(bias.data_ptr()), vp(y.data_ptr()),
        vp(torch.cuda.current_stream().cuda_stream))
    if st:
        raise qlq.QLQError(st, qlq.last_error())


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
def test_noalloc_matches_workspace_call_twice(xdt):
    # the first call fills more of the shared scratch than the second reads
    cases = [(1024, 4096, 520, True, 31), (37, 1040, 130, False, 32)]
    for M, K, N, with_bias, seed in cases:
        print(f"[noalloc] {xdt} M={M} K={K} N={N} bias={with_bias} seed={seed}", flush=True)
        inp = workloads.w8a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=with_bias, seed=seed, outlier_frac=0.01)
        wq_ref, sw_ref = oracle.quantize_rows_int8(inp["w"].numpy())
        x = inp["x"].to(dev())
        wq = torch.from_numpy(wq_ref).to(dev())
        sw = torch.from_numpy(sw_ref).to(dev())
        bias = None if inp["bias"] is None else inp["bias"].to(dev())
        y_ws = qlq.w8a8_linear_forward(x, wq, sw, bias=bias)
        y_na = torch.full((M, N), float("nan"), dtype=xdt, device=dev())
        _noalloc_c(x, wq, sw, bias, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), (M, K, N)
        *_, y_ref, D = oracle.w8a8_forward(f32(inp["x"]), wq_ref, sw_ref,
                                           bias=None if inp["bias"] is None else f32(inp["bias"]))
        assert_close(y_na, y_ref, D, K, xdt, label=f"noalloc {xdt} {(M, K, N)}")


def test_noalloc_binding_and_largest_input():
    # the binding with a preallocated output, at the largest M for K = 4096
    K, N = 4096, 96
    cap = qlq.W8A8_NOALLOC_SCRATCH_BYTES
    M = 4092                                   # xq 4092 * 4096 bytes + sx 4092 * 4 fit; 4093 rows do not
    assert qlq.w8a8_workspace_size(M, K) <= cap < qlq.w8a8_workspace_size(M + 1, K)
    inp = workloads.w8a8_inputs(M, K, N, x_dtype="f16", seed=33)
    wq_ref, sw_ref = oracle.quantize_rows_int8(inp["w"].numpy())
    x = inp["x"].to(dev())
    wq, sw = torch.from_numpy(wq_ref).to(dev()), torch.from_numpy(sw_ref).to(dev())
    out = torch.empty(M, N, dtype=torch.float16, device=dev())
    y = qlq.w8a8_linear_forward_noalloc(x, wq, sw, out=out)
    assert y.data_ptr() == out.data_ptr()
    y_ws = qlq.w8a8_linear_forward(x, wq, sw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16))
    with pytest.raises(qlq.QLQError) as e:
        qlq.w8a8_linear_forward_noalloc(torch.zeros(M + 1, K, dtype=torch.float16, device=dev()), wq, sw)
    assert e.value.code == qlq.QLQ_ERR_WORKSPACE
