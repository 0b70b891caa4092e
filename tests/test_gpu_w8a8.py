"""GPU parity for W8A8: row int8 quantization and the int32 accumulators are
bit-exact against the oracle; the scaled output is within the tolerance rule."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("vdt", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("K", [16, 1008, 2048, 4096, 4096 + 64])
def test_quantize_rows_bitexact(vdt, K):
    inp = workloads.w8a8_inputs(97, K, 8, x_dtype=ODT[vdt], seed=21 + K)
    v = inp["x"]
    v[5] = 0  # a zero row takes scale 1
    q, s = qlq.qlq_quantize_rows_int8(v.to(dev()))
    q_ref, s_ref = oracle.quantize_rows_int8(f32(v))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def _all_values_up_to(amax, dt):
    """Every finite value of dt (f16 or bf16) with |v| <= amax, both signs."""
    if dt == torch.float16:
        bits = np.arange(0, 0x7C00, dtype=np.uint16)
        vals = bits.view(np.float16).astype(np.float32)
    else:
        bits = np.arange(0, 0x7F80, dtype=np.uint32)
        vals = (bits << 16).view(np.float32)
    vals = vals[vals <= amax]
    return np.concatenate([vals, -vals[1:]])


@pytest.mark.parametrize("vdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("amax", [1.0, 0.37890625, 3.140625, 1000.0, 6.103515625e-05])
def test_quantize_rows_every_value_bitexact(vdt, amax):
    # each quotient v / (amax / 127) against the oracle's IEEE division: every
    # representable v up to the row maximum, for the wave-per-row kernel
    # (rows of 4096) and the block-per-row kernel (one row of 32768)
    vals = _all_values_up_to(amax, vdt)
    for K in (4096, 32768):
        per = K - 1
        nrows = (len(vals) + per - 1) // per
        if K == 32768 and nrows > 1:
            vals_k = vals[:per]
            nrows = 1
        else:
            vals_k = vals
        rows = np.zeros((nrows, K), dtype=np.float32)
        rows[:, 0] = amax
        flat = rows[:, 1:].reshape(-1)
        flat[: len(vals_k)] = vals_k
        rows[:, 1:] = flat.reshape(nrows, per)
        v = torch.from_numpy(rows).to(vdt)
        assert torch.equal(v.float(), torch.from_numpy(rows)), "values representable"
        q, sc = qlq.qlq_quantize_rows_int8(v.to(dev()))
        q_ref, s_ref = oracle.quantize_rows_int8(rows)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), (K, amax)
        assert np.array_equal(q.cpu().numpy(), q_ref), (K, amax)


def test_quantize_rows_workload_bitexact():
    inp = workloads.workload_inputs("w8a8_perchannel")
    q, s = qlq.qlq_quantize_rows_int8(inp["x"].to(dev()))
    q_ref, s_ref = oracle.quantize_rows_int8(f32(inp["x"]))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    # weights go through the same quantizer
    qw, sw = qlq.qlq_quantize_rows_int8(inp["w"].to(dev()))
    qw_ref, sw_ref = oracle.quantize_rows_int8(inp["w"].numpy())
    assert np.array_equal(qw.cpu().numpy(), qw_ref)
    assert np.array_equal(sw.cpu().numpy(), sw_ref)


@pytest.mark.parametrize("shape", [(77, 45, 208), (1, 1, 16), (128, 128, 128), (130, 257, 4096 + 16)])
def test_int8_matmul_bitexact(shape):
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    b = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    c = qlq.qlq_int8_matmul_int32(torch.from_numpy(a).to(dev()), torch.from_numpy(b).to(dev()))
    assert np.array_equal(c.cpu().numpy().astype(np.int64), oracle.int8_matmul_int32(a, b))


def test_int8_matmul_extremes():
    K = 4096
    a = torch.full((3, K), -128, dtype=torch.int8, device=dev())
    b = torch.full((5, K), -128, dtype=torch.int8, device=dev())
    b[1] = 127
    c = qlq.qlq_int8_matmul_int32(a, b)
    assert (c[:, 0] == 2 ** 26).all() and (c[:, 1] == -128 * 127 * K).all()


def test_int8_matmul_workload_full():
    """Every int32 sum of the workload's product, bit-exact, on the oracle's
    own quantized operands."""
    inp = workloads.workload_inputs("w8a8_perchannel")
    xq, _ = oracle.quantize_rows_int8(f32(inp["x"]))
    wq, _ = oracle.quantize_rows_int8(inp["w"].numpy())
    c = qlq.qlq_int8_matmul_int32(torch.from_numpy(xq).to(dev()), torch.from_numpy(wq).to(dev()))
    ref = oracle.int8_matmul_int32(xq, wq)
    assert c.shape == (1024, 4096)
    assert np.array_equal(c.cpu().numpy().astype(np.int64), ref)


def _w8a8_case(inp):
    x, w, bias = inp["x"], inp["w"], inp["bias"]
    wq, sw = qlq.qlq_quantize_rows_int8(w.to(dev()))
    y = qlq.w8a8_linear_forward(x.to(dev()), wq, sw, bias=None if bias is None else bias.to(dev()))
    torch.cuda.synchronize()
    wq_ref, sw_ref = oracle.quantize_rows_int8(w.numpy())
    assert np.array_equal(wq.cpu().numpy(), wq_ref)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), sw_ref.view(np.uint32))
    _, _, _, y_ref, D = oracle.w8a8_forward(f32(x), wq_ref, sw_ref, bias=None if bias is None else f32(bias))
    return y, y_ref, D


def test_w8a8_workload_full():
    inp = workloads.workload_inputs("w8a8_perchannel")
    y, y_ref, D = _w8a8_case(inp)
    assert y.shape == (1024, 4096)
    assert_close(y, y_ref, D, 4096, torch.float16, strict=True, label="w8a8 workload")


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 64, 16), (37, 208, 45), (130, 512, 300)])
def test_w8a8_variants(xdt, shape):
    M, K, N = shape
    inp = workloads.w8a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=True, seed=M + K + N, outlier_frac=0.01)
    y, y_ref, D = _w8a8_case(inp)
    assert_close(y, y_ref, D, K, xdt, label=f"w8a8 {xdt} {shape}")


def _fused_vs_unfused(x, wq, sw, bias=None, noalloc=False):
    fwd = qlq.w8a8_linear_forward_noalloc if noalloc else qlq.w8a8_linear_forward
    old = qlq.qlq_get_w8a8_fused_quant()
    try:
        qlq.qlq_set_w8a8_fused_quant(0)
        y0 = fwd(x, wq, sw, bias=bias)
        qlq.qlq_set_w8a8_fused_quant(1)
        y1 = fwd(x, wq, sw, bias=bias)
    finally:
        qlq.qlq_set_w8a8_fused_quant(old)
    torch.cuda.synchronize()
    return y0, y1


def test_fused_quant_workload_bit_identical():
    """The activation quantizer inside the GEMM gives the same codes, sums
    and epilogue as the quantizer before it: bit-identical outputs on the
    full workload, and within the tolerance rule of the oracle."""
    inp = workloads.workload_inputs("w8a8_perchannel")
    wq_ref, sw_ref = oracle.quantize_rows_int8(inp["w"].numpy())
    wq, sw = torch.from_numpy(wq_ref).to(dev()), torch.from_numpy(sw_ref).to(dev())
    y0, y1 = _fused_vs_unfused(inp["x"].to(dev()), wq, sw)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    _, _, _, y_ref, D = oracle.w8a8_forward(f32(inp["x"]), wq_ref, sw_ref)
    assert_close(y1, y_ref, D, 4096, torch.float16, strict=True, label="w8a8 fused quant workload")


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 64, 16), (37, 208, 45), (130, 512, 300), (129, 4112, 257), (300, 1040, 128)])
@pytest.mark.parametrize("noalloc", [False, True])
def test_fused_quant_ragged_bit_identical(xdt, shape, noalloc):
    # K tails inside a 256-wide k-iteration, M and N not multiples of 128
    M, K, N = shape
    inp = workloads.w8a8_inputs(M, K, N, x_dtype=ODT[xdt], bias=True, seed=M + 3 * K + N, outlier_frac=0.01)
    wq_ref, sw_ref = oracle.quantize_rows_int8(inp["w"].numpy())
    wq, sw = torch.from_numpy(wq_ref).to(dev()), torch.from_numpy(sw_ref).to(dev())
    y0, y1 = _fused_vs_unfused(inp["x"].to(dev()), wq, sw, bias=inp["bias"].to(dev()), noalloc=noalloc)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), shape
    _, _, _, y_ref, D = oracle.w8a8_forward(f32(inp["x"]), wq_ref, sw_ref, bias=f32(inp["bias"]))
    assert_close(y1, y_ref, D, K, xdt, label=f"w8a8 fused quant {xdt} {shape}")


@pytest.mark.parametrize("vdt", [torch.float16, torch.bfloat16])
def test_fused_quant_every_value(vdt):
    # every representable value up to a row maximum through the in-GEMM
    # quantizer, with an identity-like weight that exposes each code: w row n
    # has a single 1 at k = n, so the int32 sum of output n is x's code at n
    amax = 3.140625
    vals = _all_values_up_to(amax, vdt)
    K = 4096
    per = K - 1
    rows = np.zeros(((len(vals) + per - 1) // per, K), dtype=np.float32)
    rows[:, 0] = amax
    flat = rows[:, 1:].reshape(-1)
    flat[: len(vals)] = vals
    rows[:, 1:] = flat.reshape(rows.shape[0], per)
    x = torch.from_numpy(rows).to(vdt)
    xq_ref, sx_ref = oracle.quantize_rows_int8(f32(x))
    eye = np.zeros((K, K), dtype=np.float32)
    np.fill_diagonal(eye, 1.0)
    wq_ref, sw_ref = oracle.quantize_rows_int8(eye)       # 127 on the diagonal, scale 1/127
    wq, sw = torch.from_numpy(wq_ref).to(dev()), torch.from_numpy(sw_ref).to(dev())
    y0, y1 = _fused_vs_unfused(x.to(dev()), wq, sw)
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
