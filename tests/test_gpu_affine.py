"""GPU parity for the affine path: qlq_pack / qlq_unpack / qlq_dequantize are
bit-exact against the oracle; qlq_linear_forward (skinny and GEMM kernels)
is within the tolerance rule, on the full workloads and on ragged shapes."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import bit_weight_quantized_qlq_amd as qlq
from parity import ODT, assert_close, dev, f32, u32

pytestmark = pytest.mark.gpu


def _pack_both(w_cpu, bits, G, sb):
    """GPU pack and oracle quantize+pack of the same fp32 weights."""
    packed, scales, biases = qlq.qlq_pack(w_cpu.to(dev()), bits, G, sb)
    codes, s_ref, b_ref = oracle.affine_quantize(w_cpu.numpy(), bits, G, ODT[sb])
    return (packed, scales, biases), (codes, s_ref, b_ref)


def _assert_pack_equal(gpu, ref, bits):
    packed, scales, biases = gpu
    codes, s_ref, b_ref = ref
    assert np.array_equal(u32(packed), oracle.affine_pack(codes, bits))
    assert np.array_equal(f32(scales), s_ref)
    assert np.array_equal(f32(biases), b_ref)


@pytest.mark.parametrize("name", ["tiny_affine_4bit", "decode_gemv_4bit", "prefill_gemm_4bit"])
def test_pack_bitexact_workloads(name):
    cfg = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name)
    sb = workloads.TORCH_DTYPE[cfg["sb_dtype"]]
    gpu, ref = _pack_both(inp["w"], cfg["bits"], cfg["group_size"], sb)
    _assert_pack_equal(gpu, ref, cfg["bits"])


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("sb", [torch.float32, torch.float16, torch.bfloat16])
def test_pack_bitexact_variants(bits, G, sb):
    w = workloads.affine_inputs(1, 384, 37, seed=bits * 100 + G)["w"]
    gpu, ref = _pack_both(w, bits, G, sb)
    _assert_pack_equal(gpu, ref, bits)


def test_pack_degenerate_groups():
    w = torch.zeros(6, 256)
    w[1] = 0.375
    w[2] = -3.0
    w[3, :64] = 1e-30          # tiny but equal values
    w[4] = torch.linspace(-1, 1, 256)
    w[5, ::2] = 1.0
    for sb in (torch.float32, torch.bfloat16, torch.float16):
        gpu, ref = _pack_both(w, 4, 64, sb)
        _assert_pack_equal(gpu, ref, 4)


def test_pack_rejects_non_finite():
    w = torch.zeros(4, 128, device=dev())
    w[2, 5] = float("inf")
    with pytest.raises(qlq.QLQError) as e:
        qlq.qlq_pack(w, 4, 64, torch.bfloat16)
    assert e.value.code == qlq.QLQ_ERR_DATA
    w[2, 5] = 1e5
    w[2, 6] = -1e5               # scale and bias overflow fp16 storage
    with pytest.raises(qlq.QLQError) as e:
        qlq.qlq_pack(w, 4, 64, torch.float16)
    assert e.value.code == qlq.QLQ_ERR_DATA


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("N,K", [(33, 512), (7, 48)])   # 7 x 48 codes: a partial last unit at 2 bits
def test_unpack_bitexact(bits, N, K):
    if (K * bits) % 32:
        pytest.skip("rows must be whole words")
    rng = np.random.default_rng(40 + bits)
    words = rng.integers(0, 1 << 32, size=(N, K * bits // 32), dtype=np.uint64).astype(np.uint32)
    packed = torch.from_numpy(words.view(np.int32)).to(dev())
    codes = qlq.qlq_unpack(packed, K, bits)
    assert np.array_equal(codes.cpu().numpy(), oracle.affine_unpack(words, K, bits))


@pytest.mark.parametrize("bits,G,sb", [(4, 64, torch.bfloat16), (4, 128, torch.float16),
                                       (2, 32, torch.float32), (8, 64, torch.bfloat16),
                                       (3, 64, torch.bfloat16), (5, 32, torch.float32),
                                       (6, 128, torch.float16), (1, 64, torch.bfloat16)])
def test_dequantize_bitexact(bits, G, sb):
    w = workloads.affine_inputs(1, 512, 29, seed=7)["w"]
    (packed, scales, biases), (codes, s_ref, b_ref) = _pack_both(w, bits, G, sb)
    wd = qlq.qlq_dequantize(packed, scales, biases, 512, bits, G)
    ref = oracle.affine_dequantize(codes, s_ref, b_ref, G).astype(np.float32)
    assert np.array_equal(f32(wd).view(np.uint32), ref.view(np.uint32))


def _forward_case(inp, bits, G, x_dtype):
    """Pack on the GPU (checked bit-exact against the oracle's packing), run
    the forward, and return (y_gpu, y_ref, D) with y_ref computed from the
    oracle's own codes, scales and biases."""
    x = inp["x"]
    bias = inp["bias"]
    packed, scales, biases = qlq.qlq_pack(inp["w"].to(dev()), bits, G, x_dtype)
    y = qlq.qlq_linear_forward(x.to(dev()), packed, scales, biases, bits, G,
                               bias=None if bias is None else bias.to(dev()))
    torch.cuda.synchronize()
    codes, s_ref, b_ref = oracle.affine_quantize(inp["w"].numpy(), bits, G, ODT[x_dtype])
    assert np.array_equal(u32(packed), oracle.affine_pack(codes, bits))
    assert np.array_equal(f32(scales), s_ref) and np.array_equal(f32(biases), b_ref)
    y_ref, D = oracle.affine_forward(f32(x), codes, s_ref, b_ref, G,
                                     bias=None if bias is None else f32(bias))
    return y, y_ref, D


@pytest.mark.parametrize("name", ["tiny_affine_4bit", "decode_gemv_4bit", "decode_gemv_3bit"])
def test_forward_workloads_skinny(name):
    cfg = workloads.WORKLOADS[name]
    inp = workloads.workload_inputs(name)
    xdt = workloads.TORCH_DTYPE[cfg["x_dtype"]]
    y, y_ref, D = _forward_case(inp, cfg["bits"], cfg["group_size"], xdt)
    assert_close(y, y_ref, D, cfg["K"], xdt, strict=True, label=name)


@pytest.mark.parametrize("name", ["prefill_gemm_4bit", "prefill_gemm_3bit"])
def test_forward_prefill_full(name):
    """Full prefill workload through the GEMM kernel, every output element
    against the oracle."""
    cfg = workloads.WORKLOADS[name]
    assert cfg["M"] > qlq.qlq_get_skinny_max_m()
    inp = workloads.workload_inputs(name)
    y, y_ref, D = _forward_case(inp, cfg["bits"], cfg["group_size"], torch.bfloat16)
    assert y.shape == (cfg["M"], cfg["N"])
    assert_close(y, y_ref, D, cfg["K"], torch.bfloat16, strict=True, label=name)


SHAPES = [  # (M, K, N, bits, G)
    (1, 416, 200, 4, 32), (2, 448, 130, 4, 64), (3, 640, 77, 4, 128), (5, 448, 64, 2, 64),
    (8, 384, 129, 8, 128), (9, 416, 200, 4, 32), (17, 448, 250, 2, 64), (33, 640, 131, 4, 128),
    (130, 384, 257, 8, 64), (1, 4096, 96, 4, 64), (20, 416, 72, 2, 32), (40, 4160, 72, 4, 64),
    # code streams that straddle words (3, 5, 6 bits) and 1 bit; the GEMM
    # path runs them on codes transcoded to bytes
    (1, 416, 200, 3, 32), (3, 640, 77, 5, 128), (9, 448, 130, 6, 64), (17, 384, 129, 1, 128),
    (130, 384, 257, 3, 64), (40, 4160, 72, 5, 64), (33, 640, 131, 6, 128), (20, 448, 250, 1, 32),
    # M <= 2 with one, two and four 32-code chunks per lane: the flat kernel's
    # code-stream pairs (j, j+16) at 5, 6 and 1 bits
    (2, 640, 77, 5, 64), (1, 448, 130, 6, 64), (2, 384, 129, 1, 128), (1, 4096, 96, 6, 128),
    (2, 8192, 40, 5, 32), (1, 2048, 33, 3, 64),
    # the flat kernel's lane l takes chunks l + 64 i, each with its own
    # group's scale and bias: group_size 128 (four chunks a group), and K
    # with four chunks per lane and a ragged last one
    (1, 4096, 100, 4, 128), (2, 4224, 70, 4, 128), (1, 4224, 64, 3, 128), (2, 6144, 40, 4, 32),
]


@pytest.mark.parametrize("path", ["skinny", "gemm"])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
def test_forward_paths_ragged(path, xdt, shape):
    M, K, N, bits, G = shape
    if path == "gemm" and xdt == torch.float32:
        pytest.skip("fp32 x always takes the skinny kernel")
    inp = workloads.affine_inputs(M, K, N, x_dtype=ODT[xdt], bias=(M % 2 == 1), seed=M * 1000 + K + N)
    old = qlq.qlq_get_skinny_max_m()
    qlq.qlq_set_skinny_max_m(1 << 20 if path == "skinny" else 0)
    try:
        y, y_ref, D = _forward_case(inp, bits, G, xdt)
    finally:
        qlq.qlq_set_skinny_max_m(old)
    assert_close(y, y_ref, D, K, xdt, label=f"{path} {xdt} {shape}")


# enough output columns that the GEMM takes 256-row blocks for 4-bit codes
# (two blocks per compute unit; 2- and 8-bit codes keep 128-row blocks); M is
# ragged against 256 and N against 128
TALL_SHAPES = [(300, 128, 32808, 4, 32), (520, 256, 32808, 4, 128), (300, 192, 32808, 2, 64),
               (260, 128, 32808, 8, 128), (260, 128, 32808, 3, 32),
               # the tiles past the last paired round are whole tile columns:
               # their k-halves run as separate blocks and a join adds them
               # (ragged M, N ragged inside the tail columns)
               (1900, 512, 8910, 4, 128), (2048, 384, 8865, 4, 32)]


@pytest.mark.parametrize("shape", TALL_SHAPES)
def test_forward_gemm_tall_blocks_ragged(shape):
    M, K, N, bits, G = shape
    inp = workloads.affine_inputs(M, K, N, x_dtype="bf16", bias=True, seed=M + K + N + bits)
    old = qlq.qlq_get_skinny_max_m()
    qlq.qlq_set_skinny_max_m(0)
    try:
        y, y_ref, D = _forward_case(inp, bits, G, torch.bfloat16)
    finally:
        qlq.qlq_set_skinny_max_m(old)
    assert_close(y, y_ref, D, K, torch.bfloat16, label=f"gemm tall {shape}")


# M == 1 with 4-bit codes and at least 12288 rows: two rows per wave in
# blocks of 8 waves (flat kernel at one, two and four chunks per lane; the
# pair kernel at K = 4160; the fp32 generic kernel), N ragged against 16
LARGE_N_SHAPES = [(1, 512, 12301, 4, 32), (1, 2048, 12303, 4, 64), (1, 4096, 12290, 4, 128),
                  (1, 4160, 12289, 4, 64), (1, 8192, 12288, 4, 128)]


@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("shape", LARGE_N_SHAPES)
def test_forward_skinny_large_n(xdt, shape):
    M, K, N, bits, G = shape
    if xdt != torch.bfloat16 and K == 8192:
        pytest.skip("one x dtype at the largest K keeps the oracle's share short")
    inp = workloads.affine_inputs(M, K, N, x_dtype=ODT[xdt], bias=(N % 2 == 1), seed=K + N)
    y, y_ref, D = _forward_case(inp, bits, G, xdt)
    assert_close(y, y_ref, D, K, xdt, label=f"large N {xdt} {shape}")


@pytest.mark.parametrize("xdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("bias", [False, True])
def test_forward_gemm_tail_split_dtypes(xdt, bias):
    """The split tail's join kernel rounds to either 16-bit dtype, with and
    without a layer bias, like the GEMM's own epilogue."""
    M, K, N, bits, G = 1900, 256, 8910, 4, 64
    inp = workloads.affine_inputs(M, K, N, x_dtype=ODT[xdt], bias=bias, seed=N + int(bias))
    old = qlq.qlq_get_skinny_max_m()
    qlq.qlq_set_skinny_max_m(0)
    try:
        y, y_ref, D = _forward_case(inp, bits, G, xdt)
    finally:
        qlq.qlq_set_skinny_max_m(old)
    assert_close(y, y_ref, D, K, xdt, label=f"gemm tail split {xdt} bias={bias}")


def test_forward_flattens_leading_dims():
    inp = workloads.affine_inputs(6, 256, 48, x_dtype="bf16", bias=True, seed=3)
    x = inp["x"].reshape(2, 3, 256).to(dev())
    packed, scales, biases = qlq.qlq_pack(inp["w"].to(dev()), 4, 64, torch.bfloat16)
    y3 = qlq.qlq_linear_forward(x, packed, scales, biases, 4, 64, bias=inp["bias"].to(dev()))
    y2 = qlq.qlq_linear_forward(x.reshape(6, 256), packed, scales, biases, 4, 64, bias=inp["bias"].to(dev()))
    assert y3.shape == (2, 3, 48)
    assert torch.equal(y3.reshape(6, 48), y2)


def test_forward_one_hot_and_zero_input():
    """x = e_k returns the dequantized column (+ bias) and x = 0 returns the
    bias, through both kernels."""
    K, N, G = 256, 40, 64
    w = workloads.affine_inputs(1, K, N, seed=9)["w"].to(dev())
    packed, scales, biases = qlq.qlq_pack(w, 4, G, torch.bfloat16)
    wd = qlq.qlq_dequantize(packed, scales, biases, K, 4, G)
    bias = (torch.arange(N, device=dev(), dtype=torch.float32) / 64).to(torch.bfloat16)
    x = torch.zeros(20, K, device=dev(), dtype=torch.bfloat16)
    for i, k in enumerate(range(0, K, 16)):
        x[i, k] = 1.0
    for thr in (1 << 20, 0):
        qlq.qlq_set_skinny_max_m(thr)
        y = qlq.qlq_linear_forward(x, packed, scales, biases, 4, G, bias=bias)
        ref = (wd[:, 0:K:16].T + bias.float()).to(torch.bfloat16).float()
        # the kernels' factored s*P' + (b - OFF*s)*X may differ from one fused
        # multiply-add by an fp32 ulp, which can move the bf16 rounding by one
        assert torch.allclose(y[:16].float(), ref, rtol=2.0 ** -7, atol=1e-30), thr
        assert torch.equal(y[16:], bias.expand(4, N)), thr
    qlq.qlq_set_skinny_max_m(8)
