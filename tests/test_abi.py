"""C ABI checks that need no GPU: the library loads, exports every function
include/qlq.h declares, and rejects invalid arguments before any HIP call.

Pointers here are fake non-null addresses.  Each invalid call has exactly one
invalid aspect that host validation rejects, so no call reaches the device.
"""

import ctypes
import os
import re

import pytest
import torch

import bit_weight_quantized_qlq_amd as qlq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlq.h")

A = 0x100000    # 16-byte aligned fake device address
B = 0x200000
ODD = 0x100002  # 2-byte aligned only

pytestmark = pytest.mark.skipif(not os.path.exists(qlq.lib_path()), reason="libqlq.so not built")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"QLQ_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_matches_binding_and_exports():
    names = _declared()
    assert len(names) >= 15
    assert set(names) == set(qlq.SIGNATURES), set(names) ^ set(qlq.SIGNATURES)
    handle = ctypes.CDLL(qlq.lib_path())
    for n in names:
        assert hasattr(handle, n), n


def test_version_and_threshold():
    L = qlq.lib()
    assert b"gfx950" in L.qlq_version()
    old = L.qlq_get_skinny_max_m()
    assert L.qlq_set_skinny_max_m(-1) == qlq.QLQ_ERR_INVALID_ARG
    assert L.qlq_set_skinny_max_m(3) == 0 and L.qlq_get_skinny_max_m() == 3
    assert L.qlq_set_skinny_max_m(old) == 0


def _lin(**kw):
    a = dict(x=A, x_dtype=qlq.QLQ_BF16, M=4, K=256, packed=A, scales=A, biases=A,
             sb_dtype=qlq.QLQ_BF16, N=64, bits=4, G=64, bias=None, y=A, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return qlq.lib().qlq_linear_forward(a["x"], a["x_dtype"], a["M"], a["K"], a["packed"], a["scales"],
                                        a["biases"], a["sb_dtype"], a["N"], a["bits"], a["G"], a["bias"],
                                        a["y"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), qlq.QLQ_ERR_INVALID_ARG),
    (dict(y=None), qlq.QLQ_ERR_INVALID_ARG),
    (dict(M=-1), qlq.QLQ_ERR_INVALID_ARG),
    (dict(N=0), qlq.QLQ_ERR_INVALID_ARG),
    (dict(K=250), qlq.QLQ_ERR_INVALID_ARG),          # K % G != 0
    (dict(bits=7), qlq.QLQ_ERR_UNSUPPORTED),     # layer widths are 1-6 and 8
    (dict(bits=0), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(G=48), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(G=256, K=512), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(x_dtype=7, sb_dtype=7), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(sb_dtype=qlq.QLQ_F32), qlq.QLQ_ERR_DTYPE),
    (dict(x=ODD), qlq.QLQ_ERR_ALIGNMENT),
    (dict(packed=ODD), qlq.QLQ_ERR_ALIGNMENT),
    (dict(y=A + 1), qlq.QLQ_ERR_ALIGNMENT),
    (dict(M=4096), qlq.QLQ_ERR_WORKSPACE),            # GEMM path without workspace
    (dict(M=4096, ws=A, ws_bytes=16), qlq.QLQ_ERR_WORKSPACE),
])
def test_linear_forward_validation(kw, code):
    assert _lin(**kw) == code
    assert qlq.last_error() != ""


def test_transcoded_widths_need_room_for_their_codes():
    # 1-, 2- and 3-bit codes are rewritten as nibbles (N*K/2 bytes), 5- and
    # 6-bit codes as bytes (N*K); 4- and 8-bit codes are used as they are
    # (the 4-bit GEMM's workspace also holds its tail tiles' partial sums)
    L = qlq.lib()
    ws = {b: L.qlq_linear_workspace_size(2048, 4096, 11008, b, 128, qlq.QLQ_BF16) for b in (4, 8)}
    assert 0 < ws[8] <= ws[4]
    for bits, run, per in ((1, 4, 0.5), (2, 4, 0.5), (3, 4, 0.5), (5, 8, 1), (6, 8, 1)):
        assert L.qlq_linear_workspace_size(2048, 4096, 11008, bits, 128, qlq.QLQ_BF16) >= ws[run] + 11008 * 4096 * per
    assert L.qlq_linear_workspace_size(4, 4096, 11008, 3, 128, qlq.QLQ_BF16) == 0   # skinny: none


def test_workspace_sizes():
    L = qlq.lib()
    # skinny path needs none; GEMM path needs the group-sum split
    assert L.qlq_linear_workspace_size(1, 4096, 4096, 4, 64, qlq.QLQ_BF16) == 0
    assert L.qlq_linear_workspace_size(2048, 4096, 4096, 4, 64, qlq.QLQ_F32) == 0
    ws = L.qlq_linear_workspace_size(2048, 4096, 11008, 4, 128, qlq.QLQ_BF16)
    assert ws >= 2048 * 6 * 32 * 2 + 2048 * 4
    assert L.w8a8_workspace_size(1024, 4096) >= 1024 * 4096 + 1024 * 4
    assert L.w8a8_workspace_size(0, 4096) == 0


@pytest.mark.parametrize("args,code", [
    ((None, 8, 64, 4, 64, A, A, A, qlq.QLQ_BF16, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, 8, 64, 7, 64, A, A, A, qlq.QLQ_BF16, None), qlq.QLQ_ERR_UNSUPPORTED),
    ((A, 8, 64, 4, 16, A, A, A, qlq.QLQ_BF16, None), qlq.QLQ_ERR_UNSUPPORTED),
    ((A, 8, 96, 4, 64, A, A, A, qlq.QLQ_BF16, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, 8, 64, 4, 64, A, A, A, 9, None), qlq.QLQ_ERR_UNSUPPORTED),
    ((ODD, 8, 64, 4, 64, A, A, A, qlq.QLQ_BF16, None), qlq.QLQ_ERR_ALIGNMENT),
])
def test_pack_validation(args, code):
    assert qlq.lib().qlq_pack(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(N=6), qlq.QLQ_ERR_INVALID_ARG),           # N % 4
    (dict(K=48), qlq.QLQ_ERR_INVALID_ARG),          # K % 32
    (dict(ws=None), qlq.QLQ_ERR_INVALID_ARG),
    (dict(x_dtype=5), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(x=ODD), qlq.QLQ_ERR_ALIGNMENT),
    (dict(y=A + 1), qlq.QLQ_ERR_ALIGNMENT),
    (dict(K=1 << 26), qlq.QLQ_ERR_UNSUPPORTED),          # 16-bit x: K < 2^26
])
def test_bitlinear_validation(kw, code):
    a = dict(x=A, x_dtype=qlq.QLQ_BF16, M=8, K=64, packed=A, N=16, ws=B, inv=0, bias=None, y=A)
    a.update(kw)
    r = qlq.lib().bitlinear_forward(a["x"], a["x_dtype"], a["M"], a["K"], a["packed"], a["N"], a["ws"],
                                    a["inv"], a["bias"], a["y"], None)
    assert r == code


def test_bitlinear_pack_validation():
    assert qlq.lib().bitlinear_pack(A, 6, 8, A, None) == qlq.QLQ_ERR_INVALID_ARG
    assert qlq.lib().bitlinear_pack(None, 8, 8, A, None) == qlq.QLQ_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(K=40), qlq.QLQ_ERR_INVALID_ARG),
    (dict(K=131072), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(x_dtype=qlq.QLQ_F32), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(ws=None), qlq.QLQ_ERR_WORKSPACE),
    (dict(ws_bytes=100), qlq.QLQ_ERR_WORKSPACE),
    (dict(x=ODD), qlq.QLQ_ERR_ALIGNMENT),
    (dict(w=A + 8), qlq.QLQ_ERR_ALIGNMENT),
])
def test_w8a8_validation(kw, code):
    a = dict(x=A, x_dtype=qlq.QLQ_F16, M=16, K=64, w=B, sw=A, N=32, bias=None, y=A, ws=B, ws_bytes=1 << 20)
    a.update(kw)
    r = qlq.lib().w8a8_linear_forward(a["x"], a["x_dtype"], a["M"], a["K"], a["w"], a["sw"], a["N"],
                                      a["bias"], a["y"], a["ws"], a["ws_bytes"], None)
    assert r == code


def test_int8_helpers_validation():
    L = qlq.lib()
    assert L.qlq_int8_matmul_int32(A, B, 4, 4, 40, A, None) == qlq.QLQ_ERR_INVALID_ARG
    assert L.qlq_int8_matmul_int32(A, B, 4, 4, 131088, A, None) == qlq.QLQ_ERR_UNSUPPORTED
    assert L.qlq_int8_matmul_int32(ODD, B, 4, 4, 64, A, None) == qlq.QLQ_ERR_ALIGNMENT
    assert L.qlq_quantize_rows_int8(A, qlq.QLQ_F16, 4, 40, A, A, None) == qlq.QLQ_ERR_INVALID_ARG
    assert L.qlq_quantize_rows_int8(A, 11, 4, 64, A, A, None) == qlq.QLQ_ERR_UNSUPPORTED
    assert L.qlq_unpack(A, 4, 64, 7, A, None) == qlq.QLQ_ERR_UNSUPPORTED
    assert L.qlq_unpack(A, 4, 40, 3, A, None) == qlq.QLQ_ERR_INVALID_ARG    # 120 bits: not whole words
    assert L.qlq_dequantize(A, A, A, qlq.QLQ_BF16, 4, 64, 4, 48, A, None) == qlq.QLQ_ERR_UNSUPPORTED


def test_empty_batch_is_a_no_op():
    # M == 0 returns before any device work, on any machine
    assert _lin(M=0) == 0
    assert qlq.lib().w8a8_linear_forward(A, qlq.QLQ_F16, 0, 64, B, A, 32, None, A, None, 0, None) == 0


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_valid_call_without_device_reports_device_error():
    # fully valid arguments: validation passes, then the device check fails
    assert _lin() == qlq.QLQ_ERR_DEVICE
    assert qlq.lib().qlq_device_check(0) == qlq.QLQ_ERR_DEVICE
    assert "device" in qlq.last_error()


@pytest.mark.parametrize("args,code", [
    ((None, qlq.QLQ_F32, 8, 128, 64, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, qlq.QLQ_F32, 8, 128, 32, A, B, None), qlq.QLQ_ERR_UNSUPPORTED),    # group 32 not built
    ((A, qlq.QLQ_F32, 8, 192, 128, A, B, None), qlq.QLQ_ERR_INVALID_ARG),   # K % G
    ((A, 9, 8, 128, 64, A, B, None), qlq.QLQ_ERR_UNSUPPORTED),
    ((ODD, qlq.QLQ_F32, 8, 128, 64, A, B, None), qlq.QLQ_ERR_ALIGNMENT),
])
def test_quantize_groups_validation(args, code):
    assert qlq.lib().qlq_quantize_groups_int8(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), qlq.QLQ_ERR_INVALID_ARG),
    (dict(G=32), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(K=320, G=128), qlq.QLQ_ERR_INVALID_ARG),          # K % G
    (dict(x_dtype=qlq.QLQ_F32), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(M=1, K=32768), qlq.QLQ_ERR_UNSUPPORTED),           # float-x product stages x on chip
    (dict(ws=None, ws_bytes=0), qlq.QLQ_ERR_WORKSPACE),      # M > 1 quantizes x into the workspace
    (dict(x=ODD), qlq.QLQ_ERR_ALIGNMENT),
])
def test_pergroup_forward_validation(kw, code):
    a = dict(x=A, x_dtype=qlq.QLQ_F16, M=4, K=256, w=A, s=B, N=32, G=64, bias=None, y=A, ws=B, ws_bytes=1 << 20)
    a.update(kw)
    r = qlq.lib().pergroup_linear_forward(a["x"], a["x_dtype"], a["M"], a["K"], a["w"], a["s"], a["N"], a["G"],
                                          a["bias"], a["y"], a["ws"], a["ws_bytes"], None)
    assert r == code


def test_pergroup_workspace_sizes():
    L = qlq.lib()
    assert L.pergroup_workspace_size(1, 4096) == 0
    assert L.pergroup_workspace_size(2, 4096) == L.w8a8_workspace_size(2, 4096) > 0


@pytest.mark.parametrize("args,code", [
    ((None, qlq.QLQ_F32, 64, 32, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, qlq.QLQ_F32, 63, 32, A, B, None), qlq.QLQ_ERR_INVALID_ARG),      # K odd
    ((A, qlq.QLQ_F32, 0, 32, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, 9, 64, 32, A, B, None), qlq.QLQ_ERR_UNSUPPORTED),
    ((ODD, qlq.QLQ_F32, 64, 32, A, B, None), qlq.QLQ_ERR_ALIGNMENT),
    ((A, qlq.QLQ_F32, 64, 32, A, ODD, None), qlq.QLQ_ERR_ALIGNMENT),       # scale
])
def test_w4a8_pack_validation(args, code):
    assert qlq.lib().w4a8_pack_weight_int4(*args) == code


@pytest.mark.parametrize("kw,code", [
    (dict(w=None), qlq.QLQ_ERR_INVALID_ARG),
    (dict(K=40), qlq.QLQ_ERR_INVALID_ARG),                     # K % 16
    (dict(K=131072), qlq.QLQ_ERR_UNSUPPORTED),                 # int32 headroom
    (dict(K=65536, N=65536), qlq.QLQ_ERR_UNSUPPORTED),         # packed bytes >= 2^31
    (dict(x_dtype=qlq.QLQ_F32), qlq.QLQ_ERR_UNSUPPORTED),
    (dict(ws=None), qlq.QLQ_ERR_WORKSPACE),
    (dict(ws_bytes=100), qlq.QLQ_ERR_WORKSPACE),
    (dict(x=ODD), qlq.QLQ_ERR_ALIGNMENT),
    (dict(w=ODD), qlq.QLQ_ERR_ALIGNMENT),                      # packed_w needs 4 bytes
    (dict(ws=A + 8), qlq.QLQ_ERR_ALIGNMENT),
])
def test_w4a8_forward_validation(kw, code):
    a = dict(x=A, x_dtype=qlq.QLQ_F16, M=16, K=64, w=B, sw=A, N=32, bias=None, y=A, ws=B, ws_bytes=1 << 20)
    a.update(kw)
    r = qlq.lib().w4a8_linear_forward(a["x"], a["x_dtype"], a["M"], a["K"], a["w"], a["sw"], a["N"],
                                      a["bias"], a["y"], a["ws"], a["ws_bytes"], None)
    assert r == code


def test_w4a8_workspace_and_empty_batch():
    L = qlq.lib()
    assert L.w4a8_workspace_size(16, 4096, 4096) == L.w8a8_workspace_size(16, 4096) > 0
    assert L.w4a8_workspace_size(0, 4096, 4096) == 0
    # M <= 8: room for the split-K partials (32 splits of 128 input values)
    assert L.w4a8_workspace_size(1, 4096, 4096) >= 32 * 4096 * 4 + 4
    assert L.w4a8_workspace_size(8, 4096, 64) >= L.w8a8_workspace_size(8, 4096)
    assert L.w4a8_linear_forward(A, qlq.QLQ_F16, 0, 64, B, A, 32, None, A, None, 0, None) == 0


@pytest.mark.parametrize("args,code", [
    ((None, qlq.QLQ_F32, 4, 64, 99.9, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, qlq.QLQ_F32, 4, 0, 99.9, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, qlq.QLQ_F32, 4, 16385, 99.9, A, B, None), qlq.QLQ_ERR_UNSUPPORTED),   # rows sorted on chip
    ((A, qlq.QLQ_F32, 4, 64, 100.5, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, qlq.QLQ_F32, 4, 64, -1.0, A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, qlq.QLQ_F32, 4, 64, float("nan"), A, B, None), qlq.QLQ_ERR_INVALID_ARG),
    ((A, 9, 4, 64, 99.9, A, B, None), qlq.QLQ_ERR_UNSUPPORTED),
    ((ODD, qlq.QLQ_F32, 4, 64, 99.9, A, B, None), qlq.QLQ_ERR_ALIGNMENT),
])
def test_clip_quantizer_validation(args, code):
    assert qlq.lib().qlq_quantize_rows_int8_clip(*args) == code


def test_empty_batch_accepts_null_row_tensors():
    L = qlq.lib()
    assert L.qlq_linear_forward(None, qlq.QLQ_BF16, 0, 256, A, A, A, qlq.QLQ_BF16, 64, 4, 64, None, None,
                                None, 0, None) == 0
    assert L.bitlinear_forward(None, qlq.QLQ_BF16, 0, 256, A, 64, A, 0, None, None, None) == 0
    assert L.w8a8_linear_forward(None, qlq.QLQ_F16, 0, 64, B, A, 32, None, None, None, 0, None) == 0
    assert L.pergroup_linear_forward(None, qlq.QLQ_F16, 0, 256, A, B, 32, 64, None, None, None, 0, None) == 0
    assert L.w4a8_linear_forward(None, qlq.QLQ_F16, 0, 64, B, A, 32, None, None, None, 0, None) == 0
    assert L.qlq_quantize_rows_int8(None, qlq.QLQ_F16, 0, 64, None, None, None) == 0
    # a non-empty batch still needs them
    assert L.w8a8_linear_forward(None, qlq.QLQ_F16, 4, 64, B, A, 32, None, A, B, 1 << 20, None) == \
        qlq.QLQ_ERR_INVALID_ARG


def test_gemm_bound_follows_the_tallest_tile():
    # 2048 x 16256 outputs give 8 x 127 = 1016 tiles of 256 x 128, enough for
    # the launcher to pick 256-row tiles; with K = 2^22 + 128 a 256-row tile
    # of fp16 x spans 512 K > 2^31 bytes, beyond the GEMM's 32-bit buffer
    # offsets, so the call takes the skinny kernel (no workspace)
    L = qlq.lib()
    M, N, G = 2048, 16256, 128
    K_big = (1 << 22) + 128
    assert 4 * (K_big // G) * N < 2 ** 31          # the (s', b') table alone would fit
    assert L.qlq_linear_workspace_size(M, K_big, N, 4, G, qlq.QLQ_BF16) == 0
    K_ok = (1 << 22) - 128
    assert L.qlq_linear_workspace_size(M, K_ok, N, 4, G, qlq.QLQ_BF16) > 0


def test_noalloc_w8a8_validation():
    L = qlq.lib()
    text = open(HEADER).read()
    assert "#define QLQ_W8A8_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text
    assert qlq.W8A8_NOALLOC_SCRATCH_BYTES == 16 << 20
    f = L.w8a8_linear_forward_noalloc
    ok = dict(x=A, x_dtype=qlq.QLQ_F16, M=16, K=64, w=B, sw=A, N=32, bias=None, y=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["x"], a["x_dtype"], a["M"], a["K"], a["w"], a["sw"], a["N"], a["bias"], a["y"], None)

    assert call(x=None) == qlq.QLQ_ERR_INVALID_ARG
    assert call(K=40) == qlq.QLQ_ERR_INVALID_ARG
    assert call(x_dtype=qlq.QLQ_F32) == qlq.QLQ_ERR_UNSUPPORTED
    assert call(x=ODD) == qlq.QLQ_ERR_ALIGNMENT
    assert call(M=0) == 0 and call(M=0, x=None, y=None) == 0
    # beyond the static scratch: rejected before any HIP call, on any machine
    assert L.w8a8_workspace_size(4093, 4096) > qlq.W8A8_NOALLOC_SCRATCH_BYTES
    assert call(M=4093, K=4096) == qlq.QLQ_ERR_WORKSPACE
    assert "scratch" in qlq.last_error()


def test_fused_quant_switch():
    L = qlq.lib()
    old = L.qlq_get_w8a8_fused_quant()
    assert old == 0                                       # the default: quantizer before the GEMM
    assert L.qlq_set_w8a8_fused_quant(2) == qlq.QLQ_ERR_INVALID_ARG
    assert L.qlq_set_w8a8_fused_quant(1) == 0 and L.qlq_get_w8a8_fused_quant() == 1
    assert L.qlq_set_w8a8_fused_quant(0) == 0 and L.qlq_get_w8a8_fused_quant() == 0


def test_gemm_workspace_holds_tail_partials():
    """The tall 4-bit GEMM splits the tiles past its last whole paired round
    over two k-halves when they are whole tile columns and their halves fit
    one per CU; the workspace then holds the halves' fp32 partial sums."""
    L = qlq.lib()
    bf = qlq.QLQ_BF16
    base = lambda M, K, N, G: M * K * 2 + M * 4 + N * 4 + (K // G) * ((N + 3) // 4 * 4) * 4
    # 2048 x 9216: 576 tiles = 512 + 8 rows x 8 columns of tail tiles
    M, K, N, G = 2048, 4096, 9216, 128
    size = L.qlq_linear_workspace_size(M, K, N, 4, G, bf)
    assert size >= base(M, K, N, G) + 2 * M * (N - 64 * 128) * 4
    # 3-bit codes run as 4-bit ones: split, plus the transcoded codes
    size = L.qlq_linear_workspace_size(M, K, N, 3, G, bf)
    assert size >= base(M, K, N, G) + 2 * M * (N - 64 * 128) * 4 + N * K // 2
    # 8-bit codes keep 128-row tiles and never split
    size = L.qlq_linear_workspace_size(M, K, N, 8, G, bf)
    assert size < base(M, K, N, G) + 4096
    # exactly one paired round, or 176 tail tiles (their 352 halves would
    # share CUs): no split
    for n in (8192, 11008):
        size = L.qlq_linear_workspace_size(M, K, n, 4, G, bf)
        assert base(M, K, n, G) <= size < base(M, K, n, G) + 4096
